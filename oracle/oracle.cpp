// TEST INFRASTRUCTURE ONLY - the CPU oracle of the verification path.
//
// A plain, slow, fp64 implementation of what the path computes, written from the pages:
//   * "Accelerating LLM Decoding with Speculative Sampling" (DeepMind, 2302.01318) knowledge-base
//     page: sections 1, 3 and 6 (the modified rejection sampling, top-k / nucleus / temperature
//     applied to draft and target before the correction, bonus token on full acceptance);
//   * "Speculative Speculative Decoding" reading notes: sections 2.2 (one-line SD recap), 4.3
//     (Theorem 12, geometric fan-out), 4.4 (Theorem 15 / Theorem 19, Saguaro sampling), 5.1
//     (cache construction), 7.1 (Corollary 16, whole-batch miss);
//   * hyper.ai SSD/Saguaro summary, "Method" (the fan-out closed form and sigma_{F,C});
//   * Mirror-SD reading notes, sections 2 and 3.2 (greedy verify, verification-vs-reuse rule);
//   * SSD reading notes section 7.1 and the hyper.ai summary's fallback paragraph (the
//     batch-aware switch to a random-token backup speculator on a cache miss);
//   * Mirror-SD reading notes sections 3.1-3.3 (the early-exit signposts: top-kappa tokens of
//     the layer-l_e distribution with their log-probabilities; reuse of a committed prefix
//     against a draft tree that branches below its roots, as in the worked example);
//   * PyramidSD notes, "key designs" 1 and 2 (fuzzy acceptance: a drafted token passes when the
//     divergence between the verifier's and the drafter's distributions is at most a threshold;
//     the assisted variant draws the correction from the verifier's own distribution).
//
// Notation follows the DeepMind page: p = draft distribution, q = target distribution.
// Only tests/, the smoke check and the bench's CPU-baseline leg may load this library; the
// product path never does.  It shares no code with the HIP path.
//
// Every selection sorts with std::stable_sort on (logit descending, token id ascending);
// every sum is a sequential fp64 loop; the random stream is its own Philox4x64-10.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

namespace {

// ----------------------------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw: "Parallel Random Numbers: As Easy as 1, 2, 3",
// SC'11): 10 rounds of two 64x64->128 multiplies; the key is bumped by the Weyl constants
// between rounds.
// ----------------------------------------------------------------------------------------------
const uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ULL;
const uint64_t kPhiloxM1 = 0xCA5A826395121157ULL;
const uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ULL;
const uint64_t kPhiloxW1 = 0xBB67AE8584CAA73BULL;

void philox(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4]) {
    uint64_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint64_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += kPhiloxW0;
            k1 += kPhiloxW1;
        }
        unsigned __int128 a = (unsigned __int128)kPhiloxM0 * x0;
        unsigned __int128 b = (unsigned __int128)kPhiloxM1 * x2;
        uint64_t hi0 = (uint64_t)(a >> 64), lo0 = (uint64_t)a;
        uint64_t hi1 = (uint64_t)(b >> 64), lo1 = (uint64_t)b;
        x0 = hi1 ^ x1 ^ k0;
        x1 = lo1;
        x2 = hi0 ^ x3 ^ k1;
        x3 = lo0;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

// A uniform in (0, 1): the top 52 bits of a Philox word plus one half ulp, exact in fp64.
double to_uniform(uint64_t x) { return ((double)(x >> 12) + 0.5) * 0x1.0p-52; }

// Lanes of the block for (seed; round, request b, position j): 0 = acceptance u_j,
// 1 = residual / bonus v_j, 2 = draft-token sampling.
void uniforms(uint64_t seed, uint64_t round, uint64_t b, uint64_t j, double out[3]) {
    uint64_t ctr[4] = {round, b, j, 0};
    uint64_t key[2] = {seed, 0};
    uint64_t w[4];
    philox(ctr, key, w);
    out[0] = to_uniform(w[0]);
    out[1] = to_uniform(w[1]);
    out[2] = to_uniform(w[2]);
}

// ----------------------------------------------------------------------------------------------
// Inputs
// ----------------------------------------------------------------------------------------------
enum { kFP32 = 0, kBF16 = 1 };

double load_logit(const void* base, int dtype, size_t idx) {
    if (dtype == kBF16) {
        uint16_t h = static_cast<const uint16_t*>(base)[idx];
        uint32_t u = (uint32_t)h << 16;
        float f;
        std::memcpy(&f, &u, 4);
        return (double)f;
    }
    return (double)static_cast<const float*>(base)[idx];
}

void load_row(const void* base, int dtype, size_t row, int V, std::vector<double>& z) {
    z.resize(V);
    for (int i = 0; i < V; ++i) z[i] = load_logit(base, dtype, row * (size_t)V + i);
}

struct Params {
    float temperature;  // 0 => greedy
    int32_t top_k;      // <= 0 or >= V => off
    float top_p;        // >= 1 => off
};

// status bits shared with the public header (values fixed by the C ABI)
enum : uint32_t {
    ST_EMPTY_RESIDUAL = 8,
    ST_OUTSIDE_DRAFT_SUPPORT = 16,
    ST_BAD_LOGIT = 32,
    ST_BAD_TOKEN = 64,
    ST_DEGENERATE_DOWNWEIGHT = 128,
    ST_BAD_PARAM = 256,
};
// oracle-only near-boundary flags (parity excludes flagged requests and counts them)
enum : uint32_t { FL_NEAR_ACCEPT = 1, FL_NEAR_CDF = 2, FL_NEAR_NUCLEUS = 4, FL_NEAR_FUZZY = 8 };

// A divergence within this absolute distance of the fuzzy threshold flags the request (the
// divergence is an fp64 sum over the vocabulary; its rounding is ~1e-15).
const double kNearFuzzy = 1e-9;

// Near-tie bands.  A uniform within 1e-6 relative of an acceptance boundary flags the
// request.  The inverse CDF and the nucleus cut compare fp64 running sums of masses (on the
// GPU per-value sums of exact counts or fp64 sums in another order, rounding ~1e-13), so their
// bands are 1e-9 of the total mass.
const double kNearRel = 1e-6;
const double kNearCdf = 1e-9;
const double kNearNucleus = 1e-9;

// Token order used by every selection: logit descending, token id ascending on equal logits
// (IEEE equality, so -0 and +0 tie).
std::vector<int> desc_order(const std::vector<double>& z) {
    std::vector<int> ord(z.size());
    for (size_t i = 0; i < z.size(); ++i) ord[i] = (int)i;
    std::stable_sort(ord.begin(), ord.end(), [&](int a, int b) { return z[a] > z[b]; });
    return ord;
}

bool row_is_bad(const std::vector<double>& z) {
    bool any_finite = false;
    for (double v : z) {
        if (std::isnan(v) || v == std::numeric_limits<double>::infinity()) return true;
        if (std::isfinite(v)) any_finite = true;
    }
    return !any_finite;
}

// One processed distribution: temperature, then top-k, then softmax, then nucleus.
struct Proc {
    bool bad = false;
    bool greedy = false;
    int argmax = -1;
    bool near_cut = false;
    int n_kept = 0;              // tokens surviving top-k and nucleus
    std::vector<int> order;      // full (logit desc, id asc) order
    std::vector<double> p;       // processed probabilities (fp64)
};

Proc process(const std::vector<double>& z, const Params& prm) {
    Proc r;
    const int V = (int)z.size();
    if (row_is_bad(z)) {
        r.bad = true;
        return r;
    }
    r.order = desc_order(z);
    r.argmax = r.order[0];
    r.p.assign(V, 0.0);
    if (prm.temperature == 0.0f) {  // greedy: the distribution is the one-hot argmax
        r.greedy = true;
        r.p[r.argmax] = 1.0;
        r.n_kept = 1;
        return r;
    }
    const double T = (double)prm.temperature;
    int n_kept = V;
    if (prm.top_k > 0 && prm.top_k < V) n_kept = prm.top_k;
    const double m = z[r.order[0]];
    std::vector<double> e(V, 0.0);
    for (int t = 0; t < n_kept; ++t) {
        int i = r.order[t];
        e[i] = std::exp((z[i] - m) / T);
    }
    double S = 0.0;
    for (int i = 0; i < V; ++i) S += e[i];
    if ((double)prm.top_p < 1.0) {
        const double target = (double)prm.top_p * S;
        double cum = 0.0, prev = 0.0;
        int cut = n_kept;
        for (int t = 0; t < n_kept; ++t) {
            prev = cum;
            cum += e[r.order[t]];
            if (cum >= target) {
                cut = t + 1;
                break;
            }
        }
        if (cum - target <= kNearNucleus * S || target - prev <= kNearNucleus * S) r.near_cut = true;
        for (int t = cut; t < n_kept; ++t) e[r.order[t]] = 0.0;
        n_kept = cut;
    }
    double Sn = 0.0;
    for (int i = 0; i < V; ++i) Sn += e[i];
    for (int i = 0; i < V; ++i) r.p[i] = e[i] / Sn;
    r.n_kept = n_kept;
    return r;
}

// Saguaro sampling sigma_{F,C}: the first F tokens of the processed order that carry mass are
// scaled by C, then everything is renormalised.  Returns Z (the normaliser); ids gets the
// chosen tokens in rank order (padded with -1).  Z <= 0 (C = 0 with all mass on the set)
// leaves p unchanged and reports degenerate.
double downweight(Proc& pr, int F, double C, int32_t* ids, bool* degenerate) {
    *degenerate = false;
    for (int f = 0; f < F; ++f) ids[f] = -1;
    if (pr.greedy || F <= 0 || C >= 1.0) {
        int n = 0;
        if (!pr.greedy && F > 0) {
            for (int t = 0; t < (int)pr.order.size() && n < F; ++t)
                if (pr.p[pr.order[t]] > 0.0) ids[n++] = pr.order[t];
        }
        return 1.0;
    }
    const int V = (int)pr.p.size();
    std::vector<double> factor(V, 1.0);
    int n = 0;
    for (int t = 0; t < V && n < F; ++t) {
        int i = pr.order[t];
        if (pr.p[i] > 0.0) {
            ids[n++] = i;
            factor[i] = C;
        }
    }
    double Z = 0.0;
    for (int i = 0; i < V; ++i) Z += pr.p[i] * factor[i];
    if (!(Z > 0.0)) {  // the row is left as it was; its normaliser is 1
        *degenerate = true;
        return 1.0;
    }
    for (int i = 0; i < V; ++i) pr.p[i] = pr.p[i] * factor[i] / Z;
    return Z;
}

// Inverse CDF in token-id order: the first i whose running sum exceeds x * total.
int inverse_cdf(const std::vector<double>& w, double x, bool* near) {
    double total = 0.0;
    for (double v : w) total += v;
    const double target = x * total;
    double cum = 0.0;
    int last = -1;
    for (int i = 0; i < (int)w.size(); ++i) {
        if (!(w[i] > 0.0)) continue;
        double prev = cum;
        cum += w[i];
        last = i;
        if (cum > target) {
            if (target - prev <= kNearCdf * total || cum - target <= kNearCdf * total) *near = true;
            return i;
        }
    }
    *near = true;  // rounding left x * total at or above the running total
    return last;
}

// A token drawn from the uniform distribution on [0, V) by inverse CDF: the least i with
// (i + 1) / V > u, i.e. floor(u V).  u = (2a + 1) / 2^53 exactly (to_uniform), so the product
// is taken in 128-bit integers and the floor is exact.
int32_t uniform_token(double u, int V) {
    const uint64_t m = (uint64_t)(u * 0x1.0p53);  // 2a + 1, exact
    const unsigned __int128 prod = (unsigned __int128)m * (uint64_t)V;
    return (int32_t)(prod >> 53);
}

// Jensen-Shannon divergence in bits between two distributions over the same tokens:
// D = 1/2 sum p log2(p / m) + 1/2 sum q log2(q / m), m = (p + q) / 2 (0 log 0 = 0), in [0, 1].
double jsd_bits(const std::vector<double>& p, const std::vector<double>& q) {
    double d = 0.0;
    for (size_t i = 0; i < p.size(); ++i) {
        const double m = 0.5 * (p[i] + q[i]);
        if (p[i] > 0.0) d += 0.5 * p[i] * std::log2(p[i] / m);
        if (q[i] > 0.0) d += 0.5 * q[i] * std::log2(q[i] / m);
    }
    return d;
}

// Fuzzy acceptance (PyramidSD; a reading, the page leaves Div open): Div is the Jensen-Shannon
// divergence in bits of the processed distributions q_j (verifier) and p'_j (drafter).  Where
// Div <= tau the drafted token passes outright; elsewhere the lossless test and correction
// apply, so tau < 0 (or any tau below every divergence) is the lossless rule.  With
// `assisted`, a rejected position draws its correction from q_j itself.
struct Fuzzy {
    bool on = false;
    double tau = -1.0;
    bool assisted = false;
    double* div = nullptr;  // [K] divergences, nullable
};

struct Request {
    int32_t k = 0;
    int32_t t = -1;
    double W = 0.0;
    uint32_t status = 0;
    uint32_t flags = 0;
};

// The verification of one request, for given uniforms U[j][lane] (j = 0..K).
// uniform_draft: the draft distribution of every position is the uniform one on [0, V) (the
// random-token backup speculator): no draft rows are read, the request's temperature, top-k,
// top-p and sigma_{F,C} do not apply to it, and sampled draft tokens are uniform draws.
Request verify_one(const void* draft, int draft_rows, const void* target, int dtype, int b, int K, int V,
                   const Params& prm, int F, double C, int32_t* tokens, bool sample_draft,
                   const double* U, bool uniform_draft, const Fuzzy& fz = Fuzzy()) {
    Request out;
    if (!(prm.temperature >= 0.0f) || std::isinf(prm.temperature) || !(prm.top_p > 0.0f)) {
        out.status |= ST_BAD_PARAM;
        out.k = 0;
        out.t = -1;
        return out;
    }
    std::vector<double> z;
    std::vector<Proc> q(K + 1), p(K);
    bool bad = false;
    for (int j = 0; j <= K; ++j) {
        load_row(target, dtype, (size_t)b * (K + 1) + j, V, z);
        q[j] = process(z, prm);
        bad |= q[j].bad;
    }
    const double p_uniform = 1.0 / (double)V;
    for (int j = 0; j < K; ++j) {
        if (uniform_draft) {
            p[j].p.assign(V, p_uniform);
            continue;
        }
        load_row(draft, dtype, (size_t)b * draft_rows + j, V, z);
        p[j] = process(z, prm);
        bad |= p[j].bad;
    }
    if (bad) {
        out.status |= ST_BAD_LOGIT;
        out.k = 0;
        out.t = -1;
        return out;
    }
    const bool greedy = prm.temperature == 0.0f;
    std::vector<int32_t> ids(F > 0 ? F : 1);
    for (int j = 0; j < K; ++j) {
        if (q[j].near_cut) out.flags |= FL_NEAR_NUCLEUS;
        if (uniform_draft) continue;
        bool degen = false;
        downweight(p[j], F, C, ids.data(), &degen);
        if (degen) out.status |= ST_DEGENERATE_DOWNWEIGHT;
        if (p[j].near_cut) out.flags |= FL_NEAR_NUCLEUS;
    }
    if (q[K].near_cut) out.flags |= FL_NEAR_NUCLEUS;
    if (sample_draft) {
        for (int j = 0; j < K; ++j) {
            bool near = false;
            if (uniform_draft) tokens[j] = uniform_token(U[3 * j + 2], V);
            else tokens[j] = greedy ? p[j].argmax : inverse_cdf(p[j].p, U[3 * j + 2], &near);
            if (near) out.flags |= FL_NEAR_CDF;
        }
    }
    for (int j = 0; j < K; ++j) {
        if (tokens[j] < 0 || tokens[j] >= V) {
            out.status |= ST_BAD_TOKEN;
            out.k = 0;
            out.t = -1;
            return out;
        }
    }
    if (fz.on && fz.div)
        for (int j = 0; j < K; ++j) fz.div[j] = jsd_bits(q[j].p, p[j].p);
    // Acceptance scan: s_j is kept with probability min(1, q(s_j) / p(s_j)); the first
    // rejection ends the scan.
    int k = K;
    for (int j = 0; j < K; ++j) {
        const int s = tokens[j];
        bool accept;
        if (fz.on) {
            const double D = fz.div ? fz.div[j] : jsd_bits(q[j].p, p[j].p);
            if (std::fabs(D - fz.tau) <= kNearFuzzy) out.flags |= FL_NEAR_FUZZY;
            if (D <= fz.tau) continue;  // fuzzy pass
        }
        if (greedy) {
            accept = (s == q[j].argmax);
        } else {
            const double pj = p[j].p[s], qj = q[j].p[s];
            if (!(pj > 0.0)) out.status |= ST_OUTSIDE_DRAFT_SUPPORT;
            const double lhs = U[3 * j + 0] * pj;
            accept = lhs < qj;
            const double mx = std::max(lhs, qj);
            if (mx > 0.0 && std::fabs(lhs - qj) <= kNearRel * mx) out.flags |= FL_NEAR_ACCEPT;
        }
        if (!accept) {
            k = j;
            break;
        }
    }
    out.k = k;
    if (greedy) {
        out.t = q[k].argmax;
        out.W = 0.0;
        return out;
    }
    bool near = false;
    if (k < K && fz.on && fz.assisted) {
        // assisted correction: from the verifier's distribution at the rejected position
        double W = 0.0;
        for (int i = 0; i < V; ++i) W += q[k].p[i] > p[k].p[i] ? q[k].p[i] - p[k].p[i] : 0.0;
        out.W = W;
        out.t = inverse_cdf(q[k].p, U[3 * k + 1], &near);
    } else if (k < K) {
        // correction token: the normalised residual (q - p)+ at the rejected position
        std::vector<double> w(V);
        double W = 0.0;
        for (int i = 0; i < V; ++i) {
            double d = q[k].p[i] - p[k].p[i];
            w[i] = d > 0.0 ? d : 0.0;
            W += w[i];
        }
        out.W = W;
        if (W > 0.0) {
            out.t = inverse_cdf(w, U[3 * k + 1], &near);
        } else {
            out.status |= ST_EMPTY_RESIDUAL;
            out.t = inverse_cdf(q[k].p, U[3 * k + 1], &near);
        }
    } else {
        // every draft token accepted: the bonus token comes from the target's extra position
        out.W = 0.0;
        out.t = inverse_cdf(q[K].p, U[3 * K + 1], &near);
    }
    if (near) out.flags |= FL_NEAR_CDF;
    return out;
}

template <typename Fn>
void parallel_for(int n, int nthreads, Fn fn) {
    if (nthreads <= 0) nthreads = (int)std::max(1u, std::thread::hardware_concurrency());
    nthreads = std::min(nthreads, std::max(1, n));
    if (nthreads == 1) {
        for (int i = 0; i < n; ++i) fn(i);
        return;
    }
    std::vector<std::thread> th;
    for (int t = 0; t < nthreads; ++t)
        th.emplace_back([&, t] {
            for (int i = t; i < n; i += nthreads) fn(i);
        });
    for (auto& x : th) x.join();
}

bool param_ok(const Params& prm) {
    return prm.temperature >= 0.0f && !std::isinf(prm.temperature) && prm.top_p > 0.0f;
}

}  // namespace

extern "C" {

int orc_threads_used(int nthreads) {
    if (nthreads <= 0) nthreads = (int)std::max(1u, std::thread::hardware_concurrency());
    return nthreads;
}

void orc_philox4x64_10(const uint64_t* ctr, const uint64_t* key, uint64_t* out) { philox(ctr, key, out); }

// U[B][K+1][3]: the uniforms the verification consumes for (seed, round).
void orc_uniforms(uint64_t seed, uint64_t round, int B, int K, double* U) {
    for (int b = 0; b < B; ++b)
        for (int j = 0; j <= K; ++j) uniforms(seed, round, (uint64_t)b, (uint64_t)j, U + ((size_t)b * (K + 1) + j) * 3);
}

// Processes one fp64 row; p_out[V] gets the processed distribution. Returns 1 if the row is
// bad (NaN/+inf/no finite logit), else 0. *near_cut reports a nucleus near-tie.
int orc_process_row_f64(const double* z, int V, float temperature, int32_t top_k, float top_p, double* p_out,
                        int* near_cut, int* n_kept) {
    std::vector<double> zz(z, z + V);
    Params prm{temperature, top_k, top_p};
    Proc r = process(zz, prm);
    if (near_cut) *near_cut = r.near_cut ? 1 : 0;
    if (n_kept) *n_kept = r.n_kept;
    if (r.bad) return 1;
    std::memcpy(p_out, r.p.data(), sizeof(double) * V);
    return 0;
}

// sigma_{F,C} applied to one fp64 probability row given its logits (for the order).
// Returns Z; p (in/out) is replaced by the downweighted distribution; ids[F] the set.
double orc_downweight_probs_f64(const double* z, double* p, int V, int F, double C, int32_t* ids, int* degenerate) {
    Proc pr;
    pr.order = desc_order(std::vector<double>(z, z + V));
    pr.p.assign(p, p + V);
    bool deg = false;
    double Z = downweight(pr, F, C, ids, &deg);
    if (degenerate) *degenerate = deg ? 1 : 0;
    std::memcpy(p, pr.p.data(), sizeof(double) * V);
    return Z;
}

// Processed + downweighted draft rows j < K: ids[B][K][F], Z[B][K], probs[B][K][V] (nullable).
int orc_downweight(const void* draft, int draft_rows, int dtype, int B, int K, int V, const void* params, int F,
                   double C, int32_t* out_ids, double* out_Z, double* out_probs, uint32_t* out_status,
                   int nthreads) {
    const Params* prm = static_cast<const Params*>(params);
    if (!draft || B < 1 || K < 1 || V < 1 || draft_rows < K || F < 0 || !(C >= 0.0 && C <= 1.0)) return -1;
    parallel_for(B * K, nthreads, [&](int bj) {
        int b = bj / K, j = bj % K;
        std::vector<double> z;
        load_row(draft, dtype, (size_t)b * draft_rows + j, V, z);
        const bool pok = param_ok(prm[b]);
        Proc pr;
        if (pok) pr = process(z, prm[b]);
        std::vector<int32_t> ids(F > 0 ? F : 1, -1);
        uint32_t st = 0;
        double Z = 1.0;
        if (!pok) {
            st |= ST_BAD_PARAM;
            pr.bad = true;
        } else if (pr.bad) {
            st |= ST_BAD_LOGIT;
        } else {
            bool deg = false;
            Z = downweight(pr, F, C, ids.data(), &deg);
            if (deg) st |= ST_DEGENERATE_DOWNWEIGHT;
        }
        for (int f = 0; f < F; ++f) out_ids[(size_t)bj * F + f] = ids[f];
        if (out_Z) out_Z[bj] = Z;
        if (out_status) out_status[bj] = st;
        if (out_probs) {
            for (int i = 0; i < V; ++i) out_probs[(size_t)bj * V + i] = pr.bad ? 0.0 : pr.p[i];
        }
    });
    return 0;
}

// Verification with explicit uniforms U[B][K+1][3].  tokens[B][K] is read, or written when
// sample_draft != 0.  Outputs k, t*, residual mass W, status bits and oracle near-tie flags.
// tau (nullable) [B]: fuzzy thresholds (PyramidSD); assisted: corrections from q; out_div
// (nullable) [B][K]: the divergences.
int orc_verify_u(const void* draft, int draft_rows, const void* target, int dtype, int B, int K, int V,
                 const void* params, int F, double C, int32_t* tokens, int sample_draft, const double* U,
                 int32_t* out_k, int32_t* out_t, double* out_W, uint32_t* out_status, uint32_t* out_flags,
                 int nthreads, int uniform_draft, const double* tau, int assisted, double* out_div) {
    const Params* prm = static_cast<const Params*>(params);
    if ((!draft && !uniform_draft) || !target || !tokens || !U || B < 1 || K < 1 || V < 1 ||
        (!uniform_draft && draft_rows < K) || F < 0 || !(C >= 0.0 && C <= 1.0) || (dtype != kFP32 && dtype != kBF16))
        return -1;
    parallel_for(B, nthreads, [&](int b) {
        Fuzzy fz;
        if (tau) {
            fz.on = true;
            fz.tau = tau[b];
            fz.assisted = assisted != 0;
            fz.div = out_div ? out_div + (size_t)b * K : nullptr;
        }
        Request r = verify_one(draft, draft_rows, target, dtype, b, K, V, prm[b], F, C, tokens + (size_t)b * K,
                               sample_draft != 0, U + (size_t)b * (K + 1) * 3, uniform_draft != 0, fz);
        out_k[b] = r.k;
        out_t[b] = r.t;
        if (out_W) out_W[b] = r.W;
        if (out_status) out_status[b] = r.status;
        if (out_flags) out_flags[b] = r.flags;
    });
    return 0;
}

// Verification driven by the Philox stream (seed, round).
int orc_verify(const void* draft, int draft_rows, const void* target, int dtype, int B, int K, int V,
               const void* params, int F, double C, int32_t* tokens, int sample_draft, uint64_t seed, uint64_t round,
               int32_t* out_k, int32_t* out_t, double* out_W, uint32_t* out_status, uint32_t* out_flags,
               int nthreads, int uniform_draft, const double* tau, int assisted, double* out_div) {
    if (B < 1 || K < 1) return -1;
    std::vector<double> U((size_t)B * (K + 1) * 3);
    orc_uniforms(seed, round, B, K, U.data());
    return orc_verify_u(draft, draft_rows, target, dtype, B, K, V, params, F, C, tokens, sample_draft, U.data(),
                        out_k, out_t, out_W, out_status, out_flags, nthreads, uniform_draft, tau, assisted, out_div);
}

// Uniform draws of the backup speculator (for tests): tokens[n] = floor(u[n] V).
// Jensen-Shannon divergence in bits of two distributions of length V (for tests).
double orc_jsd_bits(const double* p, const double* q, int V) {
    return jsd_bits(std::vector<double>(p, p + V), std::vector<double>(q, q + V));
}

void orc_uniform_tokens(const double* u, int n, int V, int32_t* out) {
    for (int i = 0; i < n; ++i) out[i] = uniform_token(u[i], V);
}

// The batch-aware fallback (SSD reading notes 7.1: on any miss the whole batch waits for the
// fallback, and the switch between the primary drafter and the fast random-token backup is
// made by batch size against a critical b*, whose formula the text does not give).  The
// backup serves this round when some request missed (all-hit = 0) and B >= b_star; then every
// missed request takes random tokens and requests that hit keep their cached speculation.
void orc_backup_plan(int B, const uint8_t* hit, int all_hit, int b_star, int32_t* out_use_backup, int32_t* out_switch) {
    const int sw = (all_hit == 0 && B >= b_star) ? 1 : 0;
    for (int b = 0; b < B; ++b) out_use_backup[b] = (sw && !hit[b]) ? 1 : 0;
    *out_switch = sw;
}

// Mirror-SD signposts (reading notes 3.1, 3.3): the LM head at the early-exit layer gives a
// distribution p~ over the vocabulary; the message to the draft is its kappa most likely tokens
// with their log-probabilities.  Read here as the softmax of the given logits at temperature 1,
// tokens in the common order (logit descending, id ascending), log p~(v) = z_v - m - log S with
// m the row maximum and S = sum_i exp(z_i - m).  Entries past the vocabulary are id -1 with
// log-probability -inf; a row with a NaN or +inf logit, or no finite one, gets status
// ST_BAD_LOGIT, ids -1 and NaN log-probabilities.
int orc_signposts(const void* logits, int dtype, int B, int V, int kappa, int32_t* out_ids, double* out_logp,
                  uint32_t* out_status, int nthreads) {
    if (!logits || !out_ids || !out_logp || B < 1 || V < 1 || kappa < 1 || (dtype != kFP32 && dtype != kBF16))
        return -1;
    parallel_for(B, nthreads, [&](int b) {
        std::vector<double> z;
        load_row(logits, dtype, (size_t)b, V, z);
        int32_t* ids = out_ids + (size_t)b * kappa;
        double* lp = out_logp + (size_t)b * kappa;
        if (row_is_bad(z)) {
            for (int i = 0; i < kappa; ++i) {
                ids[i] = -1;
                lp[i] = std::numeric_limits<double>::quiet_NaN();
            }
            if (out_status) out_status[b] = ST_BAD_LOGIT;
            return;
        }
        const std::vector<int> ord = desc_order(z);
        const double m = z[ord[0]];
        double S = 0.0;
        for (int i = 0; i < V; ++i) S += std::exp(z[i] - m);
        const double logS = std::log(S);
        for (int i = 0; i < kappa; ++i) {
            if (i < V) {
                ids[i] = ord[i];
                lp[i] = z[ord[i]] - m - logS;
            } else {
                ids[i] = -1;
                lp[i] = -std::numeric_limits<double>::infinity();
            }
        }
        if (out_status) out_status[b] = 0;
    });
    return 0;
}

// Mirror-SD reuse against a draft tree (reading notes 3.2-3.3).  Each request's tree is N nodes
// (token, parent) with parents listed before their children; parent -1 marks a root (a signpost
// the draft expanded).  The verified path holds gamma draft tokens; with k accepted and
// correction t*, the committed prefix is (path[0..k-1], t*).  The reuse node is the lowest
// node whose chain of ancestors, read from its root down, is exactly that prefix (so it sits at
// depth k + 1); -1 when none, -2 when all gamma tokens were accepted.  A node with a negative
// token or a parent outside [-1, n) is not part of the tree, nor is anything below it.
int orc_tree_lookup(const int32_t* tokens, const int32_t* parents, int B, int N, int gamma, const int32_t* path,
                    const int32_t* kk, const int32_t* tt, int32_t* out_node, uint8_t* out_hit, int32_t* out_batch) {
    if (!tokens || !parents || !path || !kk || !tt || !out_node || !out_hit || B < 1 || N < 1 || gamma < 1)
        return -1;
    int hits = 0;
    for (int b = 0; b < B; ++b) {
        const int32_t* tok = tokens + (size_t)b * N;
        const int32_t* par = parents + (size_t)b * N;
        const int k = kk[b], t = tt[b];
        int res = -1;
        if (k == gamma) {
            res = -2;
        } else if (k >= 0 && k < gamma && t >= 0) {
            std::vector<int32_t> want(path + (size_t)b * gamma, path + (size_t)b * gamma + k);
            want.push_back(t);
            for (int n = 0; n < N && res < 0; ++n) {
                // ancestors of n, n first; give up once the chain is longer than the prefix
                std::vector<int32_t> chain;
                int cur = n;
                bool valid = true;
                while (cur != -1) {
                    if (tok[cur] < 0 || par[cur] < -1 || par[cur] >= cur || (int)chain.size() > k) {
                        valid = false;
                        break;
                    }
                    chain.push_back(tok[cur]);
                    cur = par[cur];
                }
                if (!valid || (int)chain.size() != k + 1) continue;
                std::reverse(chain.begin(), chain.end());
                if (chain == want) res = n;
            }
        }
        out_node[b] = res;
        out_hit[b] = res >= 0 ? 1 : 0;
        hits += out_hit[b];
    }
    if (out_batch) {
        out_batch[0] = hits;
        out_batch[1] = hits == B ? 1 : 0;
    }
    return 0;
}

// Theorem 12 fan-out: F_k = F0 a^{k/(1+r)} for k < K, F_K = F0 a^{K/(1+r)} (1-a)^{-1/(1+r)},
// F0 chosen so the real values sum to the budget; integers by largest remainder (ties to the
// smaller k) so they sum to the budget exactly.
int orc_fanout(int K, int budget, double a, double r, double* real_out, int32_t* int_out) {
    if (K < 1 || budget < 0 || !(a > 0.0 && a < 1.0) || !(r > -1.0)) return -1;
    std::vector<double> w(K + 1);
    const double e = 1.0 / (1.0 + r);
    for (int k = 0; k < K; ++k) w[k] = std::pow(a, k * e);
    w[K] = std::pow(a, K * e) * std::pow(1.0 - a, -e);
    double sw = 0.0;
    for (double x : w) sw += x;
    const double F0 = budget / sw;
    std::vector<double> F(K + 1);
    int used = 0;
    std::vector<int> fl(K + 1);
    for (int k = 0; k <= K; ++k) {
        F[k] = F0 * w[k];
        fl[k] = (int)std::floor(F[k]);
        used += fl[k];
        if (real_out) real_out[k] = F[k];
    }
    std::vector<int> idx(K + 1);
    for (int k = 0; k <= K; ++k) idx[k] = k;
    std::stable_sort(idx.begin(), idx.end(), [&](int x, int y) { return (F[x] - fl[x]) > (F[y] - fl[y]); });
    for (int t = 0; t < budget - used; ++t) fl[idx[t]] += 1;
    if (int_out)
        for (int k = 0; k <= K; ++k) int_out[k] = fl[k];
    return 0;
}

// Cache construction: for depth k < K the first F_k tokens of draft row k in (logit desc, id asc)
// order other than the drafted token s_k; for depth K the first F_K tokens of draft row K.
// cache[B][sum F], depth-major, rank order, -1 where the row has fewer tokens.
int orc_cache_build(const void* draft, int dtype, int B, int K, int V, const int32_t* tokens, const int32_t* fanout,
                    int32_t* out_cache, int nthreads) {
    if (!draft || !tokens || !fanout || !out_cache || B < 1 || K < 1 || V < 1) return -1;
    int budget = 0;
    for (int k = 0; k <= K; ++k) {
        if (fanout[k] < 0) return -1;
        budget += fanout[k];
    }
    parallel_for(B * (K + 1), nthreads, [&](int bk) {
        int b = bk / (K + 1), k = bk % (K + 1);
        int off = 0;
        for (int t = 0; t < k; ++t) off += fanout[t];
        std::vector<double> z;
        load_row(draft, dtype, (size_t)b * (K + 1) + k, V, z);
        // NaN never ranks: it sorts after every number, then by id
        std::vector<int> ord(V);
        for (int i = 0; i < V; ++i) ord[i] = i;
        std::stable_sort(ord.begin(), ord.end(), [&](int x, int y) {
            const bool nx = std::isnan(z[x]), ny = std::isnan(z[y]);
            if (nx || ny) return !nx && ny;
            return z[x] > z[y];
        });
        const int excl = (k < K) ? tokens[(size_t)b * K + k] : -1;
        int n = 0;
        for (int t = 0; t < V && n < fanout[k]; ++t) {
            if (ord[t] == excl) continue;
            out_cache[(size_t)b * budget + off + n++] = ord[t];
        }
        for (; n < fanout[k]; ++n) out_cache[(size_t)b * budget + off + n] = -1;
    });
    return 0;
}

// Lookup.  mode 0: hit_b = t*_b in C_{k_b}; slot = offset(k_b) + rank, or -1.
// mode 1 (branch tree): per request the primary chain is branch 0; the committed prefix is its
// accepted tokens followed by t*; reuse = lowest branch whose first k+1 tokens equal it, -1 if
// none, -2 when every token was accepted (k == gamma).  k and t* are per chain [B][kappa].
int orc_cache_lookup(int mode, const int32_t* cache, const int32_t* fanout_or_shape, int K, int B, const int32_t* kk,
                     const int32_t* tt, int32_t* out_slot, uint8_t* out_hit, int32_t* out_batch) {
    if (!cache || !fanout_or_shape || !kk || !tt || !out_slot || !out_hit || B < 1) return -1;
    int hits = 0;
    if (mode == 0) {
        if (K < 1) return -1;
        int budget = 0;
        for (int k = 0; k <= K; ++k) budget += fanout_or_shape[k];
        for (int b = 0; b < B; ++b) {
            int k = kk[b], t = tt[b];
            int slot = -1;
            if (k >= 0 && k <= K && t >= 0) {
                int off = 0;
                for (int x = 0; x < k; ++x) off += fanout_or_shape[x];
                for (int f = 0; f < fanout_or_shape[k]; ++f)
                    if (cache[(size_t)b * budget + off + f] == t) {
                        slot = off + f;
                        break;
                    }
            }
            out_slot[b] = slot;
            out_hit[b] = slot >= 0 ? 1 : 0;
            hits += out_hit[b];
        }
    } else if (mode == 1) {
        const int kappa = fanout_or_shape[0], gamma = fanout_or_shape[1];
        if (kappa < 1 || gamma < 1) return -1;
        for (int b = 0; b < B; ++b) {
            const int32_t* br = cache + (size_t)b * kappa * gamma;
            int k = kk[(size_t)b * kappa], t = tt[(size_t)b * kappa];
            int res = -1;
            if (k == gamma) {
                res = -2;
            } else if (k >= 0 && k < gamma && t >= 0) {
                for (int j = 0; j < kappa && res < 0; ++j) {
                    bool ok = br[(size_t)j * gamma + k] == t;
                    for (int d = 0; d < k && ok; ++d) ok = br[(size_t)j * gamma + d] == br[d];
                    if (ok) res = j;
                }
            }
            out_slot[b] = res;
            out_hit[b] = res >= 0 ? 1 : 0;
            hits += out_hit[b];
        }
    } else {
        return -1;
    }
    if (out_batch) {
        out_batch[0] = hits;
        out_batch[1] = hits == B ? 1 : 0;
    }
    return 0;
}

}  // extern "C"
