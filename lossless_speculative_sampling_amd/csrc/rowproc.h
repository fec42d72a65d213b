// Whole-workgroup processing of one logit row read from global memory: temperature, top-k,
// softmax, nucleus and the Saguaro downweight, with exact radix selection on the 32-bit order
// key and fp64 masses.  Used by every entry point for fp32 rows and as the general path
// (any V, any parameters); the register-resident bf16 path lives in fastpath.hip.
//
// Processing follows the DeepMind speculative-sampling page, section 6 (temperature, top-k
// and nucleus act on draft and target alike, before the correction), in the order
// temperature -> top-k -> softmax -> nucleus.  The downweight is Saguaro sampling
// sigma_{F,C} from the SSD pages (reading notes section 4.4; hyper.ai summary, Method).
#pragma once

#include "common.h"
#include "generic.h"

namespace sv {

constexpr int kRowThreads = kRowThreadsHost;

// Row statistics, uniform across the workgroup (lives in LDS).
struct RowStats {
    int bad;       // NaN / +inf / no finite logit
    int greedy;    // temperature 0
    int argmax;    // lowest id among the largest logits
    float m;       // largest logit
    double T;
    uint32_t kk;   // top-k: kept iff key > kk, or key == kk and id <= idk
    int idk;
    uint32_t kp;   // nucleus: in iff kept and (key > kp, or key == kp and id <= idp)
    int idp;
    double S;      // normaliser over the nucleus
    // downweighted set: in nucleus, mass > 0, and key > kF or (key == kF and id <= idF)
    int nS;
    uint32_t kF;
    int idF;
    double C;      // factor on the set (1 when off)
    double Z;      // normaliser after the downweight (1 when off)
    int degenerate;
    int ids[SPEC_MAX_F];
};

struct RowShared {
    uint32_t hcnt[256];
    double hmass[256];
    double redd[32];
    unsigned long long redu[32];
    int redi[32];
    int sel_digit;
    double sel_acc;
    int found;
    int list_n;
    int list[SPEC_MAX_F + 1];
    uint32_t list_key[SPEC_MAX_F + 1];
};

struct RowRef {
    const void* row;
    int dtype;
    int V;
};

// ------------------------------------------------------------------------------------------
// Row traversals with A (default kRowAhead) independent loads in flight per thread (a loop that loads one
// logit per iteration and uses it at once is bound by that load's latency).  Every thread
// still visits its columns in increasing order, so its accumulations round as in a plain loop.
// ------------------------------------------------------------------------------------------
constexpr int kRowAhead = 8;

// columns threadIdx.x, threadIdx.x + blockDim.x, ... of one row (f(i, z)) or of two rows
// read pairwise by column (f(i, z, z2))
template <int A = kRowAhead, typename F>
__device__ __forceinline__ void row_strided(const RowRef& r, F&& f) {
    const int step = blockDim.x;
    int i = threadIdx.x;
    for (; i + (A - 1) * step < r.V; i += A * step) {
        float z[A];
#pragma unroll
        for (int u = 0; u < A; ++u) z[u] = load_logit(r.row, r.dtype, i + u * step);
#pragma unroll
        for (int u = 0; u < A; ++u) f(i + u * step, z[u]);
    }
    for (; i < r.V; i += step) f(i, load_logit(r.row, r.dtype, i));
}
template <int A = kRowAhead, typename F>
__device__ __forceinline__ void row_strided2(const RowRef& r, const RowRef& r2, F&& f) {
    const int step = blockDim.x;
    int i = threadIdx.x;
    for (; i + (A - 1) * step < r.V; i += A * step) {
        float z[A], z2[A];
#pragma unroll
        for (int u = 0; u < A; ++u) {
            z[u] = load_logit(r.row, r.dtype, i + u * step);
            z2[u] = load_logit(r2.row, r2.dtype, i + u * step);
        }
#pragma unroll
        for (int u = 0; u < A; ++u) f(i + u * step, z[u], z2[u]);
    }
    for (; i < r.V; i += step) f(i, load_logit(r.row, r.dtype, i), load_logit(r2.row, r2.dtype, i));
}

// Columns [i0, i0 + A) clipped to hi, loaded ahead (z, z2; 0 past hi).
template <bool TWO, int A>
__device__ __forceinline__ void load_ahead(const RowRef& r, const RowRef& r2, int i0, int hi, float (&z)[A],
                                           float (&z2)[A]) {
#pragma unroll
    for (int u = 0; u < A; ++u) {
        const bool in = i0 + u < hi;
        z[u] = in ? load_logit(r.row, r.dtype, i0 + u) : 0.0f;
        z2[u] = (TWO && in) ? load_logit(r2.row, r2.dtype, i0 + u) : 0.0f;
    }
}

__device__ __forceinline__ bool rs_kept(const RowStats& s, uint32_t key, int i) {
    return key > s.kk || (key == s.kk && i <= s.idk);
}
__device__ __forceinline__ bool rs_in(const RowStats& s, uint32_t key, int i) {
    return rs_kept(s, key, i) && (key > s.kp || (key == s.kp && i <= s.idp));
}
__device__ __forceinline__ double rs_mass(const RowStats& s, float z) {
    return exp(((double)z - (double)s.m) / s.T);
}
__device__ __forceinline__ bool rs_in_set(const RowStats& s, uint32_t key, int i, double e) {
    return s.nS > 0 && rs_in(s, key, i) && e > 0.0 && (key > s.kF || (key == s.kF && i <= s.idF));
}
// processed probability p_i (before the downweight)
__device__ __forceinline__ double rs_prob(const RowStats& s, float z, int i) {
    if (s.greedy) return i == s.argmax ? 1.0 : 0.0;
    const uint32_t key = order_key(z);
    if (!rs_in(s, key, i)) return 0.0;
    return rs_mass(s, z) / s.S;
}
// processed probability after the downweight, p'_i = p_i f_i / Z
__device__ __forceinline__ double rs_prob_dw(const RowStats& s, float z, int i) {
    if (s.greedy) return i == s.argmax ? 1.0 : 0.0;
    const uint32_t key = order_key(z);
    if (!rs_in(s, key, i)) return 0.0;
    const double e = rs_mass(s, z);
    const double p = e / s.S;
    const double f = rs_in_set(s, key, i, e) ? s.C : 1.0;
    return p * f / s.Z;
}

// Radix selection over the 32-bit key, 8 bits per pass from the top.  Walking keys from the
// largest down over elements accepted by `filt`, weighted by 1 (COUNT) or by the element's
// mass e_i, finds the key tau at which the running weight first reaches `need`.
// Outputs: tau, the weight strictly above tau, the number of filtered elements at tau and the
// weight still needed inside tau.
template <bool MASS, int A = kRowAhead, typename Filter>
__device__ __forceinline__ void radix_select(const RowRef& r, const RowStats& st, Filter filt, double need, RowShared& sh,
                             uint32_t* tau_out, double* above_out, int* cnt_out, double* rem_out) {
    uint32_t prefix = 0, pmask = 0;
    double above = 0.0, rem = need;
    int cnt_at = 0;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int d = threadIdx.x; d < 256; d += blockDim.x) {
            sh.hcnt[d] = 0;
            sh.hmass[d] = 0.0;
        }
        __syncthreads();
        row_strided<A>(r, [&](int i, float z) {
            const uint32_t key = order_key(z);
            if ((key & pmask) != prefix || !filt(key, i, z)) return;
            const int d = (key >> shift) & 255;
            atomicAdd(&sh.hcnt[d], 1u);
            if (MASS) atomicAdd(&sh.hmass[d], rs_mass(st, z));
        });
        __syncthreads();
        if (threadIdx.x == 0) {
            double acc = 0.0;
            int pick = -1, last_nz = -1;
            double acc_last = 0.0;
            for (int d = 255; d >= 0; --d) {
                const double w = MASS ? sh.hmass[d] : (double)sh.hcnt[d];
                if (sh.hcnt[d] == 0) continue;
                if (acc + w >= rem) {
                    pick = d;
                    break;
                }
                last_nz = d;
                acc_last = acc;
                acc += w;
            }
            if (pick < 0) {  // rounding left the target just out of reach: take the lowest bin
                pick = last_nz;
                acc = acc_last;
            }
            sh.sel_digit = pick;
            sh.sel_acc = acc;
        }
        __syncthreads();
        const int d = sh.sel_digit;
        above += sh.sel_acc;
        rem -= sh.sel_acc;
        cnt_at = d >= 0 ? (int)sh.hcnt[d] : 0;
        prefix |= (uint32_t)(d < 0 ? 0 : d) << shift;
        pmask |= 0xFFu << shift;
        __syncthreads();
    }
    *tau_out = prefix;
    *above_out = above;
    *cnt_out = cnt_at;
    *rem_out = rem;
}

// The n-th (1-based) smallest id among elements with key == tau accepted by `filt`.
// Threads own contiguous id segments, so a workgroup scan of their counts locates it.
template <int A = kRowAhead, typename Filter>
__device__ __forceinline__ int nth_id_at_key(const RowRef& r, uint32_t tau, int n, Filter filt, RowShared& sh) {
    const int seg = (r.V + blockDim.x - 1) / blockDim.x;
    const int lo = threadIdx.x * seg;
    const int hi = min(r.V, lo + seg);
    int c = 0;
    for (int i0 = lo; i0 < hi; i0 += A) {
        float z[A], z2[A];
        load_ahead<false, A>(r, r, i0, hi, z, z2);
#pragma unroll
        for (int u = 0; u < A; ++u) {
            const uint32_t k = order_key(z[u]);
            if (i0 + u < hi && k == tau && filt(k, i0 + u, z[u])) ++c;
        }
    }
    int total;
    const int before = block_exclusive_scan<int>(c, sh.redi, &total);
    if (threadIdx.x == 0) sh.found = r.V - 1;
    __syncthreads();
    if (before < n && before + c >= n) {
        int cc = before;
        bool done = false;
        for (int i0 = lo; i0 < hi && !done; i0 += A) {
            float z[A], z2[A];
            load_ahead<false, A>(r, r, i0, hi, z, z2);
            for (int u = 0; u < A && i0 + u < hi && !done; ++u) {
                const uint32_t k = order_key(z[u]);
                if (k == tau && filt(k, i0 + u, z[u]) && ++cc == n) {
                    sh.found = i0 + u;
                    done = true;
                }
            }
        }
    }
    __syncthreads();
    const int res = sh.found;
    __syncthreads();
    return res;
}

// Inverse CDF in token-id order over non-negative weights w(i, z) (or w(i, z, z2) over two rows
// read pairwise): the first i with w_i > 0 whose running sum exceeds x * total (the last i with
// w_i > 0 if rounding never crosses).  Returns -1 when every weight is 0.  *total_out gets the
// total.  Threads own contiguous column segments; the owner of the crossing walks its segment
// with its weights computed A at a time.
template <bool TWO, int A, typename Weight>
__device__ __forceinline__ void weights_ahead(const RowRef& r, const RowRef& r2, int i0, int hi, Weight& wfn,
                                              double (&w)[A]) {
    float z[A], z2[A];
    load_ahead<TWO, A>(r, r2, i0, hi, z, z2);
#pragma unroll
    for (int u = 0; u < A; ++u) {
        if (i0 + u >= hi) {
            w[u] = 0.0;
        } else if constexpr (TWO) {
            w[u] = wfn(i0 + u, z[u], z2[u]);
        } else {
            w[u] = wfn(i0 + u, z[u]);
        }
    }
}

template <bool TWO, int A, typename Weight>
__device__ __forceinline__ int inverse_cdf_rows(const RowRef& r, const RowRef& r2, double x, Weight wfn, RowShared& sh,
                                double* total_out) {
    const int seg = (r.V + blockDim.x - 1) / blockDim.x;
    const int lo = threadIdx.x * seg;
    const int hi = min(r.V, lo + seg);
    double own = 0.0;
    for (int i0 = lo; i0 < hi; i0 += A) {
        double w[A];
        weights_ahead<TWO, A>(r, r2, i0, hi, wfn, w);
#pragma unroll
        for (int u = 0; u < A; ++u)
            if (w[u] > 0.0) own += w[u];
    }
    double total;
    const double before = block_exclusive_scan<double>(own, sh.redd, &total);
    const double target = x * total;
    const int cand = (own > 0.0 && before <= target) ? (int)threadIdx.x : -1;
    const int owner = block_max<int>(cand, sh.redi);
    if (threadIdx.x == 0) sh.found = -1;
    __syncthreads();
    if ((int)threadIdx.x == owner) {
        double cum = before;
        int pick = -1;
        bool done = false;
        for (int i0 = lo; i0 < hi && !done; i0 += A) {
            double w[A];
            weights_ahead<TWO, A>(r, r2, i0, hi, wfn, w);
            for (int u = 0; u < A && !done; ++u) {
                if (!(w[u] > 0.0)) continue;
                cum += w[u];
                pick = i0 + u;
                if (cum > target) done = true;
            }
        }
        sh.found = pick;
    }
    __syncthreads();
    const int res = sh.found;
    *total_out = total;
    __syncthreads();
    return res;
}

template <int A = kRowAhead, typename Weight>
__device__ __forceinline__ int inverse_cdf(const RowRef& r, double x, Weight wfn, RowShared& sh, double* total_out) {
    return inverse_cdf_rows<false, A>(r, r, x, wfn, sh, total_out);
}
template <int A = kRowAhead, typename Weight>
__device__ __forceinline__ int inverse_cdf2(const RowRef& r, const RowRef& r2, double x, Weight wfn, RowShared& sh,
                            double* total_out) {
    return inverse_cdf_rows<true, A>(r, r2, x, wfn, sh, total_out);
}

// Processes row r with (T, top_k, top_p) into st (LDS).  When `want_set`, also forms the
// downweighted set of the first F tokens with mass and its normaliser Z for factor C.
template <int A = kRowAhead>
__device__ inline void process_row(const RowRef& r, float T, int top_k, float top_p, int F, double C, bool want_set,
                            RowStats& st, RowShared& sh) {
    // pass 1: bad logits and the (largest key, lowest id) pair
    unsigned long long best = 0;
    int bad = 0, finite = 0;
    row_strided<A>(r, [&](int i, float z) {
        const uint32_t u = __float_as_uint(z);
        if ((u & 0x7FFFFFFFu) > 0x7F800000u || u == 0x7F800000u) bad = 1;
        if ((u & 0x7F800000u) != 0x7F800000u) finite = 1;
        const unsigned long long pk = ((unsigned long long)order_key(z) << 32) | (unsigned long long)(~(uint32_t)i);
        best = pk > best ? pk : best;
    });
    bad = block_max<int>(bad, sh.redi);
    finite = block_max<int>(finite, sh.redi);
    best = block_max<unsigned long long>(best, sh.redu);
    if (threadIdx.x == 0) {
        st.bad = (bad || !finite) ? 1 : 0;
        st.argmax = (int)(~(uint32_t)(best & 0xFFFFFFFFull));
        st.m = key_to_float((uint32_t)(best >> 32));
        st.greedy = (T == 0.0f) ? 1 : 0;
        st.T = (double)T;
        st.kk = 0;
        st.idk = r.V - 1;
        st.kp = 0;
        st.idp = r.V - 1;
        st.S = 1.0;
        st.nS = 0;
        st.kF = 0xFFFFFFFFu;
        st.idF = -1;
        st.C = 1.0;
        st.Z = 1.0;
        st.degenerate = 0;
        for (int f = 0; f < SPEC_MAX_F; ++f) st.ids[f] = -1;
    }
    __syncthreads();
    if (st.bad || st.greedy) return;

    // top-k: exactly top_k tokens, ties by lower id
    if (top_k > 0 && top_k < r.V) {
        uint32_t tau;
        double above, rem;
        int cnt;
        radix_select<false, A>(r, st, [](uint32_t, int, float) { return true; }, (double)top_k, sh, &tau, &above, &cnt,
                            &rem);
        const int n = (int)rem;
        const int idk = (n >= cnt) ? r.V - 1 : nth_id_at_key<A>(r, tau, n, [](uint32_t, int, float) { return true; }, sh);
        if (threadIdx.x == 0) {
            st.kk = tau;
            st.idk = idk;
        }
        __syncthreads();
    }

    // softmax normaliser over the kept tokens
    double s = 0.0;
    row_strided<A>(r, [&](int i, float z) {
        if (rs_kept(st, order_key(z), i)) s += rs_mass(st, z);
    });
    const double S_kept = block_sum<double>(s, sh.redd);

    // nucleus: the smallest prefix of the order whose mass reaches top_p * S
    double S_nuc = S_kept;
    if ((double)top_p < 1.0) {
        const double need = (double)top_p * S_kept;
        uint32_t tau;
        double above, rem;
        int cnt;
        auto kept = [&st](uint32_t key, int i, float) { return rs_kept(st, key, i); };
        radix_select<true, A>(r, st, kept, need, sh, &tau, &above, &cnt, &rem);
        const double e_tau = exp(((double)key_to_float(tau) - (double)st.m) / st.T);
        int n = cnt;
        if (e_tau > 0.0) {
            const double q = ceil((need - above) / e_tau);
            n = q < 1.0 ? 1 : (q > (double)cnt ? cnt : (int)q);
        }
        const int idp = (n >= cnt) ? r.V - 1 : nth_id_at_key<A>(r, tau, n, kept, sh);
        S_nuc = above + (double)n * e_tau;
        if (threadIdx.x == 0) {
            st.kp = tau;
            st.idp = idp;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) st.S = S_nuc;
    __syncthreads();

    if (!want_set || F <= 0) return;
    // downweighted set: the first F tokens of the order that carry mass
    int c = 0;
    row_strided<A>(r, [&](int i, float z) {
        if (rs_in(st, order_key(z), i) && rs_mass(st, z) > 0.0) ++c;
    });
    const int n_pos = block_sum<int>(c, sh.redi);
    const int Fp = F < n_pos ? F : n_pos;
    if (Fp <= 0) return;
    auto pos = [&st](uint32_t key, int i, float z) { return rs_in(st, key, i) && rs_mass(st, z) > 0.0; };
    uint32_t tau;
    double above, rem;
    int cnt;
    radix_select<false, A>(r, st, pos, (double)Fp, sh, &tau, &above, &cnt, &rem);
    const int n = (int)rem;
    const int idF = (n >= cnt) ? r.V - 1 : nth_id_at_key<A>(r, tau, n, pos, sh);
    if (threadIdx.x == 0) {
        st.kF = tau;
        st.idF = idF;
        st.nS = Fp;
        sh.list_n = 0;
    }
    __syncthreads();
    double ps = 0.0;
    row_strided<A>(r, [&](int i, float z) {
        const uint32_t key = order_key(z);
        const double e = rs_mass(st, z);
        if (rs_in_set(st, key, i, e)) {
            const int slot = atomicAdd(&sh.list_n, 1);
            if (slot < SPEC_MAX_F) {
                sh.list[slot] = i;
                sh.list_key[slot] = key;
            }
            ps += e / st.S;
        }
    });
    const double P_S = block_sum<double>(ps, sh.redd);
    if (threadIdx.x == 0) {
        const int nl = sh.list_n < SPEC_MAX_F ? sh.list_n : SPEC_MAX_F;
        // rank order: key descending, id ascending
        for (int a = 1; a < nl; ++a) {
            const int id = sh.list[a];
            const uint32_t k = sh.list_key[a];
            int b = a - 1;
            while (b >= 0 && (sh.list_key[b] < k || (sh.list_key[b] == k && sh.list[b] > id))) {
                sh.list[b + 1] = sh.list[b];
                sh.list_key[b + 1] = sh.list_key[b];
                --b;
            }
            sh.list[b + 1] = id;
            sh.list_key[b + 1] = k;
        }
        for (int f = 0; f < nl; ++f) st.ids[f] = sh.list[f];
        if (C < 1.0) {
            const double Z = 1.0 - (1.0 - C) * P_S;
            if (Z > 0.0) {
                st.C = C;
                st.Z = Z;
            } else {
                st.degenerate = 1;
            }
        }
    }
    __syncthreads();
}

// The verification of one (request b, position j) unit by the whole workgroup; the record is
// written by thread 0.  Shared by the general kernel and the fast kernel's fallback.
template <int A = kRowAhead>
__device__ inline void unit_verify(const VerifyArgs& a, int b, int j, UnitRec* rec, RowShared& sh, RowStats& stq,
                            RowStats& stp) {
    const spec_params prm = a.params[b];
    const bool param_ok = prm.temperature >= 0.0f && !isinf(prm.temperature) && prm.top_p > 0.0f;
    if (!param_ok) {
        if (threadIdx.x == 0) *rec = UnitRec{0, -1, 0.0f, kStBadParam, -1};
        return;
    }
    const size_t tstride = (size_t)a.V * (a.dtype == SPEC_BF16 ? 2 : 4);
    const char* trow = static_cast<const char*>(a.target) + ((size_t)b * (a.K + 1) + j) * tstride;
    RowRef rq{trow, a.dtype, a.V};
    process_row<A>(rq, prm.temperature, prm.top_k, prm.top_p, 0, 1.0, false, stq, sh);
    // with a uniform draft (the random-token backup) p_j(x) = 1/V and no draft row is read
    const bool uni = (a.flags & SPEC_UNIFORM_DRAFT) != 0;
    const double p_uni = 1.0 / (double)a.V;
    RowRef rp{nullptr, a.dtype, a.V};
    if (j < a.K && !uni) {
        rp.row = static_cast<const char*>(a.draft) + ((size_t)b * a.draft_rows + j) * tstride;
        const bool dw = a.F > 0 && a.C < 1.0f;
        process_row<A>(rp, prm.temperature, prm.top_k, prm.top_p, a.F, (double)a.C, dw, stp, sh);
    }
    if (stq.bad || (j < a.K && !uni && stp.bad)) {
        if (threadIdx.x == 0) *rec = UnitRec{0, -1, 0.0f, kStBadLogit, -1};
        return;
    }
    uint32_t status = (j < a.K && !uni && stp.degenerate) ? kStDegenerate : 0u;
    const bool greedy = stq.greedy != 0;

    if (j == a.K) {  // bonus position
        int t;
        if (greedy) {
            t = stq.argmax;
        } else {
            const double v = uniform_at(a.seed, a.round, b, j, 1);
            double tot;
            t = inverse_cdf<A>(rq, v, [&](int i, float z) { return rs_prob(stq, z, i); }, sh, &tot);
        }
        if (threadIdx.x == 0) *rec = UnitRec{1, t, 0.0f, status, -1};
        return;
    }

    // draft token s_j (sampled here under SPEC_SAMPLE_DRAFT)
    int s;
    if (a.flags & SPEC_SAMPLE_DRAFT) {
        if (uni) {
            s = uniform_draft_token(a.seed, a.round, b, j, a.V);
        } else if (greedy) {
            s = stp.argmax;
        } else {
            const double x = uniform_at(a.seed, a.round, b, j, 2);
            double tot;
            s = inverse_cdf<A>(rp, x, [&](int i, float z) { return rs_prob_dw(stp, z, i); }, sh, &tot);
        }
        if (threadIdx.x == 0) a.tokens[(size_t)b * a.K + j] = s;
    } else {
        s = a.tokens[(size_t)b * a.K + j];
    }
    if (s < 0 || s >= a.V) {
        if (threadIdx.x == 0) *rec = UnitRec{0, -1, 0.0f, status | kStBadToken, s};
        return;
    }

    // fuzzy acceptance (PyramidSD notes, key design 1): the drafted token passes when the
    // Jensen-Shannon divergence (bits) of q_j and p'_j is at most the request's threshold;
    // otherwise the lossless test below decides
    bool fuzzy_pass = false;
    if (a.tau) {
        double d = 0.0;
        auto term = [&](double q, double p) {
            const double m = 0.5 * (p + q);
            if (p > 0.0) d += 0.5 * p * log2(p / m);
            if (q > 0.0) d += 0.5 * q * log2(q / m);
        };
        if constexpr (A == 1) {
            for (int i = threadIdx.x; i < a.V; i += blockDim.x)
                term(rs_prob(stq, load_logit(rq.row, a.dtype, i), i),
                     uni ? p_uni : rs_prob_dw(stp, load_logit(rp.row, a.dtype, i), i));
        } else if (uni) {
            row_strided<A>(rq, [&](int i, float zq) { term(rs_prob(stq, zq, i), p_uni); });
        } else {
            row_strided2<A>(rq, rp, [&](int i, float zq, float zp) { term(rs_prob(stq, zq, i), rs_prob_dw(stp, zp, i)); });
        }
        const double D = block_sum<double>(d, sh.redd);
        if (threadIdx.x == 0 && a.out_div) a.out_div[(size_t)b * a.K + j] = (float)D;
        fuzzy_pass = D <= (double)a.tau[b];
    }
    bool accept;
    if (fuzzy_pass) {
        accept = true;
    } else if (greedy) {
        accept = (s == stq.argmax);
    } else {
        const double ps = uni ? p_uni : rs_prob_dw(stp, load_logit(rp.row, a.dtype, s), s);
        const double qs = rs_prob(stq, load_logit(rq.row, a.dtype, s), s);
        if (!(ps > 0.0)) status |= kStOutside;
        const double u = uniform_at(a.seed, a.round, b, j, 0);
        accept = u * ps < qs;
    }
    if (accept) {
        if (threadIdx.x == 0) *rec = UnitRec{1, -1, 0.0f, status, s};
        return;
    }
    int t;
    double W = 0.0;
    if (greedy) {
        t = stq.argmax;
    } else {
        const double v = uniform_at(a.seed, a.round, b, j, 1);
        // residual (q - p')+ at this position; rows are read pairwise by token id
        if constexpr (A == 1) {  // one instance for both draft kinds (fewer registers)
            t = inverse_cdf<A>(rq, v, [&](int i, float zq) {
                const double q = rs_prob(stq, zq, i);
                const double p = uni ? p_uni : rs_prob_dw(stp, load_logit(rp.row, a.dtype, i), i);
                return q > p ? q - p : 0.0;
            }, sh, &W);
        } else if (uni) {
            t = inverse_cdf<A>(rq, v, [&](int i, float zq) {
                const double q = rs_prob(stq, zq, i);
                return q > p_uni ? q - p_uni : 0.0;
            }, sh, &W);
        } else {
            t = inverse_cdf2<A>(rq, rp, v, [&](int i, float zq, float zp) {
                const double q = rs_prob(stq, zq, i);
                const double p = rs_prob_dw(stp, zp, i);
                return q > p ? q - p : 0.0;
            }, sh, &W);
        }
        if (a.flags & SPEC_ASSISTED) {
            // assisted correction (PyramidSD notes, key design 2): drawn from q_j itself
            double tot;
            t = inverse_cdf<A>(rq, v, [&](int i, float z) { return rs_prob(stq, z, i); }, sh, &tot);
        } else if (t < 0) {  // no residual mass: fall back to q itself
            status |= kStEmptyResidual;
            double tot;
            t = inverse_cdf<A>(rq, v, [&](int i, float z) { return rs_prob(stq, z, i); }, sh, &tot);
        }
    }
    if (threadIdx.x == 0) *rec = UnitRec{0, t, (float)W, status, s};
}

// ------------------------------------------------------------------------------------------
// Saguaro outcome cache, one (request b, depth k) row: C_k = the first F_k tokens of draft row
// k in token order (raw logit descending, id ascending, NaN last), leaving out the drafted
// token s_k; C_K from draft row K (SSD reading notes, section 4.3).  Any workgroup size.
// ------------------------------------------------------------------------------------------
struct CacheShared {
    int picked[SPEC_MAX_FANOUT + 1];
    uint32_t pkey[SPEC_MAX_FANOUT + 1];
    int npicked;
};

// Fk, off: a.fanout's entries at depth k, read by the caller (a copy of the fan-out arrays
// indexed by a runtime depth would live in private memory).
template <int A = kRowAhead>
__device__ inline void cache_row(const CacheArgs& a, int b, int k, int Fk, int off, RowShared& sh, RowStats& st,
                                 CacheShared& cs) {
    int32_t* out = a.out_cache + (size_t)b * a.budget + off;
    if (Fk <= 0) return;
    const size_t stride = (size_t)a.V * (a.dtype == SPEC_BF16 ? 2 : 4);
    RowRef r{static_cast<const char*>(a.draft) + ((size_t)b * (a.K + 1) + k) * stride, a.dtype, a.V};
    const int excl = (k < a.K) ? a.tokens[(size_t)b * a.K + k] : -1;
    const int want = min(a.V, Fk + (excl >= 0 && excl < a.V ? 1 : 0));
    uint32_t tau;
    double above, rem;
    int cnt;
    auto all = [](uint32_t, int, float) { return true; };
    radix_select<false, A>(r, st, all, (double)want, sh, &tau, &above, &cnt, &rem);
    const int n = (int)rem;
    const int idc = (n >= cnt) ? a.V - 1 : nth_id_at_key<A>(r, tau, n, all, sh);
    if (threadIdx.x == 0) cs.npicked = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < a.V; i += blockDim.x) {
        const uint32_t key = order_key(load_logit(r.row, a.dtype, i));
        if (key > tau || (key == tau && i <= idc)) {
            const int slot = atomicAdd(&cs.npicked, 1);
            if (slot <= SPEC_MAX_FANOUT) {
                cs.picked[slot] = i;
                cs.pkey[slot] = key;
            }
        }
    }
    __syncthreads();
    const int np = min(cs.npicked, want);
    bool excl_picked = false;
    for (int y = 0; y < np; ++y) excl_picked |= (cs.picked[y] == excl);
    // rank of each picked token in (key desc, id asc) order, less one past the drafted token
    for (int x = threadIdx.x; x < np; x += blockDim.x) {
        const int id = cs.picked[x];
        if (id == excl) continue;
        const uint32_t key = cs.pkey[x];
        int rank = 0;
        for (int y = 0; y < np; ++y) {
            const uint32_t ky = cs.pkey[y];
            if ((ky > key || (ky == key && cs.picked[y] < id)) && cs.picked[y] != excl) ++rank;
        }
        if (rank < Fk) out[rank] = id;
    }
    // rows shorter than the fan-out: pad with -1
    const int written = min(Fk, np - (excl_picked ? 1 : 0));
    for (int x = written + threadIdx.x; x < Fk; x += blockDim.x) out[x] = -1;
}

}  // namespace sv
