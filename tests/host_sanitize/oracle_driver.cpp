// Host driver for the sanitizer build of the CPU oracle (AddressSanitizer + UndefinedBehavior-
// Sanitizer): every exported routine on small inputs, including bad rows, bad parameters,
// degenerate sets and the fuzzy and uniform-draft variants.  Any sanitizer report aborts.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

extern "C" {
void orc_philox4x64_10(const uint64_t* ctr, const uint64_t* key, uint64_t* out);
void orc_uniforms(uint64_t seed, uint64_t round, int B, int K, double* U);
int orc_process_row_f64(const double* z, int V, float temperature, int32_t top_k, float top_p, double* p_out,
                        int* near_cut, int* n_kept);
double orc_downweight_probs_f64(const double* z, double* p, int V, int F, double C, int32_t* ids, int* degenerate);
int orc_downweight(const void* draft, int draft_rows, int dtype, int B, int K, int V, const void* params, int F,
                   double C, int32_t* out_ids, double* out_Z, double* out_probs, uint32_t* out_status, int nthreads);
int orc_verify(const void* draft, int draft_rows, const void* target, int dtype, int B, int K, int V,
               const void* params, int F, double C, int32_t* tokens, int sample_draft, uint64_t seed, uint64_t round,
               int32_t* out_k, int32_t* out_t, double* out_W, uint32_t* out_status, uint32_t* out_flags,
               int nthreads, int uniform_draft, const double* tau, int assisted, double* out_div);
double orc_jsd_bits(const double* p, const double* q, int V);
void orc_uniform_tokens(const double* u, int n, int V, int32_t* out);
void orc_backup_plan(int B, const uint8_t* hit, int all_hit, int b_star, int32_t* out_use_backup, int32_t* out_switch);
int orc_signposts(const void* logits, int dtype, int B, int V, int kappa, int32_t* out_ids, double* out_logp,
                  uint32_t* out_status, int nthreads);
int orc_tree_lookup(const int32_t* tokens, const int32_t* parents, int B, int N, int gamma, const int32_t* path,
                    const int32_t* k, const int32_t* t, int32_t* out_node, uint8_t* out_hit, int32_t* out_batch);
int orc_fanout(int K, int budget, double a, double r, double* real_out, int32_t* int_out);
int orc_cache_build(const void* draft, int dtype, int B, int K, int V, const int32_t* tokens, const int32_t* fanout,
                    int32_t* out_cache, int nthreads);
int orc_cache_lookup(int mode, const int32_t* cache, const int32_t* fanout_or_shape, int K, int B, const int32_t* kk,
                     const int32_t* tt, int32_t* out_slot, uint8_t* out_hit, int32_t* out_batch);
}

struct Prm {
    float t;
    int32_t k;
    float p;
};

static uint16_t bf16(float x) {
    uint32_t u;
    std::memcpy(&u, &x, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

int main() {
    std::mt19937_64 rng(7);
    std::normal_distribution<float> nd(0.0f, 1.5f);
    int calls = 0;
    {
        uint64_t c[4] = {1, 2, 3, 4}, k[2] = {5, 6}, o[4];
        orc_philox4x64_10(c, k, o);
        std::vector<double> U(3 * 4 * 6);
        orc_uniforms(9, 2, 4, 5, U.data());
        calls += 2;
    }
    for (int V : {1, 2, 7, 64, 1000}) {
        for (int dtype : {0, 1}) {
            const int B = 6, K = 3, Kd = K + 1;
            std::vector<float> zt((size_t)B * (K + 1) * V), zd((size_t)B * Kd * V);
            for (auto& x : zt) x = nd(rng);
            for (auto& x : zd) x = nd(rng);
            zt[0] = NAN;                               // request 0: a bad target row
            if (V > 3) zd[(size_t)1 * Kd * V + 2] = -INFINITY;  // request 1: a -inf draft logit
            std::vector<uint16_t> ht(zt.size()), hd(zd.size());
            for (size_t i = 0; i < zt.size(); ++i) ht[i] = bf16(zt[i]);
            for (size_t i = 0; i < zd.size(); ++i) hd[i] = bf16(zd[i]);
            const void* T = dtype ? (const void*)ht.data() : (const void*)zt.data();
            const void* D = dtype ? (const void*)hd.data() : (const void*)zd.data();
            std::vector<Prm> prm = {{1.0f, 0, 1.0f}, {0.7f, 3, 0.9f}, {0.0f, 0, 1.0f},
                                    {-1.0f, 0, 1.0f}, {1.3f, 50, 0.5f}, {1.0f, 1, 0.95f}};
            std::vector<int32_t> tok((size_t)B * K), ok((size_t)B), ot((size_t)B);
            std::vector<double> W(B), tau(B, 0.3), div((size_t)B * K);
            std::vector<uint32_t> st(B), fl(B);
            for (int sample : {0, 1})
                for (int uni : {0, 1})
                    for (int fuzzy : {0, 1}) {
                        for (size_t i = 0; i < tok.size(); ++i) tok[i] = (int32_t)(rng() % (uint64_t)V);
                        orc_verify(D, Kd, T, dtype, B, K, V, prm.data(), 2, 0.3, tok.data(), sample, 11, 1, ok.data(),
                                   ot.data(), W.data(), st.data(), fl.data(), 2, uni, fuzzy ? tau.data() : nullptr,
                                   fuzzy, fuzzy ? div.data() : nullptr);
                        ++calls;
                    }
            std::vector<int32_t> ids((size_t)B * K * 4);
            std::vector<double> Z((size_t)B * K), probs((size_t)B * K * V);
            std::vector<uint32_t> dst((size_t)B * K);
            orc_downweight(D, Kd, dtype, B, K, V, prm.data(), 4, 0.0, ids.data(), Z.data(), probs.data(), dst.data(), 2);
            std::vector<int32_t> fan(K + 1);
            std::vector<double> real(K + 1);
            orc_fanout(K, 13, 0.7, 1.0, real.data(), fan.data());
            int budget = 0;
            for (int f : fan) budget += f;
            std::vector<int32_t> cache((size_t)B * budget);
            orc_cache_build(D, dtype, B, K, V, tok.data(), fan.data(), cache.data(), 2);
            std::vector<int32_t> slot(B);
            std::vector<uint8_t> hit(B);
            int32_t batch[2];
            orc_cache_lookup(0, cache.data(), fan.data(), K, B, ok.data(), ot.data(), slot.data(), hit.data(), batch);
            const int32_t shape[2] = {2, 3};
            std::vector<int32_t> br((size_t)B * 6);
            for (auto& x : br) x = (int32_t)(rng() % (uint64_t)V);
            std::vector<int32_t> kk(B, 1), tt(B, 0);  // per chain: B / 2 requests x kappa = 2
            orc_cache_lookup(1, br.data(), shape, 0, B / 2, kk.data(), tt.data(), slot.data(), hit.data(), batch);
            std::vector<int32_t> sid((size_t)B * 3);
            std::vector<double> slp((size_t)B * 3);
            std::vector<uint32_t> sst(B);
            orc_signposts(T, dtype, B, V, 3, sid.data(), slp.data(), sst.data(), 2);
            calls += 6;
        }
    }
    {
        const int V = 9;
        std::vector<double> z(V), p(V), q(V, 1.0 / V);
        for (auto& x : z) x = nd(rng);
        int near = 0, nk = 0;
        orc_process_row_f64(z.data(), V, 0.8f, 4, 0.9f, p.data(), &near, &nk);
        std::vector<int32_t> ids(3);
        int deg = 0;
        orc_downweight_probs_f64(z.data(), p.data(), V, 3, 0.25, ids.data(), &deg);
        orc_jsd_bits(p.data(), q.data(), V);
        std::vector<double> u = {0.1, 0.5, 0.999999};
        std::vector<int32_t> ut(3);
        orc_uniform_tokens(u.data(), 3, V, ut.data());
        std::vector<uint8_t> hit = {1, 0, 1, 1};
        std::vector<int32_t> use(4), sw(1);
        orc_backup_plan(4, hit.data(), 0, 2, use.data(), sw.data());
        // a tree with padding and a broken parent
        const int B = 2, N = 6, gamma = 3;
        std::vector<int32_t> tk = {1, 2, 3, 4, -1, 5, 1, 9, 9, 2, 3, 4};
        std::vector<int32_t> par = {-1, 0, 1, 0, -1, 7, -1, 0, 1, -1, 3, 4};
        std::vector<int32_t> path = {1, 2, 3, 2, 3, 4}, kk = {1, 3}, tt = {2, 0};
        std::vector<int32_t> node(B);
        std::vector<uint8_t> th(B);
        int32_t batch[2];
        orc_tree_lookup(tk.data(), par.data(), B, N, gamma, path.data(), kk.data(), tt.data(), node.data(), th.data(),
                        batch);
        calls += 6;
    }
    std::printf("oracle driver: %d calls clean\n", calls);
    return 0;
}
