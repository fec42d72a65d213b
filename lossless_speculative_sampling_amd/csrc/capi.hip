// The C ABI: argument validation, workspace layout and kernel launches.
#include <cmath>
#include <cstring>
#include <mutex>

#include "fast_common.h"
#include "fastpath.h"
#include "generic.h"
#include "mirror.h"

using namespace sv;

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool valid_dtype(int dtype) { return dtype == SPEC_FP32 || dtype == SPEC_BF16; }

int launch_status() { return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP; }

// Workgroup size of the general path's per-position kernel: about 16 columns per thread,
// between one wave and 1024 threads (small vocabularies keep few waves per barrier; measured
// on 10^4 requests at V = 1024: 3.47 ms with 1024 threads, 0.84 with 256, 0.55 with 64).
unsigned general_threads(int V) {
    unsigned t = kWave;
    while (t < (unsigned)kRowThreadsHost && (long long)t * 16 < V) t *= 2;
    return t;
}

// Theorem 12 allocation (SSD reading notes section 4.3; hyper.ai summary, Method):
// weights a^{k/(1+r)} for k < K and a^{K/(1+r)} (1-a)^{-1/(1+r)} for k = K, scaled to the
// budget, then rounded by largest remainder with ties to the smaller depth.
int fanout_host(int K, int budget, double a, double r, int32_t* out) {
    if (K < 1 || K > kMaxK || budget < 0 || !(a > 0.0 && a < 1.0) || !(r > -1.0)) return SPEC_EINVAL;
    const double e = 1.0 / (1.0 + r);
    double w[kMaxK + 1], sum = 0.0;
    for (int k = 0; k <= K; ++k) {
        w[k] = std::pow(a, (double)k * e);
        if (k == K) w[k] *= std::pow(1.0 - a, -e);
        sum += w[k];
    }
    double frac[kMaxK + 1];
    int total = 0;
    for (int k = 0; k <= K; ++k) {
        const double real = (double)budget * w[k] / sum;
        const double fl = std::floor(real);
        out[k] = (int32_t)fl;
        frac[k] = real - fl;
        total += out[k];
    }
    for (int extra = budget - total; extra > 0; --extra) {
        int best = -1;
        for (int k = 0; k <= K; ++k)
            if (frac[k] >= 0.0 && (best < 0 || frac[k] > frac[best])) best = k;
        out[best] += 1;
        frac[best] = -1.0;
    }
    return SPEC_OK;
}

}  // namespace

extern "C" {

size_t spec_workspace_bytes(int B, int K, int V) {
    if (B < 1 || K < 1 || V < 1) return 0;
    return align_up((size_t)B * (K + 1) * sizeof(UnitRec), 256) + fast::fast_plan(B, K, V).ws_bytes;
}

int spec_verify(const void* draft_logits, int draft_rows, const void* target_logits, int dtype, int B, int K,
                int V, const spec_params* params, int F, float C, int32_t* draft_tokens, uint64_t seed,
                uint64_t round, uint32_t flags, int32_t* out_k, int32_t* out_tstar, float* out_resid_mass,
                uint32_t* out_status, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const bool uniform = (flags & SPEC_UNIFORM_DRAFT) != 0;
    if ((!draft_logits && !uniform) || !target_logits || !params || !draft_tokens || !out_k || !out_tstar)
        return SPEC_EINVAL;
    if (B < 1 || K < 1 || V < 1 || (!uniform && draft_rows != K && draft_rows != K + 1)) return SPEC_EINVAL;
    if (F < 0 || F > SPEC_MAX_F || !(C >= 0.0f && C <= 1.0f)) return SPEC_EINVAL;
    if ((flags & ~(uint32_t)(SPEC_SAMPLE_DRAFT | SPEC_UNIFORM_DRAFT)) != 0) return SPEC_EINVAL;
    if (!valid_dtype(dtype)) return SPEC_EDTYPE;
    const size_t need = spec_workspace_bytes(B, K, V);
    if (!workspace || workspace_bytes < need) return SPEC_EWORKSPACE;
    if (uniform) {
        // no draft row is read: the target stands in as a valid address, and sigma_{F,C} is off
        draft_logits = target_logits;
        draft_rows = K + 1;
        F = 0;
        C = 1.0f;
    }
    VerifyArgs a{draft_logits, target_logits, draft_rows, dtype, B, K, V, params, F, C, draft_tokens, seed,
                 round, flags, out_k, out_tstar, out_resid_mass, out_status, static_cast<UnitRec*>(workspace)};
    if (fast::fast_path_applies(a)) {
        const size_t gen = align_up((size_t)B * (K + 1) * sizeof(UnitRec), 256);
        return fast::fast_verify(a, static_cast<char*>(workspace) + gen, workspace_bytes - gen, stream);
    }
    hipLaunchKernelGGL(generic_unit_kernel, dim3((unsigned)(B * (K + 1))), dim3(general_threads(V)), 0, stream, a);
    if (launch_status() != SPEC_OK) return SPEC_EHIP;
    hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, stream, a);
    return launch_status();
}

int pyramid_verify(const void* draft_logits, int draft_rows, const void* verifier_logits, int dtype, int B, int K,
                   int V, const spec_params* params, int F, float C, const float* tau, int32_t* draft_tokens,
                   uint64_t seed, uint64_t round, uint32_t flags, int32_t* out_k, int32_t* out_tstar,
                   float* out_resid_mass, uint32_t* out_status, float* out_div, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
    const bool uniform = (flags & SPEC_UNIFORM_DRAFT) != 0;
    if ((!draft_logits && !uniform) || !verifier_logits || !params || !tau || !draft_tokens || !out_k || !out_tstar)
        return SPEC_EINVAL;
    if (B < 1 || K < 1 || V < 1 || (!uniform && draft_rows != K && draft_rows != K + 1)) return SPEC_EINVAL;
    if (F < 0 || F > SPEC_MAX_F || !(C >= 0.0f && C <= 1.0f)) return SPEC_EINVAL;
    if ((flags & ~(uint32_t)(SPEC_SAMPLE_DRAFT | SPEC_UNIFORM_DRAFT | SPEC_ASSISTED)) != 0) return SPEC_EINVAL;
    if (!valid_dtype(dtype)) return SPEC_EDTYPE;
    if (!workspace || workspace_bytes < spec_workspace_bytes(B, K, V)) return SPEC_EWORKSPACE;
    if (uniform) {
        draft_logits = verifier_logits;
        draft_rows = K + 1;
        F = 0;
        C = 1.0f;
    }
    VerifyArgs a{draft_logits, verifier_logits, draft_rows, dtype, B, K, V, params, F, C, draft_tokens, seed,
                 round, flags, out_k, out_tstar, out_resid_mass, out_status, static_cast<UnitRec*>(workspace),
                 tau, out_div};
    if (fast::fast_fuzzy_applies(a)) {
        const size_t gen = align_up((size_t)B * (K + 1) * sizeof(UnitRec), 256);
        return fast::fast_verify(a, static_cast<char*>(workspace) + gen, workspace_bytes - gen, stream);
    }
    hipLaunchKernelGGL(generic_unit_kernel, dim3((unsigned)(B * (K + 1))), dim3(general_threads(V)), 0, stream, a);
    if (launch_status() != SPEC_OK) return SPEC_EHIP;
    hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, stream, a);
    return launch_status();
}

int saguaro_backup_plan(int B, const uint8_t* hit, const int32_t* batch, int b_star, int32_t* out_use_backup,
                        int32_t* out_switch, hipStream_t stream) {
    if (!hit || !batch || !out_use_backup || !out_switch || B < 1) return SPEC_EINVAL;
    BackupArgs a{B, hit, batch, b_star, out_use_backup, out_switch};
    const int blocks = (B + 255) / 256 < 1024 ? (B + 255) / 256 : 1024;
    hipLaunchKernelGGL(backup_plan_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return launch_status();
}

int saguaro_downweight(const void* draft_logits, int draft_rows, int dtype, int B, int K, int V,
                       const spec_params* params, int F, float C, int32_t* out_ids, float* out_Z, float* out_probs,
                       uint32_t* out_status, hipStream_t stream) {
    if (!draft_logits || !params || (F > 0 && !out_ids)) return SPEC_EINVAL;
    if (B < 1 || K < 1 || V < 1 || draft_rows < K) return SPEC_EINVAL;
    if (F < 0 || F > SPEC_MAX_F || !(C >= 0.0f && C <= 1.0f)) return SPEC_EINVAL;
    if (!valid_dtype(dtype)) return SPEC_EDTYPE;
    DownweightArgs a{draft_logits, draft_rows, dtype, B, K, V, params, F, C, out_ids, out_Z, out_probs, out_status};
    hipLaunchKernelGGL(downweight_kernel, dim3((unsigned)(B * K)), dim3(kRowThreadsHost), 0, stream, a);
    return launch_status();
}

int saguaro_fanout(int K, int budget, double a, double r, int32_t* out_fanout) {
    if (!out_fanout) return SPEC_EINVAL;
    return fanout_host(K, budget, a, r, out_fanout);
}

int saguaro_cache_build(const void* draft_logits, int dtype, int B, int K, int V, const int32_t* draft_tokens,
                        int budget, double a, double r, int32_t* out_fanout_host, int32_t* out_cache,
                        hipStream_t stream) {
    if (!draft_logits || !draft_tokens || !out_cache || B < 1 || K < 1 || V < 1) return SPEC_EINVAL;
    if (!valid_dtype(dtype)) return SPEC_EDTYPE;
    CacheArgs c{};
    const int rc = fanout_host(K, budget, a, r, c.fanout.f);
    if (rc != SPEC_OK) return rc;
    c.fanout.off[0] = 0;
    for (int k = 0; k <= K; ++k) {
        if (c.fanout.f[k] > SPEC_MAX_FANOUT) return SPEC_EINVAL;
        c.fanout.off[k + 1] = c.fanout.off[k] + c.fanout.f[k];
    }
    if (out_fanout_host) std::memcpy(out_fanout_host, c.fanout.f, sizeof(int32_t) * (K + 1));
    c.draft = draft_logits;
    c.dtype = dtype;
    c.B = B;
    c.K = K;
    c.V = V;
    c.tokens = draft_tokens;
    c.budget = budget;
    c.out_cache = out_cache;
    if (budget == 0) return SPEC_OK;
    hipLaunchKernelGGL(cache_build_kernel, dim3((unsigned)(B * (K + 1))), dim3(kRowThreadsHost), 0, stream, c);
    return launch_status();
}

}  // extern "C"

namespace {
// The host-detectable argument errors of saguaro_verify_cache (workspace aside), and the fan-out.
int verify_cache_args(const void* draft_logits, const void* target_logits, int dtype, int B, int K, int V,
                      const spec_params* params, int F, float C, const int32_t* draft_tokens, uint32_t flags,
                      int budget, double a, double r, const int32_t* out_k, const int32_t* out_tstar,
                      const int32_t* out_cache, CacheArgs* c) {
    if (!draft_logits || !target_logits || !params || !draft_tokens || !out_k || !out_tstar || !out_cache)
        return SPEC_EINVAL;
    if (B < 1 || K < 1 || V < 1) return SPEC_EINVAL;
    if (F < 0 || F > SPEC_MAX_F || !(C >= 0.0f && C <= 1.0f)) return SPEC_EINVAL;
    if ((flags & ~(uint32_t)SPEC_SAMPLE_DRAFT) != 0) return SPEC_EINVAL;
    if (!valid_dtype(dtype)) return SPEC_EDTYPE;
    const int frc = fanout_host(K, budget, a, r, c->fanout.f);
    if (frc != SPEC_OK) return frc;
    c->fanout.off[0] = 0;
    for (int k = 0; k <= K; ++k) {
        if (c->fanout.f[k] > SPEC_MAX_FANOUT) return SPEC_EINVAL;
        c->fanout.off[k + 1] = c->fanout.off[k] + c->fanout.f[k];
    }
    return SPEC_OK;
}
}  // namespace

extern "C" {

int saguaro_verify_cache(const void* draft_logits, const void* target_logits, int dtype, int B, int K, int V,
                         const spec_params* params, int F, float C, int32_t* draft_tokens, uint64_t seed, uint64_t round,
                         uint32_t flags, int budget, double a, double r, int32_t* out_fanout_host, int32_t* out_k,
                         int32_t* out_tstar, float* out_resid_mass, uint32_t* out_status, int32_t* out_cache,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
    CacheArgs c{};
    const int arc = verify_cache_args(draft_logits, target_logits, dtype, B, K, V, params, F, C, draft_tokens, flags,
                                      budget, a, r, out_k, out_tstar, out_cache, &c);
    if (arc != SPEC_OK) return arc;
    const size_t need = spec_workspace_bytes(B, K, V);
    if (!workspace || workspace_bytes < need) return SPEC_EWORKSPACE;
    if (out_fanout_host) std::memcpy(out_fanout_host, c.fanout.f, sizeof(int32_t) * (K + 1));
    c.draft = draft_logits;
    c.dtype = dtype;
    c.B = B;
    c.K = K;
    c.V = V;
    c.tokens = draft_tokens;
    c.budget = budget;
    c.out_cache = out_cache;
    VerifyArgs v{draft_logits, target_logits, K + 1, dtype, B, K, V, params, F, C, draft_tokens, seed,
                 round, flags, out_k, out_tstar, out_resid_mass, out_status, static_cast<UnitRec*>(workspace)};
    if (fast::fast_cache_applies(v, c)) {
        const size_t gen = align_up((size_t)B * (K + 1) * sizeof(UnitRec), 256);
        return fast::fast_verify_cache(v, c, static_cast<char*>(workspace) + gen, workspace_bytes - gen, stream);
    }
    // otherwise the two calls one after the other (the drafted tokens are final after the first)
    const int vrc = spec_verify(draft_logits, K + 1, target_logits, dtype, B, K, V, params, F, C, draft_tokens, seed,
                                round, flags, out_k, out_tstar, out_resid_mass, out_status, workspace, workspace_bytes,
                                stream);
    if (vrc != SPEC_OK) return vrc;
    if (budget == 0) return SPEC_OK;
    hipLaunchKernelGGL(cache_build_kernel, dim3((unsigned)(B * (K + 1))), dim3(kRowThreadsHost), 0, stream, c);
    return launch_status();
}

namespace {
// saguaro_verify_cache_lookup, with optional events around the count kernel of the bf16 path
int verify_cache_lookup_impl(const void* draft_logits, const void* target_logits, int dtype, int B, int K, int V,
                             const spec_params* params, int F, float C, int32_t* draft_tokens, uint64_t seed,
                             uint64_t round, uint32_t flags, int budget, double a, double r, int32_t* out_fanout_host,
                             int32_t* out_k, int32_t* out_tstar, float* out_resid_mass, uint32_t* out_status,
                             int32_t* out_cache, int32_t* out_slot, uint8_t* out_hit, int32_t* out_batch,
                             void* workspace, size_t workspace_bytes, hipStream_t stream,
                             const fast::CountEvents* ev) {
    CacheArgs c{};
    const int arc = verify_cache_args(draft_logits, target_logits, dtype, B, K, V, params, F, C, draft_tokens, flags,
                                      budget, a, r, out_k, out_tstar, out_cache, &c);
    if (arc != SPEC_OK) return arc;
    if (!out_slot || !out_hit) return SPEC_EINVAL;
    const size_t need = spec_workspace_bytes(B, K, V);
    if (!workspace || workspace_bytes < need) return SPEC_EWORKSPACE;
    c.draft = draft_logits;
    c.dtype = dtype;
    c.B = B;
    c.K = K;
    c.V = V;
    c.tokens = draft_tokens;
    c.budget = budget;
    c.out_cache = out_cache;
    VerifyArgs v{draft_logits, target_logits, K + 1, dtype, B, K, V, params, F, C, draft_tokens, seed,
                 round, flags, out_k, out_tstar, out_resid_mass, out_status, static_cast<UnitRec*>(workspace)};
    if (budget > 0 && fast::fast_cache_applies(v, c) && fast::fast_lookup_fuses(v)) {
        if (out_fanout_host) std::memcpy(out_fanout_host, c.fanout.f, sizeof(int32_t) * (K + 1));
        const size_t gen = align_up((size_t)B * (K + 1) * sizeof(UnitRec), 256);
        const fast::LookupOut lk{out_slot, out_hit, out_batch};
        return fast::fast_verify_cache_lookup(v, c, lk, static_cast<char*>(workspace) + gen, workspace_bytes - gen,
                                              stream, ev);
    }
    // otherwise the two calls one after the other (events around the whole first call)
    if (ev && ev->before && hipEventRecord(ev->before, stream) != hipSuccess) return SPEC_EHIP;
    const int vrc = saguaro_verify_cache(draft_logits, target_logits, dtype, B, K, V, params, F, C, draft_tokens, seed,
                                         round, flags, budget, a, r, out_fanout_host, out_k, out_tstar, out_resid_mass,
                                         out_status, out_cache, workspace, workspace_bytes, stream);
    if (vrc != SPEC_OK) return vrc;
    if (ev && ev->after && hipEventRecord(ev->after, stream) != hipSuccess) return SPEC_EHIP;
    return saguaro_cache_lookup(0, out_cache, c.fanout.f, K, B, out_k, out_tstar, out_slot, out_hit, out_batch, stream);
}
}  // namespace

int saguaro_verify_cache_lookup(const void* draft_logits, const void* target_logits, int dtype, int B, int K, int V,
                                const spec_params* params, int F, float C, int32_t* draft_tokens, uint64_t seed,
                                uint64_t round, uint32_t flags, int budget, double a, double r, int32_t* out_fanout_host,
                                int32_t* out_k, int32_t* out_tstar, float* out_resid_mass, uint32_t* out_status,
                                int32_t* out_cache, int32_t* out_slot, uint8_t* out_hit, int32_t* out_batch,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return verify_cache_lookup_impl(draft_logits, target_logits, dtype, B, K, V, params, F, C, draft_tokens, seed, round,
                                    flags, budget, a, r, out_fanout_host, out_k, out_tstar, out_resid_mass, out_status,
                                    out_cache, out_slot, out_hit, out_batch, workspace, workspace_bytes, stream, nullptr);
}

int saguaro_verify_cache_lookup_timed(const void* draft_logits, const void* target_logits, int dtype, int B, int K,
                                      int V, const spec_params* params, int F, float C, int32_t* draft_tokens,
                                      uint64_t seed, uint64_t round, uint32_t flags, int budget, double a, double r,
                                      int32_t* out_fanout_host, int32_t* out_k, int32_t* out_tstar,
                                      float* out_resid_mass, uint32_t* out_status, int32_t* out_cache,
                                      int32_t* out_slot, uint8_t* out_hit, int32_t* out_batch, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream, hipEvent_t count_before,
                                      hipEvent_t count_after) {
    if (!count_before || !count_after) return SPEC_EINVAL;
    const fast::CountEvents ev{count_before, count_after};
    return verify_cache_lookup_impl(draft_logits, target_logits, dtype, B, K, V, params, F, C, draft_tokens, seed, round,
                                    flags, budget, a, r, out_fanout_host, out_k, out_tstar, out_resid_mass, out_status,
                                    out_cache, out_slot, out_hit, out_batch, workspace, workspace_bytes, stream, &ev);
}



int saguaro_cache_lookup(int mode, const int32_t* cache, const int32_t* fanout_or_shape, int K, int B,
                         const int32_t* k, const int32_t* tstar, int32_t* out_slot, uint8_t* out_hit,
                         int32_t* out_batch, hipStream_t stream) {
    if (!cache || !fanout_or_shape || !k || !tstar || !out_slot || !out_hit || B < 1) return SPEC_EINVAL;
    LookupArgs l{};
    l.mode = mode;
    l.cache = cache;
    l.B = B;
    l.K = K;
    l.k = k;
    l.tstar = tstar;
    l.out_slot = out_slot;
    l.out_hit = out_hit;
    l.out_batch = out_batch;
    if (mode == 0) {
        if (K < 1 || K > kMaxK) return SPEC_EINVAL;
        l.fanout.off[0] = 0;
        for (int x = 0; x <= K; ++x) {
            if (fanout_or_shape[x] < 0) return SPEC_EINVAL;
            l.fanout.f[x] = fanout_or_shape[x];
            l.fanout.off[x + 1] = l.fanout.off[x] + fanout_or_shape[x];
        }
        l.budget = l.fanout.off[K + 1];
    } else if (mode == 1) {
        l.kappa = fanout_or_shape[0];
        l.gamma = fanout_or_shape[1];
        if (l.kappa < 1 || l.gamma < 1) return SPEC_EINVAL;
    } else {
        return SPEC_EINVAL;
    }
    // one workgroup, a thread per request up to 1024 (whole waves: a single wave needs no barrier
    // wait in the batch count)
    const unsigned threads = (unsigned)std::min(1024, (B + kWave - 1) / kWave * kWave);
    hipLaunchKernelGGL(cache_lookup_kernel, dim3(1), dim3(threads), 0, stream, l);
    return launch_status();
}

size_t mirror_signpost_workspace_bytes(int B, int V, int kappa) {
    if (B < 1 || V < 1 || V > mirror::kMaxV || kappa < 1 || kappa > SPEC_MAX_KAPPA) return 0;
    return mirror::signpost_plan(B, V, kappa).ws_bytes;
}

int mirror_signposts(const void* logits, int dtype, int B, int V, int kappa, int32_t* out_ids, float* out_logp,
                     uint16_t* out_logp_bf16, uint32_t* out_status, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
    if (!logits || !out_ids || !out_logp) return SPEC_EINVAL;
    if (B < 1 || V < 1 || V > mirror::kMaxV || kappa < 1 || kappa > SPEC_MAX_KAPPA) return SPEC_EINVAL;
    if (!valid_dtype(dtype)) return SPEC_EDTYPE;
    const mirror::SpPlan plan = mirror::signpost_plan(B, V, kappa);
    if (plan.lds_bytes > 64 * 1024) return SPEC_EINVAL;  // (not reached within the size limits)
    if (!workspace || workspace_bytes < plan.ws_bytes) return SPEC_EWORKSPACE;
    const size_t esz = dtype == SPEC_BF16 ? 2 : 4;
    const int vec = ((reinterpret_cast<uintptr_t>(logits) & 15) == 0 && ((size_t)V * esz) % 16 == 0) ? 1 : 0;
    mirror::SignpostArgs a{logits, dtype, B, V, kappa, plan, out_ids, out_logp, out_logp_bf16, out_status,
                           static_cast<char*>(workspace)};
    mirror::launch_signposts(a, vec, stream);
    return launch_status();
}

int mirror_tree_lookup(const int32_t* tree_tokens, const int32_t* tree_parents, int B, int N, int gamma,
                       const int32_t* path_tokens, const int32_t* k, const int32_t* tstar, int32_t* out_node,
                       uint8_t* out_hit, int32_t* out_batch, hipStream_t stream) {
    if (!tree_tokens || !tree_parents || !path_tokens || !k || !tstar || !out_node || !out_hit) return SPEC_EINVAL;
    if (B < 1 || N < 1 || gamma < 1 || gamma > mirror::kMaxGamma) return SPEC_EINVAL;
    mirror::TreeArgs a{tree_tokens, tree_parents, B, N, gamma, path_tokens, k, tstar, out_node, out_hit, out_batch};
    mirror::launch_tree_lookup(a, stream);
    return launch_status();
}

}  // extern "C"

// ------------------------------------------------------------------------------------------
// saguaro_verify_cache without a caller workspace, for callers that cannot allocate device
// memory: the library's own static device scratch stands in for it.  The scratch is one
// file-scope device array; each GPU that loads the library holds its own copy until the
// process ends.  On the host the array's name only stands for the symbol: its device address
// comes from hipGetSymbolAddress, taken once per device with that device current and kept per
// device, and only that address reaches kernels.  Calls on one GPU share its scratch, which
// keeps what the last call left there: the arrival counters and request records that must
// start at zero are cleared at the start of every call by a fill kernel on the call's stream
// (shapes may change from call to call).  Calls that overlap on one GPU race on the scratch.
// ------------------------------------------------------------------------------------------
namespace {
constexpr size_t kNoallocBytes = (size_t)SPEC_NOALLOC_SCRATCH_BYTES;
static_assert(kNoallocBytes % 256 == 0, "whole 256-byte blocks");
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoallocBytes];

__global__ __launch_bounds__(256) void zero_words_kernel(uint4* __restrict__ p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

namespace {
// The current device's address of the scratch array (nullptr if it cannot be had).
char* scratch_of_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return static_cast<char*>(g_scratch_ptr[dev]);
}

// Zeroes [begin, end) of the scratch (begin 16-byte aligned; end rounded up to 16 bytes, within
// the scratch by the size check).
void zero_range(char* base, size_t begin, size_t end, hipStream_t stream) {
    const size_t n16 = (end - begin + 15) / 16;
    if (n16 == 0) return;
    const unsigned grid = (unsigned)std::min<size_t>((n16 + 255) / 256, 1024);
    hipLaunchKernelGGL(zero_words_kernel, dim3(grid), dim3(256), 0, stream, reinterpret_cast<uint4*>(base + begin),
                       n16);
}
}  // namespace

extern "C" int saguaro_verify_cache_noalloc(const void* draft_logits, const void* target_logits, int dtype, int B,
                                            int K, int V, const spec_params* params, int F, float C,
                                            int32_t* draft_tokens, uint64_t seed, uint64_t round, uint32_t flags,
                                            int budget, double a, double r, int32_t* out_fanout_host, int32_t* out_k,
                                            int32_t* out_tstar, float* out_resid_mass, uint32_t* out_status,
                                            int32_t* out_cache, hipStream_t stream) {
    CacheArgs c{};
    const int arc = verify_cache_args(draft_logits, target_logits, dtype, B, K, V, params, F, C, draft_tokens, flags,
                                      budget, a, r, out_k, out_tstar, out_cache, &c);
    if (arc != SPEC_OK) return arc;
    const size_t need = spec_workspace_bytes(B, K, V);
    if (need > kNoallocBytes) return SPEC_EWORKSPACE;  // the shape needs more than the static scratch
    char* ws = scratch_of_current_device();
    if (!ws) return SPEC_EHIP;
    // what must start at zero: the bf16 path's arrival counters (the start of its workspace) and
    // request records; everything else is written before it is read
    const int units = B * (K + 1);
    const int nS = (V + fast::kSliceCols - 1) / fast::kSliceCols;
    const size_t gen = align_up((size_t)units * sizeof(UnitRec), 256);
    const fast::Layout L = fast::layout(B, units, nS);
    zero_range(ws, gen + L.unit_ctr, gen + L.parts, stream);
    zero_range(ws, gen + L.reqs, gen + L.reqs + (size_t)B * sizeof(fast::ReqFast), stream);
    if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    return saguaro_verify_cache(draft_logits, target_logits, dtype, B, K, V, params, F, C, draft_tokens, seed, round,
                                flags, budget, a, r, out_fanout_host, out_k, out_tstar, out_resid_mass, out_status,
                                out_cache, ws, kNoallocBytes, stream);
}
