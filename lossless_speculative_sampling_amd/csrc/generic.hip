// General-path kernels: one 1024-thread workgroup per (request b, position j) unit.
//
// Unit j < K processes target row j and draft row j (plus the downweight), decides the
// acceptance of s_j with its uniform u_j and, if s_j is rejected, samples the correction token
// from the normalised residual (q_j - p_j)+ with v_j.  Unit K samples the bonus token from q_K.
// Because the Philox counter is keyed by (b, j), every unit can draw its own candidate without
// waiting for the earlier positions; the finalize kernel then takes k = the first rejected
// position and t* = that unit's candidate, which is exactly the sequential rule of the DeepMind
// speculative-sampling page (section 3) and the SSD reading notes (section 2.2).
#include "generic.h"
#include "rowproc.h"

namespace sv {

__global__ __launch_bounds__(kRowThreads) void generic_unit_kernel(VerifyArgs a) {
    __shared__ RowShared sh;
    __shared__ RowStats stq, stp;
    const int unit = blockIdx.x;
    unit_verify(a, unit / (a.K + 1), unit % (a.K + 1), a.units + unit, sh, stq, stp);
}

// Per request: k = first rejected position (K if none), t* = that unit's candidate.
__global__ void finalize_kernel(VerifyArgs a) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= a.B) return;
    const UnitRec* u = a.units + (size_t)b * (a.K + 1);
    uint32_t any = 0, deg = 0;
    for (int j = 0; j <= a.K; ++j) {
        any |= u[j].status;
        if (j < a.K) deg |= u[j].status & kStDegenerate;
    }
    int k = 0, t = -1;
    float W = 0.0f;
    uint32_t st;
    if (any & kStBadParam) {
        st = kStBadParam;
    } else if (any & kStBadLogit) {
        st = kStBadLogit;
    } else if (any & kStBadToken) {
        st = deg | kStBadToken;
    } else {
        st = deg;
        k = a.K;
        for (int j = 0; j < a.K; ++j) {
            st |= u[j].status & kStOutside;
            if (!u[j].accept) {
                k = j;
                break;
            }
        }
        t = u[k].tcand;
        W = u[k].W;
        st |= u[k].status & kStEmptyResidual;
    }
    a.out_k[b] = k;
    a.out_t[b] = t;
    if (a.out_W) a.out_W[b] = W;
    if (a.out_status) a.out_status[b] = st;
}

// saguaro_downweight: one workgroup per draft row j < K.
__global__ __launch_bounds__(kRowThreads) void downweight_kernel(DownweightArgs a) {
    __shared__ RowShared sh;
    __shared__ RowStats st;
    const int row = blockIdx.x;
    const int b = row / a.K, j = row % a.K;
    const spec_params prm = a.params[b];
    const bool param_ok = prm.temperature >= 0.0f && !isinf(prm.temperature) && prm.top_p > 0.0f;
    const size_t stride = (size_t)a.V * (a.dtype == SPEC_BF16 ? 2 : 4);
    RowRef r{static_cast<const char*>(a.draft) + ((size_t)b * a.draft_rows + j) * stride, a.dtype, a.V};
    uint32_t status = 0;
    if (!param_ok) {
        status = kStBadParam;
    } else {
        process_row(r, prm.temperature, prm.top_k, prm.top_p, a.F, (double)a.C, a.F > 0, st, sh);
        if (st.bad) status = kStBadLogit;
        else if (st.degenerate) status = kStDegenerate;
    }
    const bool valid = status == 0 || status == kStDegenerate;
    if (threadIdx.x == 0) {
        for (int f = 0; f < a.F; ++f) a.out_ids[(size_t)row * a.F + f] = valid ? st.ids[f] : -1;
        if (a.out_Z) a.out_Z[row] = valid ? (float)st.Z : 1.0f;
        if (a.out_status) a.out_status[row] = status;
    }
    if (a.out_probs) {
        float* out = a.out_probs + (size_t)row * a.V;
        for (int i = threadIdx.x; i < a.V; i += blockDim.x)
            out[i] = valid ? (float)rs_prob_dw(st, load_logit(r.row, a.dtype, i), i) : 0.0f;
    }
}

// saguaro_cache_build: one workgroup per (request b, depth k).
__global__ __launch_bounds__(kRowThreads) void cache_build_kernel(CacheArgs a) {
    __shared__ RowShared sh;
    __shared__ RowStats st;
    __shared__ CacheShared cs;
    const int k = blockIdx.x % (a.K + 1);
    cache_row(a, blockIdx.x / (a.K + 1), k, a.fanout.f[k], a.fanout.off[k], sh, st, cs);
}

// saguaro_cache_lookup: a single workgroup loops over the requests and reduces the batch stats.
constexpr int kLookupRow = 32;  // cache rows up to this width are loaded whole

__global__ __launch_bounds__(1024) void cache_lookup_kernel(LookupArgs a) {
    __shared__ int red[32];
    int hits = 0;
    for (int b = threadIdx.x; b < a.B; b += blockDim.x) {
        int res = -1;
        if (a.mode == 0 && a.budget <= kLookupRow) {
            // a short cache row is loaded whole, alongside (k, t*): one round trip to memory
            int32_t v[kLookupRow];
            const int32_t* c = a.cache + (size_t)b * a.budget;
#pragma unroll
            for (int f = 0; f < kLookupRow; ++f) v[f] = f < a.budget ? c[f] : -1;
            const int k = a.k[b], t = a.tstar[b];
            if (k >= 0 && k <= a.K && t >= 0) {
                const int lo = a.fanout.off[k], hi = lo + a.fanout.f[k];
#pragma unroll
                for (int f = kLookupRow - 1; f >= 0; --f)
                    if (f >= lo && f < hi && v[f] == t) res = f;
            }
        } else if (a.mode == 0) {
            const int k = a.k[b], t = a.tstar[b];
            if (k >= 0 && k <= a.K && t >= 0) {
                // the depth-k list in batches of eight independent loads (no load waits for the
                // comparison of the one before); the first match is the slot
                const int32_t* c = a.cache + (size_t)b * a.budget + a.fanout.off[k];
                const int n = a.fanout.f[k];
                for (int f0 = 0; f0 < n && res < 0; f0 += 8) {
                    int32_t v[8];
#pragma unroll
                    for (int d = 0; d < 8; ++d) v[d] = f0 + d < n ? c[f0 + d] : -1;
#pragma unroll
                    for (int d = 7; d >= 0; --d)
                        if (v[d] == t) res = a.fanout.off[k] + f0 + d;
                }
            }
        } else {
            const int kappa = a.kappa, gamma = a.gamma;
            const int32_t* br = a.cache + (size_t)b * kappa * gamma;
            const int k = a.k[(size_t)b * kappa], t = a.tstar[(size_t)b * kappa];
            if (k == gamma) {
                res = -2;
            } else if (k >= 0 && k < gamma && t >= 0) {
                for (int jb = 0; jb < kappa && res < 0; ++jb) {
                    bool ok = br[(size_t)jb * gamma + k] == t;
                    for (int d = 0; d < k && ok; ++d) ok = br[(size_t)jb * gamma + d] == br[d];
                    if (ok) res = jb;
                }
            }
        }
        a.out_slot[b] = res;
        a.out_hit[b] = res >= 0 ? 1 : 0;
        hits += res >= 0 ? 1 : 0;
    }
    const int total = block_sum<int>(hits, red);
    if (threadIdx.x == 0 && a.out_batch) {
        a.out_batch[0] = total;
        a.out_batch[1] = total == a.B ? 1 : 0;
    }
}

// The batch-aware fallback on a cache miss (SSD reading notes, section 7.1): any miss makes the
// whole batch wait, so from the critical batch size b* on the missed requests take the
// random-token backup; the requests that hit keep their cached speculation.
__global__ void backup_plan_kernel(BackupArgs a) {
    const int sw = (a.batch[1] == 0 && a.B >= a.b_star) ? 1 : 0;
    for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < a.B; b += gridDim.x * blockDim.x)
        a.out_use_backup[b] = (sw && !a.hit[b]) ? 1 : 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.out_switch = sw;
}

}  // namespace sv
