// Mirror-SD signposts and draft-tree reuse on gfx950 (Mirror Speculative Decoding reading notes,
// sections 3.1-3.3).
//
// Signposts.  At the early-exit layer the LM head gives a distribution p~ over the vocabulary;
// the draft receives its kappa most likely tokens with log p~.  Here p~ is the softmax of the
// given logit row (temperature 1), tokens are ranked by (logit descending, id ascending) and
// log p~(v) = z_v - m - log S with m the row maximum and S = sum exp(z - m).
//
// Per wave (2048 columns, 32 contiguous per lane):
//   1. each lane's maximum and its first column; the wave maximum m_w and
//      S_w = sum exp(z - m_w) (fp32 terms, fp64 across lanes);
//   2. the kappa-th largest lane maximum tau (lane maxima made unique by their column): every
//      element of the wave's top kappa is >= tau and sits in a lane whose maximum is >= tau, so
//      only those (at most kappa) lanes are staged in LDS and filtered against tau;
//   3. the few candidates are ranked exactly and the wave publishes its sorted list.
// The last workgroup of the row merges: m = max m_w, S = sum S_w exp(m_w - m) in fp64, and a
// kappa-round tournament over the lists' heads.
#include "mirror.h"

namespace sv {
namespace mirror {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Loads, reads and writes of one wave's LDS region become visible to its other lanes in program
// order; this keeps the compiler from moving accesses across the hand-over.
__device__ __forceinline__ void wave_lds_handover() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ int lane_rank(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Total order of the logits inside a wave, unique per element: bf16 rows use the 16-bit order
// key and the wave-local column; fp32 rows the 32-bit key and the column.  Larger = earlier.
template <int DT>
struct WaveOrder;
template <>
struct WaveOrder<SPEC_BF16> {
    using T = uint32_t;
    __device__ static T of(float z, int local, int) {
        return (order_key(z) & 0xFFFF0000u) | (uint32_t)(0xFFFF - local);
    }
};
template <>
struct WaveOrder<SPEC_FP32> {
    using T = uint64_t;
    __device__ static T of(float z, int, int col) {
        return ((uint64_t)order_key(z) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)col);
    }
};

// The order used across waves and in the published lists: 32-bit key, then the column.
__device__ __forceinline__ uint64_t row_order(float z, int col) {
    return ((uint64_t)order_key(z) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)col);
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// The 32 columns of a lane, widened to fp32; columns at or past V read as -inf.
template <int DT, bool VEC>
__device__ __forceinline__ void load_lane(const void* row, int c0, int nvalid, float (&v)[kPer]) {
    if (DT == SPEC_BF16) {
        const uint16_t* p = static_cast<const uint16_t*>(row) + c0;
        if (VEC && nvalid == kPer) {
#pragma unroll
            for (int q = 0; q < kPer / 8; ++q) {
                const u32x4 w = *reinterpret_cast<const u32x4*>(p + 8 * q);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[8 * q + 2 * e] = __uint_as_float(w[e] << 16);
                    v[8 * q + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < kPer; ++i) v[i] = i < nvalid ? __uint_as_float((uint32_t)p[i] << 16) : -INFINITY;
        }
    } else {
        const float* p = static_cast<const float*>(row) + c0;
        if (VEC && nvalid == kPer) {
#pragma unroll
            for (int q = 0; q < kPer / 4; ++q) {
                const u32x4 w = *reinterpret_cast<const u32x4*>(p + 4 * q);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * q + e] = __uint_as_float(w[e]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kPer; ++i) v[i] = i < nvalid ? p[i] : -INFINITY;
        }
    }
}

// exp(x - y) for x <= y in fp32 (the factors that move a sum of exponentials from one maximum
// to a larger one; relative error ~1e-7).
__device__ __forceinline__ float exp_diff(float x, float y) {
    return __builtin_amdgcn_exp2f((x - y) * 1.4426950408889634f);
}

// LDS of the merge: per list its maximum, count, sum and entries; the top-head lists; the
// candidate slots.
struct MergeView {
    float* m;
    int* cnt;
    int* top;
    double* S;
    uint64_t* cand;
    uint64_t* heads;
    uint64_t* ent;
};
__device__ __forceinline__ MergeView merge_view(char* lds, int L, int kappa) {
    MergeView v;
    v.m = reinterpret_cast<float*>(lds);
    v.cnt = reinterpret_cast<int*>(v.m + L);
    v.top = v.cnt + L;
    v.S = reinterpret_cast<double*>(lds + align_to((size_t)L * 8 + (size_t)kappa * 4, 8));
    v.cand = reinterpret_cast<uint64_t*>(v.S + L);
    v.heads = v.cand + (size_t)kappa * kappa;
    v.ent = v.heads + L;
    return v;
}
struct MergeRed {
    float m[kWaves];
    double S[kWaves];
    int bad[kWaves];
    int n[kWaves];   // entries
    int ne[kWaves];  // non-empty lists
    int ncand;       // candidates of the final ranking
};

__device__ __forceinline__ char* list_rec(const SignpostArgs& a, int b, int l) {
    return a.ws + a.plan.ctr_bytes + ((size_t)b * a.plan.L + l) * a.plan.rec_stride;
}

// One wave: its list of the kappa largest columns, with m_w and S_w.
template <int DT, bool VEC>
__device__ void wave_list(const SignpostArgs& a, int b, int s, char* wlds) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int kappa = a.kappa;
    const int base = s * kSliceSpan + wave * kWaveSpan;
    const int c0 = base + lane * kPer;
    const int nvalid = min(max(a.V - c0, 0), kPer);
    const size_t esz = DT == SPEC_BF16 ? 2 : 4;
    const void* row = static_cast<const char*>(a.logits) + (size_t)b * a.V * esz;

    float v[kPer];
    if (nvalid > 0) load_lane<DT, VEC>(row, c0, nvalid, v);
    else {
#pragma unroll
        for (int i = 0; i < kPer; ++i) v[i] = -INFINITY;
    }

    // 1. lane maximum, wave maximum, sum of exponentials
    float lm = v[0];
#pragma unroll
    for (int i = 1; i < kPer; ++i) lm = fmaxf(lm, v[i]);
    const bool lane_valid = nvalid > 0;
    const float mw = wave_max(lane_valid ? lm : -INFINITY);
    double Sw = 0.0;
    if (mw != -INFINITY) {  // (a NaN maximum still sums to NaN and flags the row)
        // exp(z - m_w) = 2^((z - m_w) log2 e); the difference first, so the error of each term
        // scales with its own exponent, not with m_w
        const float kLog2e = 1.4426950408889634f;
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int i = 0; i < kPer; i += 2) {
            s0 += __builtin_amdgcn_exp2f((v[i] - mw) * kLog2e);
            s1 += __builtin_amdgcn_exp2f((v[i + 1] - mw) * kLog2e);
        }
        Sw = wave_sum((double)s0 + (double)s1);
    }

    // 2. tau: the kappa-th largest lane maximum, counting ties (bitwise search on the order
    // key with ballots).  Every element of the wave's top kappa is >= tau; the elements > tau
    // sit in the (fewer than kappa) lanes whose maximum is > tau, and the elements == tau
    // needed are the first ones in column order, found in the first kappa lanes whose maximum
    // is tau.  Lanes are column-contiguous, so lane order is column order.
    const uint32_t lk = lane_valid ? order_key(lm) : 0u;  // valid keys are > 0 (NaN drops out)
    const bool all_cand = __popcll(__ballot(lk != 0u)) < kappa;
    uint32_t tau = 0;
    if (!all_cand) {
        const int lo = DT == SPEC_BF16 ? 16 : 0;  // bf16 keys carry 16 bits
        for (int bit = 31; bit >= lo; --bit) {
            const uint32_t c = tau | (1u << bit);
            if (__popcll(__ballot(lk >= c)) >= kappa) tau = c;
        }
        if (DT == SPEC_BF16 && !(tau & 0x80000000u)) tau |= 0xFFFFu;  // a negative bf16 value's key
    }
    const float tf = key_to_float(tau);
    const bool gt_lane = lane_valid && (all_cand || lm > tf);
    const bool eq_lane = !all_cand && lane_valid && lm == tf;
    const bool staged = gt_lane || (eq_lane && lane_rank(__ballot(eq_lane)) < kappa);

    float* stage = reinterpret_cast<float*>(wlds);                        // [2 kappa][kPer]
    int* slot_lane = reinterpret_cast<int*>(stage + (size_t)2 * kappa * kPer);  // [2 kappa]
    uint64_t* gl = reinterpret_cast<uint64_t*>(wlds + wave_stage_bytes(kappa));  // [kPer kappa]
    uint64_t* el = gl + (size_t)kPer * kappa;                             // [kappa]
    const uint64_t sm = __ballot(staged);
    const int nl = __popcll(sm);
    if (staged) {
        const int slot = lane_rank(sm);
#pragma unroll
        for (int i = 0; i < kPer; ++i) stage[slot * kPer + i] = v[i];
        slot_lane[slot] = lane;
    }
    wave_lds_handover();

    // classify the staged columns in column order: > tau into gl, the first kappa == tau into el
    int ngt = 0, neq = 0;
    const int total = nl * kPer;
    for (int e0 = 0; e0 < total; e0 += kWave) {
        const int e = e0 + lane;
        bool gt = false, eq = false;
        float z = 0.0f;
        int col = 0;
        if (e < total) {
            col = base + slot_lane[e / kPer] * kPer + (e % kPer);
            z = stage[e];
            if (col < a.V) {
                gt = all_cand || z > tf;
                eq = !all_cand && z == tf;
            }
        }
        const uint64_t gm = __ballot(gt), em = __ballot(eq);
        if ((gm | em) != 0ull) {
            const uint64_t key = row_order(z, col);
            if (gt) gl[ngt + lane_rank(gm)] = key;
            if (eq) {
                const int r = neq + lane_rank(em);
                if (r < kappa) el[r] = key;
            }
            ngt += __popcll(gm);
            neq += __popcll(em);
        }
    }
    wave_lds_handover();

    // 3. the list: the elements > tau ranked exactly, then those == tau in column order
    const int keep_gt = min(kappa, ngt);
    const int keep_eq = min(kappa - keep_gt, min(neq, kappa));
    char* rec = list_rec(a, b, s * kWaves + wave);
    uint64_t* ent = reinterpret_cast<uint64_t*>(rec + sizeof(ListHead));
    if (ngt <= kWave) {
        const uint64_t mine = lane < ngt ? gl[lane] : 0ull;
        int rank = 0;
        for (int i = 0; i < ngt; ++i) rank += gl[i] > mine ? 1 : 0;
        if (lane < ngt && rank < keep_gt) ent[rank] = mine;
    } else {
        for (int r = 0; r < keep_gt; ++r) {
            uint64_t best = 0;
            int bi = -1;
            for (int i = lane; i < ngt; i += kWave) {
                const uint64_t x = gl[i];
                if (x > best) {
                    best = x;
                    bi = i;
                }
            }
            const uint64_t W = wave_max(best);
            if (bi >= 0 && best == W) gl[bi] = 0ull;
            if (lane == 0) ent[r] = W;
            wave_lds_handover();
        }
    }
    if (lane < keep_eq) ent[keep_gt + lane] = el[lane];
    if (lane == 0) {
        ListHead h;
        h.m = mw;
        h.count = keep_gt + keep_eq;
        h.S = Sw;
        *reinterpret_cast<ListHead*>(rec) = h;
    }
}

// The last workgroup of a row: merge its lists into the row's signposts.  Only the lists whose
// first entry ranks among the kappa largest first entries can hold a top-kappa element (kappa
// larger heads would precede any other), so their entries (at most kappa^2) are ranked exactly.
__device__ void merge_row(const SignpostArgs& a, int b, char* lds, MergeRed* red) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int L = a.plan.L, kappa = a.kappa;
    MergeView mv = merge_view(lds, L, kappa);

    // every list's header and entries, one round trip to L2
    for (int l = threadIdx.x; l < L; l += kThreads) {
        const char* rec = list_rec(a, b, l);
        mv.m[l] = ldnt(reinterpret_cast<const float*>(rec));
        mv.cnt[l] = ldnt(reinterpret_cast<const int32_t*>(rec + 4));
        mv.S[l] = ldnt(reinterpret_cast<const double*>(rec + 8));
    }
    for (int idx = threadIdx.x; idx < L * kappa; idx += kThreads) {
        const int l = idx / kappa, i = idx - l * kappa;
        mv.ent[idx] = ldnt(reinterpret_cast<const uint64_t*>(list_rec(a, b, l) + sizeof(ListHead)) + i);
    }
    __syncthreads();

    // row maximum, sum of exponentials, bad flag, element count: per wave, then across waves
    float mloc = -INFINITY;
    int bad = 0, n = 0, ne = 0;
    for (int l = threadIdx.x; l < L; l += kThreads) {
        const int c = mv.cnt[l];
        if (c > 0 && mv.m[l] > mloc) mloc = mv.m[l];
        if (mv.S[l] != mv.S[l]) bad = 1;
        n += c;
        ne += c > 0 ? 1 : 0;
        mv.heads[l] = c > 0 ? mv.ent[(size_t)l * kappa] : 0ull;
    }
    const float mwv = wave_max(mloc);
    double sp = 0.0;
    if (mwv != -INFINITY)
        for (int l = threadIdx.x; l < L; l += kThreads)
            if (mv.m[l] > -INFINITY) sp += mv.S[l] * (double)exp_diff(mv.m[l], mwv);
    sp = wave_sum(sp);
    bad = wave_max(bad);
    n = wave_sum(n);
    ne = wave_sum(ne);
    if (lane == 0) {
        red->m[wave] = mwv;
        red->S[wave] = sp;
        red->bad[wave] = bad;
        red->n[wave] = n;
        red->ne[wave] = ne;
    }
    __syncthreads();
    // heads: rank of each list's first entry among all lists' first entries (L is a multiple
    // of 4, the loads are independent)
    for (int l = threadIdx.x; l < L; l += kThreads) {
        const uint64_t h = mv.heads[l];
        if (h == 0ull) continue;
        int r = 0;
#pragma unroll 4
        for (int j = 0; j < L; j += 4) {
            r += mv.heads[j] > h ? 1 : 0;
            r += mv.heads[j + 1] > h ? 1 : 0;
            r += mv.heads[j + 2] > h ? 1 : 0;
            r += mv.heads[j + 3] > h ? 1 : 0;
        }
        if (r < kappa) mv.top[r] = l;
    }
    float m = -INFINITY;
    int nall = 0, nne = 0;
    bad = 0;
    for (int w = 0; w < kWaves; ++w) {
        m = fmaxf(m, red->m[w]);
        bad |= red->bad[w];
        nall += red->n[w];
        nne += red->ne[w];
    }
    double S = 0.0;
    for (int w = 0; w < kWaves; ++w)
        if (red->m[w] != -INFINITY) S += red->S[w] * (double)exp_diff(red->m[w], m);
    bad |= (m == -INFINITY || m == INFINITY) ? 1 : 0;
    const double logS = log(S);
    const int nout = min(kappa, nall);   // entries the row has (fewer than kappa only if V < kappa)

    // candidates: every entry of the top-head lists (the non-empty lists with a head rank below
    // kappa), in slots rank * kappa + i
    // (entries below the kappa-th largest head cannot make the top kappa: the kappa heads
    // precede them), compacted through an LDS counter
    const int nlists = min(kappa, nne);
    if (threadIdx.x == 0) red->ncand = 0;
    __syncthreads();  // the top-head lists, the counter
    const uint64_t floor_h = nlists == kappa ? mv.heads[mv.top[kappa - 1]] : 0ull;
    for (int j = threadIdx.x; j < nlists * kappa; j += kThreads) {
        const int r = j / kappa, i = j - r * kappa;
        const int l = mv.top[r];
        const uint64_t e = i < mv.cnt[l] ? mv.ent[(size_t)l * kappa + i] : 0ull;
        if (e != 0ull && e >= floor_h) mv.cand[atomicAdd(&red->ncand, 1)] = e;
    }
    __syncthreads();
    const int ncand = red->ncand;
    const size_t o0 = (size_t)b * kappa;
    if (bad) {
        if (threadIdx.x < kappa) {
            a.out_ids[o0 + threadIdx.x] = -1;
            a.out_logp[o0 + threadIdx.x] = __uint_as_float(0x7FC00000u);
            if (a.out_logp_bf16) a.out_logp_bf16[o0 + threadIdx.x] = 0x7FC0;
        }
    } else {
        for (int j = threadIdx.x; j < ncand; j += kThreads) {
            const uint64_t c = mv.cand[j];
            int r = 0;
#pragma unroll 8
            for (int i = 0; i < ncand; ++i) r += mv.cand[i] > c ? 1 : 0;
            if (r < kappa) {
                const float z = key_to_float((uint32_t)(c >> 32));
                const float lp = (float)((double)z - (double)m - logS);
                a.out_ids[o0 + r] = (int32_t)(0xFFFFFFFFu - (uint32_t)c);
                a.out_logp[o0 + r] = lp;
                if (a.out_logp_bf16) a.out_logp_bf16[o0 + r] = bf16_rne(lp);
            }
        }
        for (int p = nout + (int)threadIdx.x; p < kappa; p += kThreads) {
            a.out_ids[o0 + p] = -1;
            a.out_logp[o0 + p] = -INFINITY;
            if (a.out_logp_bf16) a.out_logp_bf16[o0 + p] = 0xFF80;
        }
    }
    if (threadIdx.x == 0 && a.out_status) a.out_status[b] = bad ? kStBadLogit : 0u;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void signpost_kernel(SignpostArgs a) {
    extern __shared__ __align__(16) char lds[];
    __shared__ MergeRed red;
    __shared__ int last;
    const int nS = a.plan.nS;
    const int x = blockIdx.x % kXcd, l = blockIdx.x / kXcd;
    const int b = (l / nS) * kXcd + x, s = l % nS;
    if (b >= a.B) return;

    wave_list<DT, VEC>(a, b, s, lds + (size_t)(threadIdx.x / kWave) * a.plan.wave_lds);

    unsigned* ctr = reinterpret_cast<unsigned*>(a.ws + (size_t)b * 128);
    drain_stores();
    __syncthreads();
    if (threadIdx.x == 0) last = l2_fetch_add(ctr, 1u) == (unsigned)(nS - 1) ? 1 : 0;
    __syncthreads();
    if (!last) return;
    if (threadIdx.x == 0) *ctr = 0u;  // ready for the next call
    merge_row(a, b, lds, &red);
}

// ------------------------------------------------------------------------------------------
// Reuse of the committed prefix (accepted tokens, t*) against a draft tree whose nodes list
// their parents first; the reuse node is the lowest node whose root path is that prefix.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kTreeThreads) void tree_lookup_kernel(TreeArgs a) {
    extern __shared__ __align__(16) char lds[];
    __shared__ int red[kTreeThreads / kWave];
    const int b = blockIdx.x;
    const int N = a.N, gamma = a.gamma;
    const int k = a.k[b], t = a.tstar[b];
    const bool staged = N <= kTreeLdsNodes;
    int32_t* want = reinterpret_cast<int32_t*>(lds);
    int32_t* tok_l = want + kMaxGamma + 1;
    int32_t* par_l = tok_l + (staged ? N : 0);
    const int32_t* tok_g = a.tokens + (size_t)b * N;
    const int32_t* par_g = a.parents + (size_t)b * N;
    const bool active = k >= 0 && k < gamma && t >= 0;
    if (active)
        for (int d = threadIdx.x; d <= k; d += kTreeThreads) want[d] = d < k ? a.path[(size_t)b * gamma + d] : t;
    if (staged)
        for (int n = threadIdx.x; n < N; n += kTreeThreads) {
            tok_l[n] = tok_g[n];
            par_l[n] = par_g[n];
        }
    __syncthreads();
    const int32_t* tok = staged ? tok_l : tok_g;
    const int32_t* par = staged ? par_l : par_g;
    int best = 0x7FFFFFFF;
    if (active) {
        for (int n = threadIdx.x; n < N; n += kTreeThreads) {
            // node n must sit at depth k + 1: walk up, matching want[k], want[k-1], ..., want[0]
            int cur = n, d = k;
            bool ok = false;
            while (true) {
                const int tk = tok[cur], pa = par[cur];
                if (tk < 0 || pa < -1 || pa >= cur || tk != want[d]) break;
                if (pa == -1) {
                    ok = d == 0;
                    break;
                }
                if (d == 0) break;  // the chain is longer than the prefix
                cur = pa;
                --d;
            }
            if (ok && n < best) best = n;
        }
    }
    best = block_min<int>(best, red);
    if (threadIdx.x == 0) {
        const int node = k == gamma ? -2 : (best == 0x7FFFFFFF ? -1 : best);
        a.out_node[b] = node;
        a.out_hit[b] = node >= 0 ? 1 : 0;
    }
}

__global__ __launch_bounds__(1024) void tree_batch_kernel(TreeArgs a) {
    __shared__ int red[1024 / kWave];
    int hits = 0;
    for (int b = threadIdx.x; b < a.B; b += blockDim.x) hits += a.out_hit[b] ? 1 : 0;
    const int total = block_sum<int>(hits, red);
    if (threadIdx.x == 0) {
        a.out_batch[0] = total;
        a.out_batch[1] = total == a.B ? 1 : 0;
    }
}

}  // namespace

void launch_signposts(const SignpostArgs& a, int vec, hipStream_t stream) {
    const dim3 grid((unsigned)(kXcd * ((a.B + kXcd - 1) / kXcd) * a.plan.nS));
    const size_t lds = a.plan.lds_bytes;
    if (a.dtype == SPEC_BF16) {
        if (vec) hipLaunchKernelGGL((signpost_kernel<SPEC_BF16, true>), grid, dim3(kThreads), lds, stream, a);
        else hipLaunchKernelGGL((signpost_kernel<SPEC_BF16, false>), grid, dim3(kThreads), lds, stream, a);
    } else {
        if (vec) hipLaunchKernelGGL((signpost_kernel<SPEC_FP32, true>), grid, dim3(kThreads), lds, stream, a);
        else hipLaunchKernelGGL((signpost_kernel<SPEC_FP32, false>), grid, dim3(kThreads), lds, stream, a);
    }
}

void launch_tree_lookup(const TreeArgs& a, hipStream_t stream) {
    const size_t lds = (size_t)(kMaxGamma + 1) * 4 + (a.N <= kTreeLdsNodes ? (size_t)a.N * 8 : 0);
    hipLaunchKernelGGL(tree_lookup_kernel, dim3((unsigned)a.B), dim3(kTreeThreads), lds, stream, a);
    if (a.out_batch) hipLaunchKernelGGL(tree_batch_kernel, dim3(1), dim3(1024), 0, stream, a);
}

}  // namespace mirror
}  // namespace sv
