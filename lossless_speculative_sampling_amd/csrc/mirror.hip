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

__device__ __forceinline__ char* list_rec(const SignpostArgs& a, int b, int l) {
    return a.ws + a.plan.ctr_bytes + ((size_t)b * a.plan.L + l) * a.plan.rec_stride;
}

// One wave: its list of the kappa largest columns, with m_w and S_w.
template <int DT, bool VEC>
__device__ void wave_list(const SignpostArgs& a, int b, int s, char* wlds) {
    using WO = WaveOrder<DT>;
    using OT = typename WO::T;
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

    // 1. lane maximum (first column on ties), wave maximum, sum of exponentials
    float lm = v[0];
    int li = 0;
#pragma unroll
    for (int i = 1; i < kPer; ++i)
        if (v[i] > lm) {
            lm = v[i];
            li = i;
        }
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

    // 2. tau: the kappa-th largest lane maximum
    const OT lc = lane_valid ? WO::of(lm, lane * kPer + li, c0 + li) : OT(0);
    OT cur = lc, tau = 0;
    int taken = 0;
    for (int r = 0; r < kappa; ++r) {
        const OT W = wave_max(cur);
        if (W == OT(0)) break;
        tau = W;
        ++taken;
        if (cur == W) cur = OT(0);
    }
    const bool all_cand = taken < kappa;  // fewer valid lanes than kappa: every column competes
    const bool cand_lane = lane_valid && (all_cand || lc >= tau);

    // stage the candidate lanes (at most kappa) in LDS
    float* stage = reinterpret_cast<float*>(wlds);
    int* slot_lane = reinterpret_cast<int*>(stage + (size_t)kappa * kPer);
    uint64_t* cand = reinterpret_cast<uint64_t*>(wlds + align_to((size_t)kappa * kPer * 4 + (size_t)kappa * 4, 8));
    const uint64_t cm = __ballot(cand_lane);
    const int nl = __popcll(cm);
    if (cand_lane) {
        const int slot = lane_rank(cm);
#pragma unroll
        for (int i = 0; i < kPer; ++i) stage[slot * kPer + i] = v[i];
        slot_lane[slot] = lane;
    }
    wave_lds_handover();

    // candidates: staged columns whose order is >= tau
    int nc = 0;
    const int total = nl * kPer;
    for (int e0 = 0; e0 < total; e0 += kWave) {
        const int e = e0 + lane;
        bool take = false;
        uint64_t key = 0;
        if (e < total) {
            const int local = slot_lane[e / kPer] * kPer + (e % kPer);
            const int col = base + local;
            const float z = stage[e];
            if (col < a.V) {
                take = all_cand || WO::of(z, local, col) >= tau;
                key = row_order(z, col);
            }
        }
        const uint64_t tm = __ballot(take);
        if (take) cand[nc + lane_rank(tm)] = key;
        nc += __popcll(tm);
    }
    wave_lds_handover();

    // 3. exact ranking of the candidates, published in descending order
    const int keep = min(kappa, nc);
    char* rec = list_rec(a, b, s * kWaves + wave);
    uint64_t* ent = reinterpret_cast<uint64_t*>(rec + sizeof(ListHead));
    if (nc <= kWave) {
        const uint64_t mine = lane < nc ? cand[lane] : 0ull;
        int rank = 0;
        for (int i = 0; i < nc; ++i) rank += cand[i] > mine ? 1 : 0;
        if (lane < nc && rank < keep) ent[rank] = mine;
    } else {
        for (int r = 0; r < keep; ++r) {
            uint64_t best = 0;
            int bi = -1;
            for (int i = lane; i < nc; i += kWave) {
                const uint64_t x = cand[i];
                if (x > best) {
                    best = x;
                    bi = i;
                }
            }
            const uint64_t W = wave_max(best);
            if (bi >= 0 && best == W) cand[bi] = 0ull;
            if (lane == 0) ent[r] = W;
            wave_lds_handover();
        }
    }
    if (lane == 0) {
        ListHead h;
        h.m = mw;
        h.count = keep;
        h.S = Sw;
        *reinterpret_cast<ListHead*>(rec) = h;
    }
}

// The last workgroup of a row: merge its lists into the row's signposts.
__device__ void merge_row(const SignpostArgs& a, int b, char* lds, double* red_d, float* red_f, int* red_i) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int L = a.plan.L, kappa = a.kappa;
    int* cnt = reinterpret_cast<int*>(lds);
    float* mlist = reinterpret_cast<float*>(cnt + L);
    int* cursor = reinterpret_cast<int*>(mlist + L);
    double* Slist = reinterpret_cast<double*>(lds + align_to((size_t)L * 12, 8));
    uint64_t* res = reinterpret_cast<uint64_t*>(Slist + L);
    uint64_t* staged = reinterpret_cast<uint64_t*>(lds + align_to(a.plan.merge_arrays, 8));

    float mloc = -INFINITY;
    int bad = 0;
    for (int l = threadIdx.x; l < L; l += kThreads) {
        const char* rec = list_rec(a, b, l);
        const float ml = ldnt(reinterpret_cast<const float*>(rec));
        const int c = ldnt(reinterpret_cast<const int32_t*>(rec + 4));
        const double Sl = ldnt(reinterpret_cast<const double*>(rec + 8));
        cnt[l] = c;
        mlist[l] = ml;
        Slist[l] = Sl;
        cursor[l] = 0;
        if (c > 0 && ml > mloc) mloc = ml;
        if (Sl != Sl) bad = 1;
    }
    const float m = block_max<float>(mloc, red_f);
    double sp = 0.0;
    for (int l = threadIdx.x; l < L; l += kThreads)
        if (mlist[l] > -INFINITY) sp += Slist[l] * exp((double)mlist[l] - (double)m);
    const double S = block_sum<double>(sp, red_d);
    bad = block_max<int>(bad | (m == -INFINITY || m == INFINITY ? 1 : 0), red_i);
    const double logS = log(S);

    const int in_lds = a.plan.merge_in_lds;
    if (in_lds) {
        for (int idx = threadIdx.x; idx < L * kappa; idx += kThreads) {
            const int l = idx / kappa, i = idx - l * kappa;
            staged[idx] = i < cnt[l]
                              ? ldnt(reinterpret_cast<const uint64_t*>(list_rec(a, b, l) + sizeof(ListHead)) + i)
                              : 0ull;
        }
    }
    __syncthreads();
    if (wave != 0) return;

    auto entry = [&](int l, int i) -> uint64_t {
        if (i >= cnt[l]) return 0ull;
        return in_lds ? staged[(size_t)l * kappa + i]
                      : ldnt(reinterpret_cast<const uint64_t*>(list_rec(a, b, l) + sizeof(ListHead)) + i);
    };
    // tournament: each lane holds the lists l = lane (mod 64); the winner advances its cursor
    uint64_t best = 0;
    int bl = -1;
    for (int l = lane; l < L; l += kWave) {
        const uint64_t x = entry(l, 0);
        if (x > best) {
            best = x;
            bl = l;
        }
    }
    int nres = 0;
    for (; nres < kappa; ++nres) {
        const uint64_t W = wave_max(best);
        if (W == 0ull) break;
        if (lane == 0) res[nres] = W;
        if (bl >= 0 && best == W) {
            cursor[bl] += 1;
            best = 0;
            bl = -1;
            for (int l = lane; l < L; l += kWave) {
                const uint64_t x = entry(l, cursor[l]);
                if (x > best) {
                    best = x;
                    bl = l;
                }
            }
        }
    }
    wave_lds_handover();
    if (lane < kappa) {
        const size_t o = (size_t)b * kappa + lane;
        int32_t id = -1;
        float lp;
        if (bad) {
            lp = __uint_as_float(0x7FC00000u);
        } else if (lane < nres) {
            const uint64_t c = res[lane];
            id = (int32_t)(0xFFFFFFFFu - (uint32_t)c);
            const float z = key_to_float((uint32_t)(c >> 32));
            lp = (float)((double)z - (double)m - logS);
        } else {
            lp = -INFINITY;
        }
        a.out_ids[o] = id;
        a.out_logp[o] = lp;
        if (a.out_logp_bf16) a.out_logp_bf16[o] = bf16_rne(lp);
    }
    if (lane == 0 && a.out_status) a.out_status[b] = bad ? kStBadLogit : 0u;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void signpost_kernel(SignpostArgs a) {
    extern __shared__ __align__(16) char lds[];
    __shared__ double red_d[kWaves];
    __shared__ float red_f[kWaves];
    __shared__ int red_i[kWaves];
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
    merge_row(a, b, lds, red_d, red_f, red_i);
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
