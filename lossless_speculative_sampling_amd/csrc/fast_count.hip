// Count kernel of the bf16 verification path: every slice of every (request, position) unit
// loads its token columns of the target row (and the draft row), counts every distinct bf16
// value in LDS and publishes a compact summary for the resolve kernel.
#include "fast_common.h"

namespace sv {
namespace fast {

// ------------------------------------------------------------------------------------------
// Count kernel: every slice of every unit loads its columns, counts them and publishes its
// summaries (no waiting on other workgroups).
// ------------------------------------------------------------------------------------------
struct CountSmem {
    double segm[kSegs];
    uint32_t segc[2][kSegs];
    uint32_t hraw[2][kHistRow];
    __device__ __forceinline__ uint32_t* hist(int r) { return &hraw[r][kHistLead]; }
    uint32_t sp_key[2][kSpecial];
    int32_t sp_id[2][kSpecial];
    uint32_t n_sp[2];
    uint32_t top_key[2][kTop];
    int32_t top_id[2][kTop];
    uint32_t n_top[2];
    uint32_t cnt_s[2];
    uint32_t flags[2];
    uint32_t neginf[2];
    int32_t scan[kWaves + 1];
    double redd[kWaves];
    int32_t redi[kWaves];
    uint32_t s_bits[2];
    uint32_t tau;
    int need;
    int ties;      // elements of the slice at key tau
    uint32_t maxkey;
};

// Per-segment element counts of both rows into sm.segc: a thread adds 8 bins, eight lanes a
// group of 64; the last wave also sorts each row's specials into their four segments.
// (Callers synchronise.)
__device__ __forceinline__ void seg_counts(CountSmem& sm, int rows) {
    constexpr int kPerRow = kBins / 8;  // 360 threads per row
    for (int i = threadIdx.x; i < rows * kPerRow; i += blockDim.x) {  // 8-aligned lane groups
        const int r = i / kPerRow, t = i % kPerRow;
        const u32x4* h4 = reinterpret_cast<const u32x4*>(sm.hist(r) + t * 8);
        const u32x4 a = h4[0], b = h4[1];
        const uint32_t c = group8_sum(a[0] + a[1] + a[2] + a[3] + b[0] + b[1] + b[2] + b[3]);
        if ((t & 7) == 0) sm.segc[r][seg_of_group(t / 8)] = c;
    }
    const int lane = threadIdx.x & (kWave - 1);
    if (threadIdx.x / kWave == kWaves - 1) {
        for (int r = 0; r < rows; ++r) {
            const int nsp = min((int)sm.n_sp[r], kSpecial);
            const int sg = lane < nsp ? special_seg(sm.sp_key[r][lane]) : -1;
            const int sps[4] = {kSegHugePos, kSegTinyPos, kSegTinyNeg, kSegHugeNeg};
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const uint32_t cx = (uint32_t)__popcll(__ballot(sg == sps[x]));
                if (lane == 0) sm.segc[r][sps[x]] = cx;
            }
        }
    }
}

// Wave 0: the key of the L-th element (token order) of row r in this slice, and how many
// elements at that key are taken, into sm.tau / sm.need; (0, 0) when the slice holds fewer
// than L finite elements.  Scans the segment counts, then the 64 bins of the crossing group,
// or the specials of the crossing segment.
__device__ __forceinline__ void local_threshold(CountSmem& sm, int r, int L) {
    const int lane = threadIdx.x & (kWave - 1);
    if (lane == 0) {
        sm.tau = 0u;
        sm.need = 0;
        sm.ties = 0;
    }
    const int c = lane < kSegs ? (int)sm.segc[r][lane] : 0;
    int cex;
    const int cin = wave_scan(c, &cex);
    const uint64_t hit = __ballot(lane < kSegs && cin >= L);
    if (hit == 0) return;
    const int sg = first_lane(hit);
    const int rem = L - wave_bcast(cex, sg);
    const int g = group_of_seg(sg);
    if (g >= 0) {
        const int bin = bin_of_sel(g, lane);  // lane order = descending key
        const int n = (int)sm.hist(r)[bin];
        int nex;
        const int nin = wave_scan(n, &nex);
        const int i = first_lane(__ballot(nin >= rem));
        if (lane == i) {
            sm.tau = bin_key(bin);
            sm.need = rem - nex;
            sm.ties = n;
        }
    } else {
        const int nsp = min((int)sm.n_sp[r], kSpecial);
        uint32_t k = 0;
        bool mine = false;
        if (lane < nsp) {
            k = sm.sp_key[r][lane];
            mine = special_seg(k) == sg;
        }
        int gt = 0, eq = 0;
        for (int i = 0; i < nsp; ++i) {
            const uint32_t k2 = sm.sp_key[r][i];
            if (special_seg(k2) != sg) continue;
            gt += k2 > k ? 1 : 0;
            eq += k2 == k ? 1 : 0;
        }
        if (mine && gt < rem && gt + eq >= rem) {
            sm.tau = k;
            sm.need = rem - gt;
            sm.ties = eq;
        }
    }
}

// The first L elements (token order: key desc, id asc) of row r in this slice, sorted, into
// sm.top_key[r] / sm.top_id[r]; sm.n_top[r] gets their number.
__device__ __forceinline__ void local_top(CountSmem& sm, int r, int L, int c0, int V, const u32x4 (&v)[kLoads]) {
    if (threadIdx.x < kWave) local_threshold(sm, r, L);
    if (threadIdx.x == 0) sm.n_top[r] = 0;
    __syncthreads();
    const uint32_t tau = sm.tau;
    const int need = sm.need;
    // when every element at tau is needed the ties need no ordering
    const bool all_ties = sm.ties == need;
    // pairs of values whose larger order key reaches tau - 1 (-0 has the packed key 0x7FFF,
    // one below +0) are examined one by one; the rest are skipped two at a time
    const uint16_t lo_t = tau > 0u ? (uint16_t)(tau - 1u) : (uint16_t)0;
    uint32_t tiemask = 0;
#pragma unroll
    for (int q = 0; q < kLoads; ++q)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t w = v[q][d];
            const uint32_t neg = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, w) >> (i16x2)(int16_t)15);
            const u16x2 k2 = __builtin_bit_cast(u16x2, w ^ (neg | 0x80008000u));
            if (max(k2[0], k2[1]) < lo_t) continue;
            for (int e2 = 0; e2 < 2; ++e2) {
                const int e = 2 * d + e2;
                const int col = col_of(c0, q, e);
                const uint32_t h = e2 ? (w >> 16) : (w & 0xFFFFu);
                if (col >= V || (h & 0x7FFFu) >= 0x7F80u) continue;  // past the row, inf, NaN
                const uint32_t k = key16(h);
                if (k > tau || (k == tau && all_ties && need > 0)) {
                    const int slot = (int)atomicAdd(&sm.n_top[r], 1u);
                    if (slot < kTop) {
                        sm.top_key[r][slot] = k;
                        sm.top_id[r][slot] = col;
                    }
                } else if (k == tau && need > 0) {
                    tiemask |= 1u << (q * 8 + e);
                }
            }
        }
    __syncthreads();
    int base = min((int)sm.n_top[r], kTop);
    int need_left = all_ties ? 0 : need;
    // then the first `need` elements at tau in token order (uniform loop)
    for (int q = 0; q < kLoads && need_left > 0; ++q) {
        const uint32_t mq = (tiemask >> (q * 8)) & 0xFFu;
        int total;
        const int before = block_exclusive_scan<int>(__popc(mq), sm.scan, &total);
        int k = 0;
        for (int e = 0; e < 8; ++e) {
            if (!(mq & (1u << e))) continue;
            const int rank = before + k++;
            const int slot = base + rank;
            if (rank < need_left && slot < kTop) {
                sm.top_key[r][slot] = tau;
                sm.top_id[r][slot] = col_of(c0, q, e);
            }
        }
        const int took = min(total, need_left);
        base += took;
        need_left -= took;
    }
    __syncthreads();
    const int n = min(base, kTop);
    // sort: key desc, id asc (rank by counting)
    uint32_t mk = 0;
    int mi = 0, rank = 0;
    if ((int)threadIdx.x < n) {
        mk = sm.top_key[r][threadIdx.x];
        mi = sm.top_id[r][threadIdx.x];
        for (int i = 0; i < n; ++i) {
            const uint32_t k2 = sm.top_key[r][i];
            const int i2 = sm.top_id[r][i];
            rank += (k2 > mk || (k2 == mk && i2 < mi)) ? 1 : 0;
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < n) {
        sm.top_key[r][rank] = mk;
        sm.top_id[r][rank] = mi;
    }
    if (threadIdx.x == 0) sm.n_top[r] = (uint32_t)n;
    __syncthreads();
}

// Elements of row r in this slice with the draft token's key that precede the token (token
// order): all of them when the slice lies before the token's slice, none after it.
__device__ __forceinline__ void local_rank(CountSmem& sm, int r, int c0, int s_tok, const u32x4 (&v)[kLoads]) {
    const uint32_t h_s = sm.s_bits[r];
    uint32_t cnt = 0;
    if (s_tok >= c0 + kSliceCols) {
        // the whole slice precedes the token: the count of its key (bin or special)
        if ((h_s & 0x7FFFu) < 0x7F80u) {
            const uint32_t ks = key16(h_s);
            if (key_is_binned(ks)) {
                cnt = threadIdx.x == 0 ? sm.hist(r)[key_bin(ks)] : 0u;
            } else {
                const int nsp = min((int)sm.n_sp[r], kSpecial);
                cnt = ((int)threadIdx.x < nsp && sm.sp_key[r][threadIdx.x] == ks) ? 1u : 0u;
            }
        }
    } else if (s_tok >= c0 && (h_s & 0x7FFFu) < 0x7F80u) {
        const uint32_t ks = key16(h_s);
#pragma unroll
        for (int q = 0; q < kLoads; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int col = col_of(c0, q, e);
                const uint32_t w = v[q][e >> 1];
                const uint32_t h = (e & 1) ? (w >> 16) : (w & 0xFFFFu);
                cnt += (col < s_tok && (h & 0x7FFFu) < 0x7F80u && key16(h) == ks) ? 1u : 0u;
            }
    }
    cnt = block_sum<uint32_t>(cnt, reinterpret_cast<uint32_t*>(sm.redi));
    if (threadIdx.x == 0) sm.cnt_s[r] = cnt;
}

// Publishes the summary of row r (its element passes are done): largest logit, per-segment
// counts and masses, specials, the fine counts, the candidate list and the token's rank.
__device__ __forceinline__ void publish_row(const FastArgs& f, CountSmem& sm, int unit, int slice, int r,
                                            const spec_params& prm) {
    RowPart* P = part_of(f, unit, slice, r);
    const double T = (double)prm.temperature;
    const int nsp = min((int)sm.n_sp[r], kSpecial);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    // largest key: the first non-empty segment, then its highest bin or special (wave 0)
    if (wave == 0) {
        const uint64_t ne = __ballot(lane < kSegs && sm.segc[r][lane] != 0u);
        uint32_t mk = 0;
        if (ne != 0) {
            const int sg = first_lane(ne);
            const int g = group_of_seg(sg);
            if (g >= 0) {
                const int i = first_lane(__ballot(sm.hist(r)[bin_of_sel(g, lane)] != 0u));
                mk = bin_key(bin_of_sel(g, i));
            } else {
                const uint32_t k = lane < nsp ? sm.sp_key[r][lane] : 0u;
                mk = wave_max((lane < nsp && special_seg(k) == sg) ? k : 0u);
            }
        }
        if (lane == 0) sm.maxkey = mk;
    }
    __syncthreads();
    const uint32_t mk = sm.maxkey;
    const float m = mk ? key16_value(mk) : -__builtin_inff();
    // per-group masses (relative to this slice's largest logit), one wave per group
#pragma unroll 1
    for (int g = wave; g < kGroups; g += kWaves) {
        if (sm.segc[r][seg_of_group(g)] == 0u) {
            if (lane == 0) sm.segm[seg_of_group(g)] = 0.0;
            continue;
        }
        const int bin = g * kGroup + lane;
        const uint32_t c = sm.hist(r)[bin];
        double ms = 0.0;
        if (c != 0 && T > 0.0) ms = (double)c * mass_of(key16_value(bin_key(bin)), m, T);
        ms = wave_sum(ms);
        if (lane == 0) sm.segm[seg_of_group(g)] = ms;
    }
    // the four special segments, one lane per special
    if (wave == kWaves - 1) {
        int sg = -1;
        double ms = 0.0;
        if (lane < nsp) {
            const uint32_t k = sm.sp_key[r][lane];
            sg = special_seg(k);
            if (T > 0.0) ms = mass_of(key16_value(k), m, T);
        }
        const int sps[4] = {kSegHugePos, kSegTinyPos, kSegTinyNeg, kSegHugeNeg};
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const double sx = wave_sum(sg == sps[x] ? ms : 0.0);
            if (lane == 0) sm.segm[sps[x]] = sx;
        }
    }
    __syncthreads();
    if (wave == 0) {
        const double S = wave_sum(lane < kSegs ? sm.segm[lane] : 0.0);
        const uint32_t nfin = wave_sum(lane < kSegs ? sm.segc[r][lane] : 0u);
        if (lane == 0) {
            P->m = m;
            P->flags = (sm.flags[r] & 1u) | ((int)sm.n_sp[r] > kSpecial ? 2u : 0u);
            P->n_finite = nfin;
            P->n_special = (uint32_t)nsp;
            P->n_top = sm.n_top[r];
            P->cnt_s = sm.cnt_s[r];
            P->s_bits = sm.s_bits[r];
            P->n_neginf = sm.neginf[r];
            P->S = S;
        }
    }
    for (int sg = threadIdx.x; sg < kSegs; sg += blockDim.x) {
        P->seg_mass[sg] = sm.segm[sg];
        P->seg_count[sg] = sm.segc[r][sg];
    }
    if ((int)threadIdx.x < nsp) {
        P->sp_key[threadIdx.x] = sm.sp_key[r][threadIdx.x];
        P->sp_id[threadIdx.x] = sm.sp_id[r][threadIdx.x];
    }
    if ((int)threadIdx.x < (int)sm.n_top[r]) {
        P->top_key[threadIdx.x] = sm.top_key[r][threadIdx.x];
        P->top_id[threadIdx.x] = sm.top_id[r][threadIdx.x];
    }
    // fine counts, two per dword (a slice holds < 65536 columns)
    uint32_t* fine32 = reinterpret_cast<uint32_t*>(P->fine);
#pragma unroll 1
    for (int i = threadIdx.x; i < kBins / 2; i += blockDim.x)
        fine32[i] = (sm.hist(r)[2 * i] & 0xFFFFu) | (sm.hist(r)[2 * i + 1] << 16);
    __syncthreads();  // segm is reused by the next row
}

// Counts this thread's columns of row r: every value goes to its bin or a padding word (one
// LDS add each, no branch).
__device__ __forceinline__ void count_row(CountSmem& sm, int r, const u32x4 (&v)[kLoads]) {
    char* base = reinterpret_cast<char*>(&sm.hraw[r][0]);
#pragma unroll
    for (int q = 0; q < kLoads; ++q)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t o = hist_offsets2(v[q][d]);
            atomicAdd(reinterpret_cast<uint32_t*>(base + (o & 0xFFFFu)), 1u);
            atomicAdd(reinterpret_cast<uint32_t*>(base + (o >> 16)), 1u);
        }
}

// Second pass over the values the packed count sent to the padding words: zeros, specials,
// -inf, +inf, NaN (and the zero fill past the row's end).
__device__ __forceinline__ void count_rare(CountSmem& sm, int r, int c0, int V, const u32x4 (&v)[kLoads]) {
    uint32_t bad = 0, ninf = 0;
    for (int q = 0; q < kLoads; ++q)
        for (int e = 0; e < 8; ++e) {
            const int col = col_of(c0, q, e);
            const uint32_t w = v[q][e >> 1];
            const uint32_t h = (e & 1) ? (w >> 16) : (w & 0xFFFFu);
            const uint32_t off = (h & 0x7FFFu) - (uint32_t)(kExpLo << 7);
            if (col >= V || off < (uint32_t)kNegBins) continue;
            int bin;
            const int kind = classify(h, &bin);
            if (kind == kKindBin) {
                atomicAdd(&sm.hist(r)[bin], 1u);
            } else if (kind == kKindSpecial) {
                const uint32_t slot = atomicAdd(&sm.n_sp[r], 1u);
                if (slot < (uint32_t)kSpecial) {
                    sm.sp_key[r][slot] = key16(h);
                    sm.sp_id[r][slot] = col;
                }
            } else if (kind == kKindNegInf) {
                ++ninf;
            } else {
                bad = 1;
            }
        }
    if (bad) atomicOr(&sm.flags[r], 1u);
    if (ninf) atomicAdd(&sm.neginf[r], ninf);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(6, 8))) void fast_count_kernel(FastArgs f) {
    __shared__ CountSmem sm;
    const VerifyArgs& a = f.a;
    const Place P = place_of(f);
    if (P.b >= a.B) return;
    const int j = P.j, slice = P.slice, unit = P.unit;
    const int c0 = slice * kSliceCols;
    const bool two = j < a.K;
    const spec_params prm = a.params[P.b];
    if (!params_ok(prm)) return;  // the resolve kernel reports BAD_PARAM without reading summaries
    const size_t stride = (size_t)a.V;
    const uint16_t* trow = static_cast<const uint16_t*>(a.target) + ((size_t)P.b * (a.K + 1) + j) * stride;
    const uint16_t* drow = two ? static_cast<const uint16_t*>(a.draft) + ((size_t)P.b * a.draft_rows + j) * stride : nullptr;
    const int s_tok = two ? a.tokens[(size_t)P.b * a.K + j] : -1;
    const bool tok_ok = !two || (s_tok >= 0 && s_tok < a.V);

    u32x4 vq[kLoads], vp[kLoads];
    load_slice(trow, c0, a.V, vq);
    if (two) load_slice(drow, c0, a.V, vp);
    for (int i = threadIdx.x; i < 2 * kHistRow / 4; i += blockDim.x)
        reinterpret_cast<u32x4*>(&sm.hraw[0][0])[i] = u32x4{0, 0, 0, 0};
    if (threadIdx.x < 2) {
        sm.n_sp[threadIdx.x] = 0;
        sm.flags[threadIdx.x] = 0;
        sm.neginf[threadIdx.x] = 0;
    }
    // the rows' values at the draft token (every slice counts the token's key); one thread
    // writes both words, zero without a token
    if (threadIdx.x == kWave) {
        const bool has = two && tok_ok;
        sm.s_bits[0] = has ? trow[s_tok] : 0u;
        sm.s_bits[1] = has ? drow[s_tok] : 0u;
    }
    __syncthreads();
    count_row(sm, 0, vq);
    if (two) count_row(sm, 1, vp);
    __syncthreads();
    const bool rare0 = (sm.hraw[0][kHistLead - 1] | sm.hraw[0][kHistLead + kBins]) != 0;
    const bool rare1 = two && (sm.hraw[1][kHistLead - 1] | sm.hraw[1][kHistLead + kBins]) != 0;
    if (rare0) count_rare(sm, 0, c0, a.V, vq);
    if (rare1) count_rare(sm, 1, c0, a.V, vp);
    if (threadIdx.x < 2) {
        sm.n_top[threadIdx.x] = 0;
        sm.cnt_s[threadIdx.x] = 0;
    }
    __syncthreads();
    seg_counts(sm, two ? 2 : 1);
    __syncthreads();
    // passes over the columns (registers) first, so the columns are dead for the summaries
    const bool holds_s = two && tok_ok && s_tok >= c0;  // at or after this slice: count its key
    const int want_q = list_len(a, prm, false), want_p = two ? list_len(a, prm, true) : 0;
    if (want_q > 0) local_top(sm, 0, want_q, c0, a.V, vq);
    if (holds_s) local_rank(sm, 0, c0, s_tok, vq);
    if (two) {
        if (want_p > 0) local_top(sm, 1, want_p, c0, a.V, vp);
        if (holds_s) local_rank(sm, 1, c0, s_tok, vp);
    }
    __syncthreads();
    publish_row(f, sm, unit, slice, 0, prm);
    if (two) publish_row(f, sm, unit, slice, 1, prm);
}

void launch_count(const FastArgs& f, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(fast_count_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, f);
}

}  // namespace fast
}  // namespace sv
