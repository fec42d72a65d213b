// Count kernel of the bf16 verification path: every slice of every (request, position) unit
// loads its token columns of the target row (and the draft row), counts every distinct bf16
// value in LDS and publishes a compact summary for the resolve kernel.
#include <hip/hip_ext.h>

#include <atomic>

#include "fast_settle.h"

namespace sv {
namespace fast {

// ------------------------------------------------------------------------------------------
// Count kernel: every slice of every unit loads its columns, counts them and publishes its
// summaries; the last slice of a unit to finish settles the unit, and the last unit of a
// request to be settled decides the request (no workgroup waits on another).
// ------------------------------------------------------------------------------------------
struct CountSmem {
    alignas(16) uint32_t hraw[2][kHistRow];  // counting; when settling, the unit's merged
                                             // histograms, then the occupied slots' lists
    __device__ __forceinline__ uint32_t* hist(int r) { return &hraw[r][kHistLead]; }
    __device__ __forceinline__ const uint32_t* hist(int r) const { return &hraw[r][kHistLead]; }
    uint32_t segc[2][kSegs];
    uint32_t sp_key[2][kSpecial];
    int32_t sp_id[2][kSpecial];
    uint32_t n_sp[2];
    uint32_t th_tau[2];  // each row's candidate threshold (Threshold) from the entry scan
    int32_t th_need[2];
    int32_t th_ties[2];
    uint64_t red64[kWaves];
    uint32_t n_ent[2];   // occupied bins per row (entries published)
    uint32_t cnt_s[2];
    uint32_t flags[2];
    uint32_t neginf[2];
    int32_t scan[kWaves + 1];
    double redd[kWaves];
    int32_t redi[kWaves];
    uint32_t s_bits[2];
    int last;
    int rare[2];
    double u_acc;  // the acceptance draw of the unit's position
    double u_res;  // its residual / bonus draw
    uint32_t unit_code;  // the settled unit's outcome (unit_code)
    uint32_t xcc;        // the XCD this workgroup runs on
    SettleSmem ss;       // settling the unit
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

// The key of the L-th element (token order) of row r in this slice, how many elements at that
// key are taken and how many the slice holds at it; (0, 0, 0) when the slice holds fewer than
// L finite elements.  Scans the segment counts, then the 64 bins of the crossing group, or the
// specials of the crossing segment.  Every wave computes it for itself (uniform results), so
// no barrier is needed before the element pass.
struct Threshold {
    uint32_t tau;
    int need, ties;
};
__device__ __forceinline__ Threshold local_threshold(const CountSmem& sm, int r, int L) {
    const int lane = threadIdx.x & (kWave - 1);
    Threshold th{0u, 0, 0};
    const int c = lane < kSegs ? (int)sm.segc[r][lane] : 0;
    int cex;
    const int cin = wave_scan(c, &cex);
    const uint64_t hit = __ballot(lane < kSegs && cin >= L);
    if (hit == 0) return th;
    const int sg = first_lane(hit);
    const int rem = L - wave_bcast(cex, sg);
    const int g = group_of_seg(sg);
    if (g >= 0) {
        const int bin = bin_of_sel(g, lane);  // lane order = descending key
        const int n = (int)sm.hist(r)[bin];
        int nex;
        const int nin = wave_scan(n, &nex);
        const int i = first_lane(__ballot(nin >= rem));
        th.tau = bin_key(wave_bcast(bin, i));
        th.need = rem - wave_bcast(nex, i);
        th.ties = wave_bcast(n, i);
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
        const uint64_t at = __ballot(mine && gt < rem && gt + eq >= rem);
        if (at != 0) {
            const int x = first_lane(at);
            th.tau = wave_bcast(k, x);
            th.need = rem - wave_bcast(gt, x);
            th.ties = wave_bcast(eq, x);
        }
    }
    return th;
}

// Word i (= 4 q + d: load q, word d) of this thread's columns of a row, for an index that differs
// between lanes: a select over the loads, then over the words (no indexed register access).
__device__ __forceinline__ uint32_t word_at(const u32x4 (&v)[kLoads], int i) {
    // (masks rather than selects, which the compiler would turn back into an indexed access of a
    // register array placed in scratch memory)
    uint32_t w = 0u;
#pragma unroll
    for (int qq = 0; qq < kLoads; ++qq)
#pragma unroll
        for (int d = 0; d < 4; ++d) w |= v[qq][d] & (0u - (uint32_t)(i == qq * 4 + d));
    return w;
}

// Marks this thread's elements of one row: cand for those above the threshold key (and at it
// when every element there is needed), ties for those at it otherwise.  One pass over the words
// finds those holding a value whose order key is at least tau - 1 (-0 has the packed key 0x7FFF,
// one below +0); only those words are examined element by element (few: the threshold leaves at
// most a few dozen elements of the slice above it).
struct TopMarks {
    uint32_t cand, ties;
};
__device__ __forceinline__ TopMarks top_marks(const Threshold& th, int c0, int V, const u32x4 (&v)[kLoads]) {
    const uint32_t tau = th.tau;
    const bool all_ties = th.ties == th.need;
    const uint16_t lo_t = tau > 0u ? (uint16_t)(tau - 1u) : (uint16_t)0;
    uint32_t words = 0u;  // bit 4 q + d: word d of load q holds a key >= lo_t
#pragma unroll
    for (int q = 0; q < kLoads; ++q)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t w = v[q][d];
            const uint32_t neg = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2, w) >> (i16x2)(int16_t)15);
            const u16x2 k2 = __builtin_bit_cast(u16x2, w ^ (neg | 0x80008000u));
            words |= (max(k2[0], k2[1]) >= lo_t ? 1u : 0u) << (q * 4 + d);
        }
    uint32_t cand = 0u, ties = 0u;
    while (words != 0u) {
        const int i = __builtin_ctz(words);
        words &= words - 1u;
        const uint32_t w = word_at(v, i);
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
            const int b = 2 * i + e2;  // element bit: 8 q + e
            const uint32_t h = e2 ? (w >> 16) : (w & 0xFFFFu);
            if (col_of(c0, b >> 3, b & 7) >= V || (h & 0x7FFFu) >= 0x7F80u) continue;  // past the row, inf, NaN
            const uint32_t k = key16(h);
            const bool at = k == tau && th.need > 0;
            const bool c = k > tau || (at && all_ties);
            cand |= (c ? 1u : 0u) << b;
            ties |= (at && !c ? 1u : 0u) << b;
        }
    }
    return TopMarks{cand, ties};
}

// This thread's marked elements of a row (bit 8 q + e of m) into the row's candidate list from
// slot on, in bit order (a lane holds one or two at most, mostly).
__device__ __forceinline__ void write_marked(RowPart* P, uint32_t m, int slot, int c0, const u32x4 (&v)[kLoads]) {
    while (m != 0u && slot < kTop) {
        const int b = __builtin_ctz(m);
        m &= m - 1u;
        const uint32_t w = word_at(v, b >> 1);
        P->top_key[slot] = key16((w >> (16 * (b & 1))) & 0xFFFFu);
        P->top_id[slot] = col_of(c0, b >> 3, b & 7);
        ++slot;
    }
}

// The first L[r] elements (token order: key desc, id asc) of each row r in this slice (none for
// L[r] = 0), in no particular order, straight into the rows' records (top_key / top_id); returns
// their numbers in n.  The threshold of a row comes from the entry scan (sm.th_*) or, for a row
// with values outside the bins (slow), from the segment counts.  One pass marks every thread's
// elements above each row's threshold (and at it when every element there is needed); one
// workgroup scan of both rows' mark counts (at most L[r] <= 64 each, packed in 16-bit halves)
// gives each marked element its slot in thread order; the elements at a threshold of which only
// some are needed follow in token order (rare).  The settle step ranks the lists itself.
__device__ __forceinline__ void local_tops(const FastArgs& f, CountSmem& sm, int unit, int slice, const int (&L)[2],
                                           const bool (&slow)[2], int c0, int V, const u32x4 (&vq)[kLoads],
                                           const u32x4 (&vp)[kLoads], int (&n)[2]) {
    Threshold th[2] = {{0u, 0, 0}, {0u, 0, 0}};
    uint32_t cand[2] = {0u, 0u}, ties[2] = {0u, 0u};
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        if (L[r] <= 0) continue;
        th[r] = slow[r] ? local_threshold(sm, r, L[r]) : Threshold{sm.th_tau[r], sm.th_need[r], sm.th_ties[r]};
        // (uniform values: kept in scalar registers)
        th[r].tau = __builtin_amdgcn_readfirstlane(th[r].tau);
        th[r].need = __builtin_amdgcn_readfirstlane(th[r].need);
        th[r].ties = __builtin_amdgcn_readfirstlane(th[r].ties);
        const TopMarks m = r ? top_marks(th[r], c0, V, vp) : top_marks(th[r], c0, V, vq);
        cand[r] = m.cand;
        ties[r] = m.ties;
    }
    int total;
    const int before = block_exclusive_scan<int>(__popc(cand[0]) | (__popc(cand[1]) << 16), sm.scan, &total);
    n[0] = total & 0xFFFF;
    n[1] = total >> 16;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const uint32_t m = cand[r];
        if (m == 0u) continue;
        RowPart* P = part_of(f, unit, slice, r);
        int slot = r ? before >> 16 : before & 0xFFFF;
        if (r) write_marked(P, m, slot, c0, vp);
        else write_marked(P, m, slot, c0, vq);
    }
    // then the first `need` elements at tau in token order (uniform loop; rare)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        if (L[r] <= 0 || th[r].ties == th[r].need) continue;
        RowPart* P = part_of(f, unit, slice, r);
        int need_left = th[r].need;
        for (int q = 0; q < kLoads && need_left > 0; ++q) {
            const uint32_t mq = (ties[r] >> (q * 8)) & 0xFFu;
            int cnt;
            const int pre = block_exclusive_scan<int>(__popc(mq), sm.scan, &cnt);
            int k = 0;
            for (int e = 0; e < 8; ++e) {
                if (!(mq & (1u << e))) continue;
                const int rank = pre + k++;
                const int slot = n[r] + rank;
                if (rank < need_left && slot < kTop) {
                    P->top_key[slot] = th[r].tau;
                    P->top_id[slot] = col_of(c0, q, e);
                }
            }
            const int took = min(cnt, need_left);
            n[r] += took;
            need_left -= took;
        }
    }
    n[0] = min(n[0], kTop);
    n[1] = min(n[1], kTop);
}

// Elements of each row in this slice with the draft token's key that precede the token (token
// order): all of them when the slice lies before the token's slice (a histogram or specials
// lookup, no element pass), those left of the token in its own slice (one element pass per
// row, both rows' counts packed into one workgroup sum).  Callers synchronise.
__device__ __forceinline__ void local_ranks(CountSmem& sm, bool two, int c0, int s_tok, const u32x4 (&vq)[kLoads],
                                            const u32x4 (&vp)[kLoads]) {
    const int rows = two ? 2 : 1;
    if (s_tok >= c0 + kSliceCols) {
        const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
        if (wave < rows) {
            const int r = wave;
            const uint32_t h_s = sm.s_bits[r];
            uint32_t cnt = 0;
            if ((h_s & 0x7FFFu) < 0x7F80u) {
                const uint32_t ks = key16(h_s);
                if (key_is_binned(ks)) {
                    cnt = sm.hist(r)[key_bin(ks)];
                } else {
                    const int nsp = min((int)sm.n_sp[r], kSpecial);
                    cnt = (uint32_t)__popcll(__ballot(lane < nsp && sm.sp_key[r][lane] == ks));
                }
            }
            if (lane == 0) sm.cnt_s[r] = cnt;
        }
        return;
    }
    // Equal keys are equal bf16 bit patterns, except that -0 and +0 share one key: a word's two
    // values are compared with the token's pattern at once (the sign bits masked off for zero),
    // and a 16-bit half is zero exactly when ((x & 0x7FFF) + 0x7FFF) | x has its top bit clear.
    // Loads past the token's column hold no element before it (a uniform skip); in the load that
    // holds it, each thread masks the elements at or after it.
    const int q_tok = (s_tok - c0) / (kThreads * 8);  // the load holding the token's column
    uint32_t packed = 0;  // row 0 in the low half, row 1 in the high half (each < 2^16)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        if (r == 1 && !two) break;
        const uint32_t h_s = sm.s_bits[r];
        if ((h_s & 0x7FFFu) >= 0x7F80u) continue;  // (a non-finite token value has no rank)
        const uint32_t pat = (h_s & 0x7FFFu) == 0u ? 0u : h_s;
        const uint32_t keep = pat == 0u ? 0x7FFF7FFFu : 0xFFFFFFFFu;
        const uint32_t pat2 = pat * 0x10001u;
        const u32x4(&v)[kLoads] = r == 0 ? vq : vp;
        uint32_t miss = 0, slots = 0;  // compared halves that differ, halves compared
#pragma unroll
        for (int q = 0; q < kLoads; ++q) {
            if (q > q_tok) break;
            // elements of this thread's 8 columns of load q that precede the token: 8 below q_tok
            const int rel = q < q_tok ? 8 : min(max(s_tok - col_of(c0, q, 0), 0), 8);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t y = (v[q][d] & keep) ^ pat2;
                const uint32_t t = ((y & 0x7FFF7FFFu) + 0x7FFF7FFFu) | y;
                const int left = rel - 2 * d;  // elements of word d before the token: 2, 1 or 0
                const uint32_t vm = left >= 2 ? 0x80008000u : (left == 1 ? 0x8000u : 0u);
                miss += (uint32_t)__popc(t & vm);
                slots += (uint32_t)__popc(vm);
            }
        }
        packed += (slots - miss) << (16 * r);
    }
    packed = block_sum<uint32_t>(packed, reinterpret_cast<uint32_t*>(sm.redi));
    if (threadIdx.x < (unsigned)rows) sm.cnt_s[threadIdx.x] = (packed >> (16 * threadIdx.x)) & 0xFFFFu;
}

// Places both rows' occupied bins as (bin, count) entries in ascending bin order (returns this
// thread's exclusive scan word for write_entries); thread t reads bins [6t, 6t + 6).  One workgroup scan of both rows' entry and element
// counts places every entry and tells each thread how many of the row's binned elements lie
// above its bins, so for a row listing L > 0 candidates without values outside the bins (fast)
// the thread holding the L-th element from the top records it as the row's threshold (sm.th_*:
// key, elements taken at it, elements there; 0 when the slice holds fewer than L).  n_ent gets
// the entry counts (sm.n_ent).
__device__ __forceinline__ uint32_t scan_entries(CountSmem& sm, bool two, const int (&L)[2], const bool (&fast)[2]) {
    constexpr int kPer = 6;
    constexpr int kPubThreads = kBins / kPer;  // 480
    static_assert(kPer * kPubThreads == kBins && kPubThreads <= kThreads, "bins per thread");
    const int rows = two ? 2 : 1;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    // (the counts are read again after the scan: the columns stay live in registers meanwhile)
    uint32_t nz[2] = {0u, 0u}, cs[2] = {0u, 0u};
    const int b0 = tid < kPubThreads ? tid * kPer : 0;  // (reads are unconditional, then masked)
    const bool mine = tid < kPubThreads;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const uint32_t c0 = sm.hist(r)[b0 + i];
            const uint32_t c = (r < rows && mine) ? c0 : 0u;
            cs[r] += c;
            nz[r] += c != 0u ? 1u : 0u;
        }
    // entries (12 bits) and elements (15 bits) of both rows in one 64-bit scan (one barrier)
    const uint64_t v = (uint64_t)nz[0] | ((uint64_t)cs[0] << 12) | ((uint64_t)nz[1] << 27) | ((uint64_t)cs[1] << 39);
    uint64_t exc;
    const uint64_t inc = wave_scan(v, &exc);
    if (lane == kWave - 1) sm.red64[wave] = inc;
    __syncthreads();
    uint64_t before = 0ull, total = 0ull;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const uint64_t x = sm.red64[w];
        if (w < wave) before += x;
        total += x;
    }
    exc += before;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int sh = r ? 27 : 0;
        if (tid == 0) sm.n_ent[r] = (uint32_t)((total >> sh) & 0xFFFu);
        if (r >= rows) break;
        if (fast[r] && L[r] > 0) {
            uint32_t cnt[kPer];
#pragma unroll
            for (int i = 0; i < kPer; ++i) cnt[i] = mine ? sm.hist(r)[b0 + i] : 0u;
            const uint32_t all = (uint32_t)(total >> (sh + 12)) & 0x7FFFu;
            const uint32_t below = (uint32_t)(exc >> (sh + 12)) & 0x7FFFu;
            const uint32_t above = all - below - cs[r];  // binned elements in higher bins
            if (above < (uint32_t)L[r] && above + cs[r] >= (uint32_t)L[r]) {
                uint32_t cum = above;
                bool done = false;
#pragma unroll
                for (int i = kPer - 1; i >= 0; --i) {
                    if (!done && cnt[i] != 0u && cum + cnt[i] >= (uint32_t)L[r]) {
                        done = true;
                        sm.th_tau[r] = bin_key(tid * kPer + i);
                        sm.th_need[r] = (int)((uint32_t)L[r] - cum);
                        sm.th_ties[r] = (int)cnt[i];
                    }
                    cum += cnt[i];
                }
            }
        }
    }
    return (uint32_t)(exc & 0xFFFu) | ((uint32_t)((exc >> 27) & 0xFFFu) << 12);
}

// Writes both rows' entries at the places the scan gave them (pos: this thread's first entry of
// row 0 and of row 1, 12 bits each).
__device__ __forceinline__ void write_entries(const FastArgs& f, const CountSmem& sm, int unit, int slice, bool two,
                                              uint32_t pos) {
    constexpr int kPer = 6;
    constexpr int kPubThreads = kBins / kPer;
    const int tid = threadIdx.x;
    if (tid >= kPubThreads) return;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        if (r == 1 && !two) break;
        RowPart* P = part_of(f, unit, slice, r);
        int o = (int)((pos >> (r ? 12 : 0)) & 0xFFFu);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const uint32_t c = sm.hist(r)[tid * kPer + i];
            if (c != 0u) P->ent[o++] = ((uint32_t)(tid * kPer + i) << 16) | c;
        }
    }
}

// The rest of both rows' slice summaries (RowPart): the specials, the drafted token's value and
// rank, and the header (after the candidates, whose number it holds).
__device__ __forceinline__ void publish_header(const FastArgs& f, CountSmem& sm, int unit, int slice, bool two,
                                               const int (&n_top)[2]) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        if (r == 1 && !two) break;
        RowPart* P = part_of(f, unit, slice, r);
        const int nsp = min((int)sm.n_sp[r], kSpecial);
        if (tid < nsp) {
            P->sp_key[tid] = sm.sp_key[r][tid];
            P->sp_id[tid] = sm.sp_id[r][tid];
        }
        if (tid == r) {
            const uint32_t flags = (sm.flags[r] & 1u) | ((int)sm.n_sp[r] > kSpecial ? 2u : 0u) | (sm.rare[r] ? 4u : 0u);
            reinterpret_cast<u32x4*>(P)[0] = u32x4{flags, sm.n_ent[r], (uint32_t)nsp, (uint32_t)n_top[r]};
            reinterpret_cast<u32x4*>(P)[1] = u32x4{sm.cnt_s[r], sm.s_bits[r], sm.neginf[r], sm.xcc};
        }
    }
}

// Counts this thread's columns of row r: every value goes to its bin or a padding word (one
// LDS add each, no branch).  Vectors past the row's end (zero fill) are skipped.
__device__ __forceinline__ void count_row(CountSmem& sm, int r, int c0, int V, const u32x4 (&v)[kLoads]) {
    char* base = reinterpret_cast<char*>(&sm.hraw[r][0]);
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
        if (col_of(c0, q, 0) >= V) continue;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t o = hist_offsets2(v[q][d]);
            atomicAdd(reinterpret_cast<uint32_t*>(base + (o & 0xFFFFu)), 1u);
            atomicAdd(reinterpret_cast<uint32_t*>(base + (o >> 16)), 1u);
        }
    }
}

// Second pass over the values the packed count sent to the padding words: zeros, specials,
// -inf, +inf, NaN (and the zero fill past the row's end).
__device__ __forceinline__ void count_rare(CountSmem& sm, int r, int c0, int V, const u32x4 (&v)[kLoads]) {
    uint32_t bad = 0, ninf = 0;
#pragma unroll
    for (int q = 0; q < kLoads; ++q)
#pragma unroll
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

// A unit's outcome in 7 bits for the request rendezvous: accepted, general path, and the
// status bits the decision reads.
__device__ __forceinline__ uint32_t unit_code(int accept, int fallback, uint32_t st) {
    return (accept ? 1u : 0u) | (fallback ? 2u : 0u) | ((st & kStBadParam) ? 4u : 0u) | ((st & kStBadLogit) ? 8u : 0u) |
           ((st & kStBadToken) ? 16u : 0u) | ((st & kStDegenerate) ? 32u : 0u) | ((st & kStOutside) ? 64u : 0u);
}
constexpr int kCodeBits = 7, kCountBits = 4;
constexpr int kPackedUnits = (64 - kCountBits) / kCodeBits;  // 8: requests with K + 1 <= 8 units

// The last slice of a unit: combine, acceptance test, unit record.
__device__ __forceinline__ void settle_unit(const FastArgs& f, CountSmem& sm, const Place& P, const spec_params& prm,
                                            bool param_ok, bool two, int s_tok, bool tok_ok) {
    const VerifyArgs& a = f.a;
    const int unit = P.unit;
    SettleSmem& us = sm.ss;
    uint32_t status = 0;
    int accept = 0, fallback = 0;
    if (!param_ok) {
        status = kStBadParam;
    } else {
        const bool vd = P.j < a.K;      // the drafted token is verified here
        const bool vrow = vd && two;     // against a draft row (not the uniform draft)
        settle_rows(f, sm, unit, P.slice, P.j, two ? 2 : 1, prm, vd, s_tok);
        // every value the outcome needs, read at once and combined without branches (a chain of
        // dependent reads and branches costs a round trip each)
        const RowView& v0 = us.rv[0];
        const RowView& v1 = us.rv[1];
        const int bad0 = v0.bad, bad1 = v1.bad, ov0 = v0.overflow, ov1 = v1.overflow, dg1 = v1.degenerate;
        const int gr0 = v0.greedy, am0 = v0.argmax;
        const uint32_t xb0 = v0.xcc_bad, xb1 = v1.xcc_bad;
        const double ps_row = us.ps, qs = us.qs, u = sm.u_acc;
        const bool bad = (bad0 != 0) | (vrow & (bad1 != 0));
        const bool ovf = (ov0 != 0) | (vrow & (ov1 != 0));
        // the unit's slices did not share one XCD's L2: the request is redone by the general path
        const bool misplaced = (xb0 != 0u) | (two & (xb1 != 0u));
        fallback = ((!bad & ovf) | misplaced) ? 1 : 0;
        if (misplaced && threadIdx.x == 0) atomicOr(&reinterpret_cast<ReqFast*>(f.ws + f.L.reqs)[P.b].pad, (int32_t)kStPlacement);
        const double ps = f.uniform ? 1.0 / (double)a.V : ps_row;
        const int acc_v = gr0 ? (s_tok == am0 ? 1 : 0) : (u * ps < qs ? 1 : 0);
        const uint32_t st = ((vrow & (dg1 != 0)) ? kStDegenerate : 0u) | (!tok_ok ? kStBadToken : 0u) |
                            ((tok_ok & vd & (gr0 == 0) & !(ps > 0.0)) ? kStOutside : 0u);
        status = bad ? kStBadLogit : fallback ? 0u : st;
        accept = (bad | (fallback != 0) | !tok_ok) ? 0 : (vd ? acc_v : 1);  // (the bonus position accepts)
    }
    // the outcome cache's depth-j list: the first F_j candidates of the draft row in token order,
    // less the drafted token; rows the candidate lists cannot settle (NaN or +inf, too many
    // specials, too few finite values) go to the general selection in the resolve kernel
    if (f.cache && f.fan.f[P.j] > 0) {
        const int Fj = f.fan.f[P.j];
        const int want = Fj + (P.j < a.K ? 1 : 0);
        const RowView& rv = us.rv[1];
        const bool general = !param_ok | (rv.bad != 0) | (rv.overflow != 0) | (rv.nm < min(want, a.V));
        if (threadIdx.x == 0) reinterpret_cast<int32_t*>(f.ws + f.L.cache_gen)[unit] = general ? 1 : 0;
        if (!general && threadIdx.x < kWave) {
            const int lane = threadIdx.x;
            const int excl = (P.j < a.K && tok_ok) ? s_tok : -1;
            const int n = rv.nm;
            const int id = lane < n ? us.oid[1][lane] : -1;
            const uint64_t ex = __ballot(lane < n && id == excl);
            const int xpos = first_lane(ex);  // -1: the drafted token is not listed
            int32_t* out = f.out_cache + (size_t)P.b * f.budget + f.fan.off[P.j];
            if (lane < n && lane != xpos) {
                const int pos = (xpos >= 0 && lane > xpos) ? lane - 1 : lane;
                if (pos < Fj) out[pos] = id;
            }
            const int got = min(Fj, n - (xpos >= 0 ? 1 : 0));
            for (int x = got + lane; x < Fj; x += kWave) out[x] = -1;
        }
    }
    if (threadIdx.x == 0 && P.j < a.K && f.uniform && (a.flags & SPEC_SAMPLE_DRAFT))
        a.tokens[(size_t)P.b * a.K + P.j] = s_tok;  // the drawn backup token is an output
    if (threadIdx.x == 0) {
        sm.unit_code = unit_code(accept, fallback, status);
        UnitFast* U = reinterpret_cast<UnitFast*>(f.ws + f.L.units) + unit;
        U->accept = accept;
        U->status = status;
        U->fallback = fallback;
        U->u_res = param_ok ? sm.u_res : 0.0;  // (no draws for a request with bad parameters)
        if (param_ok) {
            for (int r = 0; r < (two ? 2 : 1); ++r) {
                const RowView& rv = us.rv[r];
                RowFinal rf;
                rf.m = rv.m;
                rf.invT = rv.invT;
                rf.S = rv.S;
                rf.C = rv.C;
                rf.Z = rv.Z;
                rf.kk = rv.has_k ? rv.ck.key : 0u;
                rf.kp = rv.has_p ? rv.cp.key : 0u;
                rf.kF = rv.kF;
                rf.idF = rv.idF;
                rf.nS = rv.nset;
                rf.argmax = rv.argmax;
                rf.greedy = rv.greedy;
                rf.has_special = rv.has_special;
                if (r == 0) U->rq = rf;
                else U->rp = rf;
                const Cut* cs[2] = {&rv.ck, &rv.cp};
                const int on[2] = {rv.has_k, rv.has_p};
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    UnitCut uc;
                    uc.key = on[c] ? cs[c]->key : 0u;
                    uc.explicit_id = cs[c]->explicit_id;
                    uc.owner = cs[c]->explicit_id >= 0 ? cs[c]->explicit_id / kSliceCols : cs[c]->owner;
                    uc.owner_take = cs[c]->owner_take;
                    U->cut[r][c] = uc;
                }
            }
        }
    }
}

// The last unit of a request, from the units' codes gathered by the rendezvous atomic: k, the
// status, and the outputs when no residual is needed (thread 0; one load for a greedy
// request's argmax).
__device__ __forceinline__ void decide_packed(const FastArgs& f, int b, uint64_t word, bool greedy) {
    const VerifyArgs& a = f.a;
    const int K = a.K;
    bool any_fb = false;
    uint32_t any = 0, deg = 0;
    int k = K;
    for (int j = 0; j <= K; ++j) {
        const uint32_t c = (uint32_t)(word >> (kCountBits + kCodeBits * j)) & 0x7Fu;
        any_fb |= (c & 2u) != 0;
        any |= ((c & 4u) ? kStBadParam : 0u) | ((c & 8u) ? kStBadLogit : 0u) | ((c & 16u) ? kStBadToken : 0u);
        if (j < K) {
            if (c & 32u) deg = kStDegenerate;
            if (k == K && !(c & 1u)) k = j;
        }
    }
    uint32_t outside = 0;
    for (int j = 0; j < K && j <= k; ++j)
        if ((word >> (kCountBits + kCodeBits * j)) & 64u) outside = kStOutside;
    ReqFast* R = reinterpret_cast<ReqFast*>(f.ws + f.L.reqs) + b;
    // set by a unit whose slices were misplaced (which also sends the request to the general path)
    const uint32_t place = any_fb ? (uint32_t)ldnt(&R->pad) : 0u;
    int mode = 0, t = -1, kk = 0;
    uint32_t status;
    if (any_fb) {
        mode = 2;
        status = place;  // the general path reports the rest
    } else if (any & kStBadParam) {
        status = kStBadParam;
    } else if (any & kStBadLogit) {
        status = kStBadLogit;
    } else if (any & kStBadToken) {
        status = deg | kStBadToken;
    } else if (a.tau) {
        // fuzzy acceptance: the divergence kernel decides (greedy rows: the general path)
        mode = greedy ? 2 : 3;
        status = 0;
    } else {
        status = deg | outside;
        kk = k;
        if (greedy) {
            const UnitFast* U = reinterpret_cast<const UnitFast*>(f.ws + f.L.units) + (size_t)b * (K + 1) + k;
            t = ldnt(&U->rq.argmax);
        } else {
            mode = 1;
        }
    }
    R->mode = mode;
    R->k = kk;
    R->status = status;
    R->pad = 0;
    if (mode == 0) {
        a.out_k[b] = kk;
        a.out_t[b] = t;
        if (a.out_W) a.out_W[b] = 0.0f;
        if (a.out_status) a.out_status[b] = status;
    }
}

// The last unit of a request: k, the status, and the outputs when no residual is needed.
__device__ __forceinline__ void decide_request(const FastArgs& f, int b) {
    const VerifyArgs& a = f.a;
    const int K = a.K;
    const UnitFast* U = reinterpret_cast<const UnitFast*>(f.ws + f.L.units) + (size_t)b * (K + 1);
    const int lane = threadIdx.x & (kWave - 1);
    if (threadIdx.x >= kWave) return;
    uint32_t st = 0;
    int acc = 1, fb = 0;
    if (lane <= K) {
        st = ldnt(&U[lane].status);
        acc = ldnt(&U[lane].accept);
        fb = ldnt(&U[lane].fallback);
    }
    const bool any_fb = __ballot(fb != 0) != 0;
    const uint32_t any = wave_or(st);
    const uint32_t deg = wave_or(lane < K ? (st & kStDegenerate) : 0u);
    int k = first_lane(__ballot(lane < K && !acc));
    if (k < 0) k = K;
    const uint32_t outside = wave_or((lane < K && lane <= k) ? (st & kStOutside) : 0u);
    ReqFast* R = reinterpret_cast<ReqFast*>(f.ws + f.L.reqs) + b;
    // set by a unit whose slices were misplaced (which also sends the request to the general path)
    const uint32_t place = any_fb ? (uint32_t)ldnt(&R->pad) : 0u;
    int mode = 0, t = -1, kk = 0;
    uint32_t status;
    if (any_fb) {
        mode = 2;
        status = place;  // the general path reports the rest
    } else if (any & kStBadParam) {
        status = kStBadParam;
    } else if (any & kStBadLogit) {
        status = kStBadLogit;
    } else if (any & kStBadToken) {
        status = deg | kStBadToken;
    } else if (a.tau) {
        // fuzzy acceptance: the divergence kernel decides (greedy rows: the general path)
        mode = ldnt(&U[k].rq.greedy) ? 2 : 3;
        status = 0;
    } else {
        status = deg | outside;
        kk = k;
        if (ldnt(&U[k].rq.greedy)) t = ldnt(&U[k].rq.argmax);
        else mode = 1;
    }
    if (lane == 0) {
        R->mode = mode;
        R->k = kk;
        R->status = status;
        R->pad = 0;
        if (mode == 0) {
            a.out_k[b] = kk;
            a.out_t[b] = t;
            if (a.out_W) a.out_W[b] = 0.0f;
            if (a.out_status) a.out_status[b] = status;
        }
    }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(6, 8))) void fast_count_kernel(FastArgs f) {
    __shared__ CountSmem sm;
    const VerifyArgs& a = f.a;
    if (blockIdx.x == 0 && threadIdx.x == 0 && f.lookup && f.out_batch) {
        f.out_batch[0] = 0;  // the fused lookup's batch hit count and all-hit flag, which the
        f.out_batch[1] = 1;  // resolve kernel's requests add into
    }
    const Place P = place_of(f);
    if (P.b >= a.B) return;
    // when the whole grid is resident at once, slices issue ahead of the settle steps that
    // share their CU (see the settle below)
    if (f.slice_prio) __builtin_amdgcn_s_setprio(1);
    const int j = P.j, slice = P.slice, unit = P.unit;
    const int c0 = slice * kSliceCols;
    // the draft row of position j: verified (j < K) or, at the bonus position, only listed for
    // the outcome cache
    // (uniform: kept in a scalar register)
    const bool two = __builtin_amdgcn_readfirstlane((!f.uniform && (j < a.K || (f.cache && f.fan.f[j] > 0))) ? 1 : 0) != 0;
    const spec_params prm = a.params[P.b];
    const bool param_ok = params_ok(prm);
    const size_t stride = (size_t)a.V;
    const uint16_t* trow = static_cast<const uint16_t*>(a.target) + ((size_t)P.b * (a.K + 1) + j) * stride;
    const uint16_t* drow = two ? static_cast<const uint16_t*>(a.draft) + ((size_t)P.b * a.draft_rows + j) * stride : nullptr;
    // (the backup speculator's tokens are drawn here: every workgroup of the unit draws the same)
    const bool draw = f.uniform && (a.flags & SPEC_SAMPLE_DRAFT);
    const int s_tok = j < a.K ? (draw ? uniform_draft_token(a.seed, a.round, P.b, j, a.V) : a.tokens[(size_t)P.b * a.K + j])
                              : -1;
    const bool tok_ok = j == a.K || (s_tok >= 0 && s_tok < a.V);

    // the draws of position j (acceptance, residual / bonus: words 0 and 1 of one Philox
    // block), in the shadow of the first loads (wave 1 only), kept in LDS for the settle step
    if (param_ok) {  // (a request with bad parameters is reported without its summaries)
        // (without a draft row the second set re-reads the target and goes unused: unconditional
        // loads keep the compiler's waits exact)
        u32x4 vq[kLoads], vp[kLoads];
        load_slice<true>(trow, c0, a.V, vq);
        load_slice<true>(two ? drow : trow, c0, a.V, vp);
        if (threadIdx.x / kWave == 1) {
            const Block4 x = philox4x64_10(a.round, (uint64_t)P.b, (uint64_t)j, 0, a.seed, 0);
            if (threadIdx.x == kWave) {
                sm.u_acc = word_to_uniform(x.w[0]);
                sm.u_res = word_to_uniform(x.w[1]);
            }
        }
        for (int i = threadIdx.x; i < 2 * kHistRow / 4; i += blockDim.x)
            reinterpret_cast<u32x4*>(&sm.hraw[0][0])[i] = u32x4{0, 0, 0, 0};
        if (threadIdx.x < 2) {
            sm.n_sp[threadIdx.x] = 0;
            sm.flags[threadIdx.x] = 0;
            sm.neginf[threadIdx.x] = 0;
            sm.cnt_s[threadIdx.x] = 0;
            sm.th_tau[threadIdx.x] = 0u;
            sm.th_need[threadIdx.x] = 0;
            sm.th_ties[threadIdx.x] = 0;
        }
        if (threadIdx.x == 2) sm.xcc = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xFu;  // XCC_ID
        // the rows' values at the draft token (every slice counts the token's key), zero without
        // a token: loaded after the slice, stored once the counts have waited for it anyway
        uint32_t sb0 = 0u, sb1 = 0u;
        if (threadIdx.x == kWave && j < a.K && tok_ok) {
            sb0 = trow[s_tok];
            sb1 = two ? drow[s_tok] : 0u;  // (no draft row with the uniform draft)
        }
        __syncthreads();
        count_row(sm, 0, c0, a.V, vq);
        if (two) count_row(sm, 1, c0, a.V, vp);
        if (threadIdx.x == kWave) {
            sm.s_bits[0] = sb0;
            sm.s_bits[1] = sb1;
        }
        __syncthreads();
        const bool rare0 = (sm.hraw[0][kHistLead - 1] | sm.hraw[0][kHistLead + kBins]) != 0;
        const bool rare1 = two && (sm.hraw[1][kHistLead - 1] | sm.hraw[1][kHistLead + kBins]) != 0;
        if (rare0) count_rare(sm, 0, c0, a.V, vq);
        if (rare1) count_rare(sm, 1, c0, a.V, vp);
        if (threadIdx.x < 2) sm.rare[threadIdx.x] = threadIdx.x == 0 ? rare0 : rare1;  // (read after later barriers)
        if (rare0 || rare1) __syncthreads();  // the second pass's counts and specials
        // the summaries; passes over the columns (registers) while they are still live
        const bool holds_s = j < a.K && tok_ok && s_tok >= c0;  // at or after this slice: count its key
        const int want[2] = {list_len(a, prm, false), two ? draft_list_len(f, prm, j) : 0};
        // rows with values outside the bins find their candidate threshold from segment counts
        const bool slow[2] = {want[0] > 0 && sm.n_sp[0] > 0u, want[1] > 0 && sm.n_sp[1] > 0u};
        const bool fast[2] = {!slow[0], !slow[1]};
        int n_top[2] = {0, 0};
        const uint32_t ent_pos = scan_entries(sm, two, want, fast);
        if (slow[0] || slow[1]) seg_counts(sm, two ? 2 : 1);
        if (holds_s) local_ranks(sm, two, c0, s_tok, vq, vp);
        __syncthreads();
        if (want[0] > 0 || want[1] > 0) local_tops(f, sm, unit, slice, want, slow, c0, a.V, vq, vp, n_top);
        write_entries(f, sm, unit, slice, two, ent_pos);
        publish_header(f, sm, unit, slice, two, n_top);
    }

    // ---- unit rendezvous: the last slice of the unit settles it ----
    drain_stores();
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned* uc = reinterpret_cast<unsigned*>(f.ws + f.L.unit_ctr + (size_t)unit * 128);
        const unsigned old = l2_fetch_add(uc, 1u);
        sm.last = (old + 1 == (unsigned)f.nS) ? 1 : 0;
        if (sm.last) *uc = 0u;  // every slice has arrived: ready for the next call
    }
    __syncthreads();
    if (!sm.last) return;
    // The settling workgroup is the unit's last slice to arrive.  With the whole grid resident
    // (one round of workgroups), the call ends with the last unit's settle, which starts when
    // that unit's last slice arrives: slices then issue ahead of settles, so the last ones
    // arrive sooner (measured on the B = 16, K = 5, V = 128256 call: 58.9 -> 57.0 us).  Over
    // several rounds the work is throughput-bound and a slower settle holds its slot longer
    // (measured 4% slower on 512 chains at V = 151936), so there all waves keep one priority.
    if (f.slice_prio) __builtin_amdgcn_s_setprio(0);
    settle_unit(f, sm, P, prm, param_ok, two, s_tok, tok_ok);

    // ---- request rendezvous: the last unit of the request decides k ----
    drain_stores();
    __syncthreads();
    if (a.K + 1 <= kPackedUnits) {
        // the arrival count and every unit's code in one 64-bit word: the last arriver decides
        // from the atomic's result alone
        if (threadIdx.x == 0) {
            uint64_t* rc = reinterpret_cast<uint64_t*>(f.ws + f.L.req_ctr + (size_t)P.b * 128);
            const uint64_t add = 1ull + ((uint64_t)sm.unit_code << (kCountBits + kCodeBits * P.j));
            const uint64_t now = l2_fetch_add64(rc, add) + add;
            if ((now & ((1ull << kCountBits) - 1ull)) == (uint64_t)(a.K + 1)) {
                *rc = 0ull;  // every unit has arrived: ready for the next call
                decide_packed(f, P.b, now, prm.temperature == 0.0f);
            }
        }
        return;
    }
    if (threadIdx.x == 0) {
        unsigned* rc = reinterpret_cast<unsigned*>(f.ws + f.L.req_ctr + (size_t)P.b * 128);
        const unsigned old = l2_fetch_add(rc, 1u);
        sm.last = (old + 1 == (unsigned)(a.K + 1)) ? 1 : 0;
        if (sm.last) *rc = 0u;
    }
    __syncthreads();
    if (sm.last) decide_request(f, P.b);
}

int count_resident() {
    // per device, worked out once (0 until then; a failed query counts as not resident)
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fast_count_kernel, kThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu <= 0 || cus <= 0)
        return 0;
    v = per_cu * cus;
    cached[dev].store(v, std::memory_order_relaxed);
    return v;
}

void launch_count(const FastArgs& f, int grid, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    if (start || stop)  // (the events bound the kernel's own execution)
        hipExtLaunchKernelGGL(fast_count_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, start, stop, 0u, f);
    else
        hipLaunchKernelGGL(fast_count_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, f);
}

}  // namespace fast
}  // namespace sv
