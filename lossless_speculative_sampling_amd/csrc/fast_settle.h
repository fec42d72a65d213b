// Settling one (request, position) unit from its slices' summaries: the exact processed
// distributions of the target and draft rows (temperature, top-k, softmax, nucleus; DeepMind
// speculative-sampling page, section 6), the Saguaro downweighted set of the draft row (SSD
// reading notes, section 4.4), and the processed probabilities of the drafted token that the
// acceptance test compares.  Run by the last slice of a unit to finish counting.
//
// Every slice publishes its occupied bins as (bin, count) entries.  The settle step adds them
// into one histogram per row, then walks the row's values in descending order once: counts
// give the maximum and the top-k cut, one fp64 exp per occupied bin gives the masses, the
// nucleus cut and the normaliser.  The slices' entries at a cut bin say which slice holds the
// cut's last kept element (its owner) for the resolve kernel.
#pragma once

#include "fast_common.h"

namespace sv {
namespace fast {

// ------------------------------------------------------------------------------------------
// Scan slots: every exact bin and the four groups of finite values outside the bins, in
// descending key order.  Slot 0 holds the huge positive values (>= 32), slots 1..1408 the
// positive bins from the top, 1409 the tiny positive values (below 2^-6), 1410 zero, 1411 the
// tiny negative values, 1412..2819 the negative bins from -2^-6 down, 2820 the huge negative.
// ------------------------------------------------------------------------------------------
constexpr int kSlotHP = 0, kSlotTP = 1 + kNegBins, kSlotZero = kSlotTP + 1, kSlotTN = kSlotZero + 1;
constexpr int kSlotHN = kSlotTN + 1 + kNegBins, kSlots = kSlotHN + 1;  // 2820, 2821
constexpr int kRowThreads = kThreads / 2;                            // a row's share of the workgroup
constexpr int kSlotsPer = (kSlots + kRowThreads - 1) / kRowThreads;    // 12 consecutive slots per thread
static_assert(kSlotsPer * kRowThreads >= kSlots, "slots covered");
constexpr int kSpMerge = 256;   // specials of one row merged in LDS (more: the general path)
constexpr int kEntIt = 8;       // sparse entries each thread loads with the headers
constexpr int kNone = 0x7FFFFFFF;

__device__ __forceinline__ int slot_bin(int s) {
    if (s >= 1 && s < kSlotTP) return kBins - s;            // 2879 .. 1472
    if (s == kSlotZero) return kZeroBin;
    if (s > kSlotTN && s < kSlotHN) return kSlotHN - 1 - s;  // 1407 .. 0
    return -1;
}
// aggregate index of a slot of specials: 0 huge positive, 1 tiny positive, 2 tiny negative,
// 3 huge negative; -1 for a bin
__device__ __forceinline__ int slot_agg(int s) {
    return s == kSlotHP ? 0 : s == kSlotTP ? 1 : s == kSlotTN ? 2 : s == kSlotHN ? 3 : -1;
}
__device__ __forceinline__ int agg_of_key(uint32_t k) {
    const int sg = special_seg(k);
    return sg == kSegHugePos ? 0 : sg == kSegTinyPos ? 1 : sg == kSegTinyNeg ? 2 : 3;
}

struct Cut {       // a cut in token order: keep key > key, and the first `take` elements at key
    uint32_t key;     // 0: no cut
    int take;
    int explicit_id;  // >= 0: explicit cut, the id of the last kept element at `key` (unused here)
    int owner;        // slice holding the last kept element at `key`
    int owner_take;   // elements at `key` that slice keeps
    int count_above;  // elements with a larger key
    int slot;         // scan slot of `key`
};

struct RowView {   // the settled view of one row
    int bad, overflow, greedy, argmax;
    float m;
    double invT;               // 1 / temperature
    int has_k, has_p;
    Cut ck, cp;
    uint32_t n_finite;
    int has_special;
    int nm;                    // merged candidates (okey / oid)
    double S_kept, S;
    int n_kept, n_nuc;
    int nset;                  // downweighted set size (0: off)
    uint32_t kF;
    int idF;
    double C, Z;
    int degenerate;
    uint32_t s_bits;           // the drafted token's value, its mass and its rank among the
    double e_s;                // elements with its key (token order)
    int rank_s;
    uint32_t xcc_bad;          // slices of the unit ran on different XCDs
};

struct SettleSmem {
    RowView rv[2];
    uint32_t hdr[2][kMaxSlices][8];   // each slice's header words
    uint32_t okey[2][kTop];           // merged candidates in token order
    int32_t oid[2][kTop];
    uint32_t spk[2][kSpMerge];        // every slice's specials of a row
    int32_t spi[2][kSpMerge];
    uint32_t n_spm[2];
    uint32_t agg_n[2][4];             // specials per aggregate slot: count, largest key, mass
    uint32_t agg_key[2][4];
    double agg_m[2][4];
    uint32_t pc[2][2][kMaxSlices];    // per-slice counts at the top-k / nucleus cut bins
    uint32_t wu[2][4];                // per-row wave partials
    double wd[2][4];
    int wi[2][4];
    int list_start[2][kMaxSlices];
    int cross[2];     // the thread of a row whose run holds the nucleus cut
    double xbase[kThreads];    // each thread's mass and kept count before its run (the crossing
    uint32_t xcbase[kThreads]; // thread reads its own after a barrier, out of registers)
    double qs, ps;                    // the drafted token's processed probabilities
};

// Candidate lists of every slice, staged for the merge (laid over the histogram rows).
struct StageSmem {
    uint32_t key[2][kMergeCap];
    int32_t id[2][kMergeCap];
};

// e^x for the masses of the settle step (x <= 0 there), written for a small register
// footprint: x = k ln 2 + r with |r| <= ln(2) / 2 (ln 2 split in a 31-bit head and a tail, so
// k times the head is exact), e^r by its Taylor series to degree 13 (the next term is below
// 1e-17) in Horner form, then scaled by 2^k.  Relative error within a few ulp of e^x.  The
// constants sit in constant memory and reach the arithmetic through scalar loads.
__constant__ double kExpConst[17] = {
    1.4426950408889634,    // 1 / ln 2
    0.6931471803691238,    // ln 2, head
    1.9082149292705877e-10,  // ln 2, tail
    1.6059043836821613e-10, 2.08767569878681e-09, 2.505210838544172e-08, 2.755731922398589e-07,
    2.7557319223985893e-06, 2.48015873015873e-05, 0.0001984126984126984, 0.001388888888888889,
    0.008333333333333333, 0.041666666666666664, 0.16666666666666666, 0.5, 1.0, 1.0};  // 1/13!, ..., 1/0!
__device__ __forceinline__ double exp_mass(double x) {
    if (x < -745.0) return 0.0;
    const double k = rint(x * kExpConst[0]);
    double r = fma(-k, kExpConst[1], x);
    r = fma(-k, kExpConst[2], r);
    double p = kExpConst[3];
#pragma unroll
    for (int c = 4; c < 17; ++c) p = fma(p, r, kExpConst[c]);
    return ldexp(p, (int)k);
}
__device__ __forceinline__ double mass_lean(float z, float m, double invT) {
    return exp_mass(((double)z - (double)m) * invT);
}

// Bin of an order key in the exact range (or zero), computed directly.
__device__ __forceinline__ int bin_of_key(uint32_t k) {
    const uint32_t h = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
    const uint32_t mag = h & 0x7FFFu;
    if (mag == 0u) return kZeroBin;
    const int off = (int)mag - (kExpLo << 7);
    return (h & 0x8000u) ? (kNegBins - 1 - off) : (kPosBase + off);
}

// (row, slice) of a row-major index rt < 2 nS without a division (a row count of at most 2)
__device__ __forceinline__ void row_slice(int rt, int nS, int* r, int* t) {
    *r = rt >= nS ? 1 : 0;
    *t = rt - *r * nS;
}

__device__ __forceinline__ const RowPart* part_c(const FastArgs& f, int unit, int slice, int r) {
    return reinterpret_cast<const RowPart*>(f.ws + f.L.parts) + ((size_t)unit * f.nS + slice) * 2 + r;
}
// The same record for a wave-uniform (row, slice), its address kept in scalar registers.
__device__ __forceinline__ const RowPart* part_u(const FastArgs& f, int unit, int slice, int r) {
    const uint64_t pa = reinterpret_cast<uint64_t>(part_c(f, unit, slice, r));
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)pa), hi = __builtin_amdgcn_readfirstlane((uint32_t)(pa >> 32));
    return reinterpret_cast<const RowPart*>(((uint64_t)hi << 32) | lo);
}

// Exclusive prefix over the 256 threads of row r in thread order (wave w of the row, lane);
// *inc gets the inclusive value and *total the row's sum.  Every thread of the workgroup calls
// it (one barrier); exc of thread u + 1 equals inc of thread u bit for bit.
template <typename T>
__device__ __forceinline__ T row_scan(T v, T (*wtot)[4], T* inc, T* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int r = threadIdx.x / kRowThreads, w = (threadIdx.x % kRowThreads) / kWave;
    T exc;
    const T in = wave_scan(v, &exc);
    if (lane == kWave - 1) wtot[r][w] = in;
    __syncthreads();
    T before = T(0), all = T(0);
    for (int x = 0; x < 4; ++x) {
        const T t = wtot[r][x];
        if (x < w) before += t;
        all += t;
    }
    *total = all;
    *inc = before + in;
    return before + exc;
}

__device__ __forceinline__ int row_min(int v, int (*wtot)[4]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int r = threadIdx.x / kRowThreads, w = (threadIdx.x % kRowThreads) / kWave;
    v = wave_min(v);
    if (lane == 0) wtot[r][w] = v;
    __syncthreads();
    return min(min(wtot[r][0], wtot[r][1]), min(wtot[r][2], wtot[r][3]));
}

__device__ __forceinline__ bool cut_keeps_s(const RowView& rv, const Cut& c, uint32_t key_s) {
    if (key_s > c.key) return true;
    if (key_s < c.key) return false;
    return rv.rank_s < c.take;
}

// Processed probability of the drafted token s in row r (after the settle).
__device__ __forceinline__ double prob_of_s(const SettleSmem& ss, int r, int s, bool draft) {
    const RowView& rv = ss.rv[r];
    const uint32_t h = rv.s_bits;
    if ((h & 0x7FFFu) >= 0x7F80u) return 0.0;
    const uint32_t key = key16(h);
    if (rv.has_k && !cut_keeps_s(rv, rv.ck, key)) return 0.0;
    if (rv.has_p && !cut_keeps_s(rv, rv.cp, key)) return 0.0;
    const double e = rv.e_s;
    const double p = e / rv.S;
    if (!draft) return p;
    const double fct = (rv.nset > 0 && e > 0.0 && in_cut_id(rv.kF, rv.idF, key, s)) ? rv.C : 1.0;
    return (p * fct) / rv.Z;
}

// Merges the slices' candidate lists of both rows (staged in st, slice-major) into ss.okey /
// ss.oid in token order (key desc, id asc), keeping the first want[r]; all threads.
__device__ __forceinline__ void merge_candidates(SettleSmem& ss, const StageSmem& st, int nS, int rows, int want0,
                                                 int want1) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    // (two scalars per row, selected by row: indexed private arrays would live in scratch memory)
    int total0 = 0, total1 = 0;
    for (int t = 0; t < nS; ++t) {
        total0 += (int)ss.hdr[0][t][3];
        total1 += rows > 1 ? (int)ss.hdr[1][t][3] : 0;
    }
    if (want0 <= 0) total0 = 0;
    if (want1 <= 0) total1 = 0;
#define WANT_OF(r) ((r) ? want1 : want0)
#define TOTAL_OF(r) ((r) ? total1 : total0)
    // up to 64 candidates of a row: wave r holds one per lane and ranks each against all
    // others through lane reads
    if (wave < rows && WANT_OF(wave) > 0 && TOTAL_OF(wave) <= kWave) {
        const int r = wave;
        int t = 0, x = lane;
        for (int u = 0; u < nS; ++u) {
            const int stt = ss.list_start[r][u];
            if (lane >= stt) {
                t = u;
                x = lane - stt;
            }
        }
        const bool live = lane < TOTAL_OF(r);
        const uint32_t k = live ? st.key[r][t * kTop + x] : 0u;
        const int32_t id = live ? st.id[r][t * kTop + x] : 0;
        const uint64_t ord = ((uint64_t)k << 32) | (uint32_t)~id;  // token order (ids are non-negative)
        int rank = 0;
        for (int y = 0; y < TOTAL_OF(r); y += 4) {
#pragma unroll
            for (int d = 0; d < 4; ++d) rank += wave_bcast(ord, y + d) > ord ? 1 : 0;
        }
        if (live && rank < WANT_OF(r)) {
            ss.okey[r][rank] = k;
            ss.oid[r][rank] = id;
        }
    }
    // more (long lists: top candidates of many slices): the rank of every entry is its position
    // in its own list plus a binary search in every other list of its row
    if (total0 > kWave || total1 > kWave) {
#pragma unroll 1
        for (int i = threadIdx.x; i < 2 * nS * kTop; i += blockDim.x) {
            const int r = i / (nS * kTop), t = (i / kTop) % nS, x = i % kTop;
            if (r >= rows || WANT_OF(r) <= 0 || TOTAL_OF(r) <= kWave || x >= (int)ss.hdr[r][t][3]) continue;
            const uint32_t k = st.key[r][t * kTop + x];
            const int32_t id = st.id[r][t * kTop + x];
            const uint64_t ord = ((uint64_t)k << 32) | (uint32_t)~id;
            int rank = x;
#pragma unroll 1
            for (int t2 = 0; t2 < nS; ++t2) {
                const int n = t2 == t ? 0 : (int)ss.hdr[r][t2][3];
                int lo = 0, hi = n;  // entries of list t2 before `ord` in token order: [0, lo)
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    const int e = t2 * kTop + mid;
                    const uint64_t o2 = ((uint64_t)st.key[r][e] << 32) | (uint32_t)~st.id[r][e];
                    if (o2 > ord) lo = mid + 1;
                    else hi = mid;
                }
                rank += lo;
            }
            if (rank < WANT_OF(r)) {
                ss.okey[r][rank] = k;
                ss.oid[r][rank] = id;
            }
        }
    }
    if (threadIdx.x < (unsigned)rows) ss.rv[threadIdx.x].nm = min(TOTAL_OF(threadIdx.x), WANT_OF(threadIdx.x));
#undef WANT_OF
#undef TOTAL_OF
}

// One thread's run of kSlotsPer consecutive slots of a row, in descending key order: the weight
// of each slot is its kept count times the per-element mass exp((z - m) / T) (an aggregate of
// specials carries its summed mass).  Every mass is the same function of (z - m) / T, so rows
// that differ by a constant shift get bit-identical masses.  The run's counts are read in one
// batch (each LDS read can queue behind other workgroups' histogram atomics).  With PICK the
// sweep stops at the first slot whose weight takes the running mass from base to `need`
// (need >= 0) or at slot `target`, and reports it.
struct Pick {
    int i;               // slot index in the run (-1: none)
    double above, e, w;  // mass before it, its per-element mass, its weight
    uint32_t cabove, n;  // kept elements before it, kept elements in it
};
template <bool PICK>
__device__ __forceinline__ double sweep_run(const uint32_t* hist_r, const uint32_t* agg_n_r, const double* agg_m_r, int s0,
                                            float m, double invT, int ks, uint32_t take_k, double base, uint32_t cbase,
                                            double need, int target, int* last, Pick* pk) {
    uint32_t c[kSlotsPer];
#pragma unroll
    for (int i = 0; i < kSlotsPer; ++i) {
        const int s = s0 + i;
        const int b = slot_bin(s);
        c[i] = s >= kSlots ? 0u : (b >= 0 ? hist_r[b] : agg_n_r[slot_agg(s)]);
    }
    double cum = base;
    uint32_t ccum = cbase;
    if (PICK) pk->i = -1;
    *last = -1;
#pragma unroll 1
    for (int i = 0; i < kSlotsPer; ++i) {
        const int s = s0 + i;
        if (s >= kSlots || s > ks) break;
        if (c[i] == 0u) continue;
        const int b = slot_bin(s);
        uint32_t n;
        double e = 0.0, w;
        if (b < 0) {
            n = c[i];
            w = agg_m_r[slot_agg(s)];
        } else {
            e = mass_lean(key16_value(bin_key(b)), m, invT);
            n = s == ks ? take_k : c[i];
            w = (double)n * e;
        }
        *last = i;
        if (PICK && ((need >= 0.0 && w > 0.0 && cum + w >= need) || s == target)) {
            *pk = Pick{i, cum, e, w, ccum, n};
            break;
        }
        cum += w;
        ccum += n;
    }
    return cum - base;
}

// ------------------------------------------------------------------------------------------
// The settle step: both rows' processed distributions (maxima, normalisers, top-k and nucleus
// cuts with their owner slices), the draft row's downweighted set (dw) and the drafted token's
// processed probabilities.  All threads; hist(r) of the caller is free LDS (the slice's own
// histograms are published by now) and holds the merged histograms.
// ------------------------------------------------------------------------------------------
template <typename Smem>
__device__ __forceinline__ void settle_rows(const FastArgs& f, Smem& sm, int unit, int j, int rows,
                                            const spec_params& prm, bool dw, int s_tok) {
    const VerifyArgs& a = f.a;
    SettleSmem& ss = sm.ss;
    StageSmem& st = *reinterpret_cast<StageSmem*>(&sm.hraw[0][0]);
    const int nS = f.nS;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int want0 = list_len(a, prm, false);
    const int want1 = rows > 1 ? draft_list_len(f, prm, j) : 0;
    // entries each (row, slice) loads with the headers: a power of two, at most kEntIt * kThreads
    // in all and never past a record's kBins entries
    int lg = 0;
    while ((2 << lg) * rows * nS <= kEntIt * kThreads && (2 << lg) <= kBins) ++lg;
    const int per = 1 << lg;

    // ---- round trip 1: headers, the first `per` entries of every slice, candidate lists ----
    u32x4 hw = {0u, 0u, 0u, 0u};
    const bool hload = tid < rows * nS * 2;
    if (hload) {
        int r, t;
        row_slice(tid >> 1, nS, &r, &t);
        hw = ldnt(reinterpret_cast<const u32x4*>(part_c(f, unit, t, r)) + (tid & 1));
    }
    uint32_t ent[kEntIt];
#pragma unroll
    for (int it = 0; it < kEntIt; ++it) {
        const int i = tid + it * kThreads;
        const int rt = i >> lg;
        ent[it] = 0u;
        if (rt < rows * nS) {
            int r, t;
            row_slice(rt, nS, &r, &t);
            ent[it] = ldnt(&part_c(f, unit, t, r)->ent[i & (per - 1)]);
        }
    }
    constexpr int kCandLoads = 2 * kMaxSlices * kTop / kThreads;  // 4
    uint32_t ck_[kCandLoads];
    int32_t ci_[kCandLoads];
#pragma unroll
    for (int it = 0; it < kCandLoads; ++it) {
        const int i = tid + it * kThreads;
        const int r = i >> 10, t = (i >> 6) & (kMaxSlices - 1), x = i & (kTop - 1);
        ck_[it] = 0u;
        ci_[it] = 0;
        if (r < rows && t < nS && x < (r ? want1 : want0)) {
            const RowPart* P = part_c(f, unit, t, r);
            ck_[it] = ldnt(&P->top_key[x]);
            ci_[it] = ldnt(&P->top_id[x]);
        }
    }
    if (tid < 2) {
        ss.n_spm[tid] = 0u;
        ss.cross[tid] = kNone;
    }
    if (tid < 8) {
        ss.agg_n[tid >> 2][tid & 3] = 0u;
        ss.agg_key[tid >> 2][tid & 3] = 0u;
        ss.agg_m[tid >> 2][tid & 3] = 0.0;
    }
    if (tid < 2 * 2 * kMaxSlices) (&ss.pc[0][0][0])[tid] = 0u;
    if (hload) {
        int r, t;
        row_slice(tid >> 1, nS, &r, &t);
        const int w = tid & 1;
#pragma unroll
        for (int x = 0; x < 4; ++x) ss.hdr[r][t][4 * w + x] = hw[x];
    }
    __syncthreads();
    // ---- per-row flags from the headers; candidate list offsets (wave r) ----
    if (wave < rows) {
        const int r = wave;
        RowView& rv = ss.rv[r];
        const bool lv = lane < nS;
        const uint32_t fl = lv ? ss.hdr[r][lane][0] : 0u;
        const uint32_t nsp = lv ? ss.hdr[r][lane][2] : 0u;
        const uint32_t ntop = lv ? ss.hdr[r][lane][3] : 0u;
        const uint32_t cnt = lv ? ss.hdr[r][lane][4] : 0u;
        const uint32_t xcc = lv ? ss.hdr[r][lane][7] : ss.hdr[r][0][7];
        const uint32_t flo = wave_or(fl);
        int ls;
        wave_scan((int)ntop, &ls);
        if (lv) ss.list_start[r][lane] = ls;
        const int rank = (int)wave_sum(cnt);
        const uint32_t nsp_all = wave_sum(nsp);
        const bool xbad = __ballot(xcc != ss.hdr[r][0][7]) != 0;
        if (lane == 0) {
            rv.invT = inv_temperature(prm.temperature);
            rv.greedy = prm.temperature == 0.0f ? 1 : 0;
            rv.argmax = -1;
            rv.has_k = (prm.top_k > 0 && prm.top_k < a.V) ? 1 : 0;
            rv.has_p = ((double)prm.top_p < 1.0) ? 1 : 0;
            rv.ck = Cut{0u, 0, -1, 0, 0, 0, kNone};
            rv.cp = Cut{0u, 0, -1, 0, 0, 0, kNone};
            rv.nset = 0;
            rv.kF = 0xFFFFFFFFu;
            rv.idF = -1;
            rv.C = 1.0;
            rv.Z = 1.0;
            rv.degenerate = 0;
            rv.bad = (flo & 1u) ? 1 : 0;
            rv.overflow = ((flo & 2u) || nsp_all > (uint32_t)kSpMerge) ? 1 : 0;
            rv.has_special = nsp_all > 0u ? 1 : 0;
            rv.s_bits = ss.hdr[r][0][5];
            rv.rank_s = rank;
            rv.xcc_bad = xbad ? 1u : 0u;
            rv.e_s = 0.0;
        }
    }
    // ---- candidates to the stage, then merged ----
#pragma unroll
    for (int it = 0; it < kCandLoads; ++it) {
        const int i = tid + it * kThreads;
        const int r = i >> 10, t = (i >> 6) & (kMaxSlices - 1), x = i & (kTop - 1);
        if (r < rows && t < nS && x < (int)ss.hdr[r][t][3] && x < (r ? want1 : want0)) {
            st.key[r][t * kTop + x] = ck_[it];
            st.id[r][t * kTop + x] = ci_[it];
        }
    }
    __syncthreads();
    merge_candidates(ss, st, nS, rows, want0, want1);
    __syncthreads();
    // ---- the merged histograms: zero, then every slice's entries; the rows' specials ----
    for (int i = tid; i < rows * kHistRow / 4; i += kThreads)
        reinterpret_cast<u32x4*>(&sm.hraw[0][0])[i] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kEntIt; ++it) {
        const int i = tid + it * kThreads;
        const int rt = i >> lg;
        if (rt < rows * nS) {
            int r, t;
            row_slice(rt, nS, &r, &t);
            if ((i & (per - 1)) < (int)ss.hdr[r][t][1]) atomicAdd(&sm.hist(r)[ent[it] >> 16], ent[it] & 0xFFFFu);
        }
    }
    for (int rt = 0; rt < rows * nS; ++rt) {  // entries past the preloaded ones (uniform loop)
        int r, t;
        row_slice(rt, nS, &r, &t);
        const int n = (int)ss.hdr[r][t][1];
        if (n <= per) continue;
        const RowPart* P = part_u(f, unit, t, r);
        for (int x = per + tid; x < n; x += kThreads) {
            const uint32_t e = ldnt(&P->ent[x]);
            atomicAdd(&sm.hist(r)[e >> 16], e & 0xFFFFu);
        }
    }
    for (int r = 0; r < rows; ++r) {  // specials (uniform loop; rows without them skip)
        if (!ss.rv[r].has_special || ss.rv[r].overflow || ss.rv[r].bad) continue;
        for (int i = tid; i < nS * kSpecial; i += kThreads) {
            const int t = i / kSpecial, x = i % kSpecial;
            if (x >= min((int)ss.hdr[r][t][2], kSpecial)) continue;
            const RowPart* P = part_c(f, unit, t, r);
            const uint32_t k = ldnt(&P->sp_key[x]);
            const int32_t id = ldnt(&P->sp_id[x]);
            const uint32_t slot = atomicAdd(&ss.n_spm[r], 1u);
            if (slot < (uint32_t)kSpMerge) {
                ss.spk[r][slot] = k;
                ss.spi[r][slot] = id;
            }
            const int g = agg_of_key(k);
            atomicAdd(&ss.agg_n[r][g], 1u);
            atomicMax(&ss.agg_key[r][g], k);
        }
    }
    __syncthreads();

    // ---- pass A (counts): maximum, finite count, top-k cut; threads [256 r, 256 r + 256) ----
    const int r = tid / kRowThreads;
    const int u = tid % kRowThreads;
    const bool live_row = r < rows;
    RowView& rv = ss.rv[live_row ? r : 0];
    const int s0 = u * kSlotsPer;
    // the count of slot i of this thread (read again where needed: registers are scarce here)
    auto cnt_at = [&](int i) -> uint32_t {
        const int s = s0 + i;
        if (!live_row || s >= kSlots) return 0u;
        const int b = slot_bin(s);
        return b >= 0 ? sm.hist(r)[b] : ss.agg_n[r][slot_agg(s)];
    };
    int first = kNone;
    uint32_t nloc = 0;
#pragma unroll
    for (int i = 0; i < kSlotsPer; ++i) {
        const uint32_t n = cnt_at(i);
        if (n != 0u && first == kNone) first = s0 + i;
        nloc += n;
    }
    const int max_slot = row_min(first, ss.wi);
    uint32_t cinc, nfin;
    const uint32_t cexc = row_scan(nloc, ss.wu, &cinc, &nfin);
    const bool proc = live_row && !rv.bad && !rv.overflow;  // uniform per row
    float m = 0.0f;
    if (live_row && max_slot != kNone) {
        const int b = slot_bin(max_slot);
        m = key16_value(b >= 0 ? bin_key(b) : ss.agg_key[r][slot_agg(max_slot)]);
    }
    const double invT = live_row ? rv.invT : 0.0;
    const bool greedy = live_row && rv.greedy;
    const int top_k = prm.top_k;
    const bool k_over = live_row && rv.has_k && (uint32_t)top_k > nfin;
    if (u == 0 && live_row) {
        rv.n_finite = nfin;
        rv.m = m;
        if (nfin == 0u) rv.bad = 1;
        if (!greedy && k_over) rv.overflow = 1;  // -inf tokens would be kept
    }
    const bool cuts = proc && !greedy && nfin > 0u && !k_over;  // uniform per row
    if (cuts && rv.has_k && cexc < (uint32_t)top_k && cinc >= (uint32_t)top_k) {
        uint32_t cum = cexc;
#pragma unroll 1
        for (int i = 0; i < kSlotsPer; ++i) {
            const uint32_t ci = cnt_at(i);
            if (ci != 0u && cum + ci >= (uint32_t)top_k && cum < (uint32_t)top_k) {
                const int s = s0 + i;
                const int b = slot_bin(s);
                if (b < 0) {
                    rv.overflow = 1;  // the cut falls among specials: the general path
                } else {
                    rv.ck = Cut{bin_key(b), (int)((uint32_t)top_k - cum), -1, 0, 0, (int)cum, s};
                    rv.n_kept = top_k;
                }
            }
            cum += ci;
        }
    }
    // the specials' masses (one wave per row with specials)
    if (cuts && rv.has_special && (u >> 6) == 1) {
        const int n = min((int)ss.n_spm[r], kSpMerge);
        double ms[4] = {0.0, 0.0, 0.0, 0.0};
        for (int i = lane; i < n; i += kWave) {
            const uint32_t k = ss.spk[r][i];
            const double e = mass_lean(key16_value(k), m, invT);
            const int g = agg_of_key(k);
#pragma unroll
            for (int x = 0; x < 4; ++x) ms[x] += g == x ? e : 0.0;
        }
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const double sx = wave_sum(ms[x]);
            if (lane == 0) ss.agg_m[r][x] = sx;
        }
    }
    __syncthreads();

    // ---- pass B (masses): the kept mass, the nucleus cut and the normaliser ----
    const bool cuts2 = cuts && !rv.overflow;
    const int ks = (cuts2 && rv.has_k) ? rv.ck.slot : kNone;
    const uint32_t take_k = (cuts2 && rv.has_k) ? (uint32_t)rv.ck.take : 0u;
    const int rr0 = live_row ? r : 0;
    const uint32_t* hist_r = sm.hist(rr0);
    int last_i = -1;
    Pick pk;
    double wloc = 0.0;
    if (cuts2 && nloc != 0u)
        wloc = sweep_run<false>(hist_r, ss.agg_n[rr0], ss.agg_m[rr0], s0, m, invT, ks, take_k, 0.0, 0u, -1.0, -1, &last_i, &pk);
    double winc, Skept;
    const double wexc = row_scan(wloc, ss.wd, &winc, &Skept);
    // the thread whose run holds top_p * S: [exc, inc] of neighbouring threads tile [0, S] (exc
    // of one thread is inc of the one before, bit for bit), so one exists; the first one if
    // rounding makes more
    const double need = (double)prm.top_p * Skept;
    if (cuts2) {
        if (rv.has_p && wexc < need && winc >= need) atomicMin(&ss.cross[r], u);
        ss.xbase[tid] = wexc;
        ss.xcbase[tid] = cexc;
        if (u == 0) {
            rv.S_kept = Skept;
            if (!rv.has_k) rv.n_kept = (int)nfin;
            if (!rv.has_p) {
                rv.S = Skept;
                rv.n_nuc = rv.has_k ? top_k : (int)nfin;
            }
        }
    }
    __syncthreads();
    // the crossing thread of each row settles the nucleus cut, its inputs read back from LDS
    if (cuts2 && rv.has_p && u == ss.cross[r]) {
        const double base = ss.xbase[tid], need2 = (double)prm.top_p * rv.S_kept;
        const uint32_t cbase = ss.xcbase[tid];
        const float mr = rv.m;
        const double it = rv.invT;
        const int ks2 = rv.has_k ? rv.ck.slot : kNone;
        const uint32_t tk2 = rv.has_k ? (uint32_t)rv.ck.take : 0u;
        int lst;
        sweep_run<true>(hist_r, ss.agg_n[rr0], ss.agg_m[rr0], s0, mr, it, ks2, tk2, base, cbase, need2, -1, &lst, &pk);
        bool partial = true;
        if (pk.i < 0) {  // rounding: the run ends short of the scan's total; its last kept slot, whole
            sweep_run<true>(hist_r, ss.agg_n[rr0], ss.agg_m[rr0], s0, mr, it, ks2, tk2, base, cbase, -1.0, s0 + lst, &lst,
                            &pk);
            partial = false;
        }
        const int s = s0 + pk.i;
        const int b = pk.i >= 0 ? slot_bin(s) : -1;
        if (b < 0) {
            rv.overflow = 1;  // the cut falls among specials (or nowhere): the general path
        } else {
            int take = (int)pk.n;
            if (partial && pk.e > 0.0) {
                const double q = ceil((need2 - pk.above) / pk.e);
                take = q < 1.0 ? 1 : (q > (double)pk.n ? (int)pk.n : (int)q);
            }
            rv.cp = Cut{bin_key(b), take, -1, 0, 0, (int)pk.cabove, s};
            rv.S = pk.above + (double)take * pk.e;
            rv.n_nuc = (int)pk.cabove + take;
        }
    }
    if (cuts2 && rv.has_p && u == 0 && ss.cross[r] == kNone) rv.overflow = 1;  // (not reached: see above)
    __syncthreads();

    // ---- owners of the cut ties: every slice's count at each cut bin ----
    // cut bins of (row, cut) as four scalars: CBIN(rr, cc)
    auto cut_bin = [&](int rr, int cc) {
        const RowView& v = ss.rv[rr];
        const bool ok = rr < rows && !v.bad && !v.overflow && !v.greedy;
        const Cut& c = cc ? v.cp : v.ck;
        return (ok && (cc ? v.has_p : v.has_k) && c.key != 0u) ? bin_of_key(c.key) : -1;
    };
    const int cb00 = cut_bin(0, 0), cb01 = cut_bin(0, 1), cb10 = cut_bin(1, 0), cb11 = cut_bin(1, 1);
#define CBIN(rr, cc) ((rr) ? ((cc) ? cb11 : cb10) : ((cc) ? cb01 : cb00))
    const bool any_cut = cb00 >= 0 || cb01 >= 0 || cb10 >= 0 || cb11 >= 0;
    if (any_cut) {
        // the entries are read again from L2 (held in registers through the mass passes they
        // would not fit the count kernel's register budget): the preload's batch, then any past it
        uint32_t e2[kEntIt];
#pragma unroll
        for (int it = 0; it < kEntIt; ++it) {
            const int i = tid + it * kThreads;
            const int rt = i >> lg;
            e2[it] = 0u;
            if (rt < rows * nS) {
                int rr, t;
                row_slice(rt, nS, &rr, &t);
                if ((i & (per - 1)) < (int)ss.hdr[rr][t][1] && (CBIN(rr, 0) >= 0 || CBIN(rr, 1) >= 0))
                    e2[it] = ldnt(&part_c(f, unit, t, rr)->ent[i & (per - 1)]);
            }
        }
#pragma unroll
        for (int it = 0; it < kEntIt; ++it) {
            const int i = tid + it * kThreads;
            const int rt = i >> lg;
            if (rt < rows * nS && e2[it] != 0u) {
                int rr, t;
                row_slice(rt, nS, &rr, &t);
                const int b = (int)(e2[it] >> 16);
                if (b == CBIN(rr, 0)) ss.pc[rr][0][t] = e2[it] & 0xFFFFu;
                if (b == CBIN(rr, 1)) ss.pc[rr][1][t] = e2[it] & 0xFFFFu;
            }
        }
        for (int rt = 0; rt < rows * nS; ++rt) {  // entries past the batch (uniform loop; rare)
            int rr, t;
            row_slice(rt, nS, &rr, &t);
            const int n = (int)ss.hdr[rr][t][1];
            if (n <= per || (CBIN(rr, 0) < 0 && CBIN(rr, 1) < 0)) continue;
            const RowPart* P = part_u(f, unit, t, rr);
            for (int x = per + tid; x < n; x += kThreads) {
                const uint32_t e3 = ldnt(&P->ent[x]);
                const int b = (int)(e3 >> 16);
                if (b == CBIN(rr, 0)) ss.pc[rr][0][t] = e3 & 0xFFFFu;
                if (b == CBIN(rr, 1)) ss.pc[rr][1][t] = e3 & 0xFFFFu;
            }
        }
    }
    __syncthreads();
    if (wave < 4 && any_cut) {  // wave 2 rr + c settles row rr's cut c
        const int rr = wave >> 1, cc = wave & 1;
        if (CBIN(rr, cc) >= 0) {
            Cut& cut = cc ? ss.rv[rr].cp : ss.rv[rr].ck;
            const int nt = lane < nS ? (int)ss.pc[rr][cc][lane] : 0;
            int tex;
            const int tin = wave_scan(nt, &tex);
            const int own = first_lane(__ballot(lane < nS && tin >= cut.take));
            const int before = wave_bcast(tex, own < 0 ? 0 : own);
            if (lane == 0) {
                cut.owner = own < 0 ? nS - 1 : own;
                cut.owner_take = own < 0 ? 0 : cut.take - before;
            }
        }
    }
#undef CBIN
    __syncthreads();
    // ---- greedy argmax, the downweighted set, the drafted token's probabilities ----
    if (wave < rows && lane == 0 && ss.rv[wave].greedy) ss.rv[wave].argmax = ss.rv[wave].nm > 0 ? ss.oid[wave][0] : -1;
    if (dw && rows > 1 && wave == 1) {
        RowView& v = ss.rv[1];
        const bool want_set = a.F > 0 && a.C < 1.0f && !v.greedy && !v.bad && !v.overflow;
        if (want_set) {
            const int n0 = min(min(a.F, v.n_nuc), v.nm);
            const double e2 = lane < n0 ? mass_lean(key16_value(ss.okey[1][lane]), v.m, v.invT) : 0.0;
            const int n = last_lane(__ballot(lane < n0 && e2 > 0.0)) + 1;
            const double ps = wave_sum(lane < n ? e2 / v.S : 0.0);
            if (lane == 0) {
                v.nset = n;
                if (n > 0) {
                    v.kF = ss.okey[1][n - 1];
                    v.idF = ss.oid[1][n - 1];
                    const double Cd = (double)a.C;
                    const double Z = 1.0 - (1.0 - Cd) * ps;
                    if (Z > 0.0) {
                        v.C = Cd;
                        v.Z = Z;
                    } else {
                        v.degenerate = 1;
                    }
                }
            }
        }
    }
    __syncthreads();
    if (dw && s_tok >= 0 && s_tok < a.V && wave < rows && lane == 0 && !ss.rv[wave].greedy) {
        RowView& v = ss.rv[wave];
        const uint32_t sb = v.s_bits;  // the drafted token's mass exp((z_s - m) / T)
        v.e_s = ((sb & 0x7FFFu) < 0x7F80u && v.n_finite > 0u) ? mass_lean(__uint_as_float(sb << 16), v.m, v.invT) : 0.0;
        const double p = prob_of_s(ss, wave, s_tok, wave == 1);
        if (wave == 0) ss.qs = p;
        else ss.ps = p;
    }
    __syncthreads();
}

}  // namespace fast
}  // namespace sv
