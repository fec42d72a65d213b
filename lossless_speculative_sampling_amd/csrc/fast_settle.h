// Settling one (request, position) unit from its slices' summaries: the exact processed
// distributions of the target and draft rows (temperature, top-k, softmax, nucleus; DeepMind
// speculative-sampling page, section 6), the Saguaro downweighted set of the draft row (SSD
// reading notes, section 4.4), and the processed probabilities of the drafted token that the
// acceptance test compares.  Run by the last slice of a unit to finish counting.
//
// Every slice publishes its occupied bins as (bin, count) entries.  The settling slice adds the
// other slices' entries to its own histograms, then walks each row's values in descending
// order: counts give the maximum and the top-k cut and list the occupied values compactly;
// one fp64 exp per occupied value, spread evenly over the row's threads, gives the masses, the
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
// the row threads' slot kinds in pass A (see there)
constexpr int kBinThreads = (kNegBins + kSlotsPer - 1) / kSlotsPer;     // 118 per sign
constexpr int kBinTail = kNegBins - (kBinThreads - 1) * kSlotsPer;      // 4
constexpr int kTinyThread = 1 + kBinThreads;                           // 119
constexpr int kNegThread0 = kTinyThread + 1;                           // 120
constexpr int kHugeNegThread = kNegThread0 + kBinThreads;              // 238
static_assert(kHugeNegThread < kRowThreads && kBinTail > 0 && kBinTail <= kSlotsPer, "pass A thread kinds");
static_assert(kSlotTP - kSlotHP - 1 == kNegBins && kSlotHN - kSlotTN - 1 == kNegBins, "bins per sign");
constexpr int kSpMerge = 256;   // specials of one row merged in LDS (more: the general path)
constexpr int kEntIt = 12;      // sparse entries each thread loads per batch
constexpr int kStageCap = 512;  // staged candidates per row: every slice's list
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

typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));

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
    alignas(16) uint32_t hdr[2][kMaxSlices][8];   // each slice's header words
    uint64_t stage[2][kStageCap];     // every slice's candidates, (key << 32) | ~id, slice t at t * want
    uint32_t okey[2][kTop];           // merged candidates in token order
    int32_t oid[2][kTop];
    uint32_t spk[2][kSpMerge];        // every slice's specials of a row
    int32_t spi[2][kSpMerge];
    uint32_t n_spm[2];
    uint32_t agg_n[2][4];             // specials per aggregate slot: count, largest key, mass
    uint32_t agg_key[2][4];
    double agg_m[2][4];
    uint32_t pc[2][2][kMaxSlices];    // per-slice counts at the top-k / nucleus cut bins
    double cand_e[kTop];              // masses of the draft row's leading candidates
    double cand_pre[kTop];            // and their inclusive prefix sums in token order
    uint64_t wq[2][4];                // per-row wave partials of the scans
    double wd[2][4];
    uint32_t wk[2][4];
    int crossed[2];                   // the nucleus cut was placed
    double qs, ps;                    // the drafted token's processed probabilities
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
// it (one barrier).
__device__ __forceinline__ uint64_t row_scan_u64(uint64_t v, uint64_t (*wtot)[4], uint64_t* inc, uint64_t* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int r = threadIdx.x / kRowThreads, w = (threadIdx.x % kRowThreads) / kWave;
    uint64_t exc;
    const uint64_t in = wave_scan(v, &exc);
    if (lane == kWave - 1) wtot[r][w] = in;
    __syncthreads();
    uint64_t before = 0, all = 0;
    for (int x = 0; x < 4; ++x) {
        const uint64_t t = wtot[r][x];
        if (x < w) before += t;
        all += t;
    }
    *total = all;
    *inc = before + in;
    return before + exc;
}

// The same for a (mass, count) pair with one barrier.  The exclusive mass of thread u + 1
// equals the inclusive mass of thread u bit for bit, so the intervals (exc, inc] of the
// threads with mass tile (0, total] without overlap.
struct Scan2 {
    double wexc, winc, wtot;
    uint32_t kexc, ktot;
};
__device__ __forceinline__ Scan2 row_scan2(double w, uint32_t k, SettleSmem& ss) {
    const int lane = threadIdx.x & (kWave - 1);
    const int r = threadIdx.x / kRowThreads, wv = (threadIdx.x % kRowThreads) / kWave;
    double we;
    uint32_t ke;
    const double wi = wave_scan(w, &we);
    const uint32_t ki = wave_scan(k, &ke);
    if (lane == kWave - 1) {
        ss.wd[r][wv] = wi;
        ss.wk[r][wv] = ki;
    }
    __syncthreads();
    double before = 0.0, all = 0.0;
    uint32_t kb = 0u, ka = 0u;
    for (int x = 0; x < 4; ++x) {
        const double t = ss.wd[r][x];
        const uint32_t tk = ss.wk[r][x];
        if (x < wv) {
            before += t;
            kb += tk;
        }
        all += t;
        ka += tk;
    }
    return Scan2{before + we, before + wi, all, kb + ke, ka};
}

__device__ __forceinline__ bool cut_keeps_s(const RowView& rv, const Cut& c, uint32_t key_s) {
    if (key_s > c.key) return true;
    if (key_s < c.key) return false;
    return rv.rank_s < c.take;
}

// Processed probability of the drafted token s (bf16 bits h, rank_s elements of its key before
// it in token order, mass e) in a row with normaliser S and the given cuts: e / S when both
// cuts keep it, else 0.
__device__ __forceinline__ double prob_of_s(uint32_t h, int rank_s, bool has_k, uint32_t kk, int takek, bool has_p,
                                            uint32_t kp, int takep, double S, double e) {
    if ((h & 0x7FFFu) >= 0x7F80u) return 0.0;
    const uint32_t key = key16(h);
    const bool keep_k = !has_k || key > kk || (key == kk && rank_s < takek);
    const bool keep_p = !has_p || key > kp || (key == kp && rank_s < takep);
    return (keep_k && keep_p) ? e / S : 0.0;
}

// A compact list entry of an occupied scan slot: (slot << 20) | count (a count is at most
// kMaxSlices * kSliceCols = 2^18).
constexpr int kListShift = 20;
constexpr uint32_t kListCount = (1u << kListShift) - 1u;
static_assert(kMaxSlices * kSliceCols <= (int)kListCount && kSlots < (1 << (32 - kListShift)), "list entry fields");

// ------------------------------------------------------------------------------------------
// The settle step: both rows' processed distributions (maxima, normalisers, top-k and nucleus
// cuts with their owner slices), the draft row's downweighted set (dw) and the drafted token's
// processed probabilities.  All threads.  On entry sm.hist(r) holds this slice's (own) counts
// of row r; the other slices' entries are added to them, and the merged rows are then turned
// into compact lists of the occupied slots.
// ------------------------------------------------------------------------------------------
template <typename Smem>
__device__ __forceinline__ void settle_rows(const FastArgs& f, Smem& sm, int unit, int own, int j, int rows,
                                            const spec_params& prm, bool dw, int s_tok) {
    const VerifyArgs& a = f.a;
    SettleSmem& ss = sm.ss;
    const int nS = f.nS;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int want0 = list_len(a, prm, false);
    const int want1 = rows > 1 ? draft_list_len(f, prm, j) : 0;
    // (row, slice) groups of entries: 2^lgt threads each, kEntIt entries a thread per batch
    const int G = rows * nS;
    int lgt = 0;
    while ((G << (lgt + 1)) <= kThreads) ++lgt;
    const int tpg = 1 << lgt;
    const int gi = tid >> lgt;
    int gr = 0, gt = 0;
    if (gi < G) row_slice(gi, nS, &gr, &gt);
    const int cover = tpg * kEntIt;  // entries of a group the batch covers

    // ---- round trip 1: headers, the other slices' entries, the candidate lists ----
    u32x4 hw = {0u, 0u, 0u, 0u};
    const bool hload = tid < 2 * G;
    if (hload) {
        int r, t;
        row_slice(tid >> 1, nS, &r, &t);
        hw = ldnt(reinterpret_cast<const u32x4*>(part_c(f, unit, t, r)) + (tid & 1));
    }
    // (every load is issued, at a clamped index of a valid record, so none waits on a branch;
    // which of them count is decided where they are used)
    uint32_t ent[kEntIt];
    const bool merge_mine = gi < G && gt != own;
    const uint32_t* ebase = part_c(f, unit, gt, gr)->ent;  // (gi >= G: the unit's first record, unused)
    const int x0 = tid & (tpg - 1);
    // thread x0 of a group takes entries [x0 kEntIt, x0 kEntIt + kEntIt) in 16-byte loads (a
    // start inside the list ends inside it: kBins is a multiple of kEntIt; later starts read
    // entry 0 and count none)
    static_assert(kBins % kEntIt == 0 && kEntIt % 4 == 0, "whole 16-byte loads within a list");
    const int e0 = x0 * kEntIt < kBins ? x0 * kEntIt : 0;
#pragma unroll
    for (int it = 0; it < kEntIt; it += 4) {
        const u32x4 v = ldnt(reinterpret_cast<const u32x4*>(ebase + e0 + it));
        ent[it] = v[0];
        ent[it + 1] = v[1];
        ent[it + 2] = v[2];
        ent[it + 3] = v[3];
    }
    // candidates: thread u of row r stages positions u and u + 256 of the row's slice-major list
    const int cr = tid / kRowThreads, cu = tid % kRowThreads;
    const int cwant = cr < rows ? (cr ? want1 : want0) : 0;
    const bool cstage = cwant > 0 && nS * cwant <= kStageCap;  // (more: the row takes the general path)
    // (a listed candidate has a finite value, so its key and the order word are non-zero; slots
    // past a slice's list and the padding to a multiple of 8 hold 0)
    const int nst = cstage ? nS * cwant : 0, nst8 = (nst + 7) & ~7;
    uint64_t cord[2] = {0ull, 0ull};
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int p = cu + it * kRowThreads;
        if (p < nst) {
            const int t = p / cwant, x = p - t * cwant;
            const RowPart* P = part_c(f, unit, t, cr);
            const uint64_t o = ((uint64_t)ldnt(&P->top_key[x]) << 32) | (uint32_t)~ldnt(&P->top_id[x]);
            cord[it] = x < (int)ldnt(&P->n_top) ? o : 0ull;
        }
    }
    if (tid < 2) {
        ss.n_spm[tid] = 0u;
        ss.crossed[tid] = 0;
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
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int p = cu + it * kRowThreads;
        if (p < nst8) ss.stage[cr][p] = cord[it];
    }
    __syncthreads();

    // header digest, in every wave (uniform values without a serial walk): lane l < G reads the
    // first header words of (row, slice) l
    u32x4 hv = {0u, 0u, 0u, 0u};
    int hr = 0;
    if (lane < G) {
        int ht;
        row_slice(lane, nS, &hr, &ht);
        hv = *reinterpret_cast<const u32x4*>(&ss.hdr[hr][ht][0]);
    }
    const bool more_ent = __ballot(lane < G && (int)hv[1] > cover) != 0;  // entries past the batch
    const uint32_t nsp0 = wave_sum(hr == 0 ? hv[2] : 0u), nsp1 = wave_sum(hr == 1 ? hv[2] : 0u);
    const uint32_t fl0 = wave_or(hr == 0 ? hv[0] : 0u), fl1 = wave_or(hr == 1 ? hv[0] : 0u);

    // ---- the other slices' entries into this slice's histograms; per-row flags; specials;
    //      the candidates' ranks ----
    if (merge_mine) {
        const int n = (int)ss.hdr[gr][gt][1];
        const int nv = min(max(n - x0 * kEntIt, 0), kEntIt);  // this thread's entries below n
#pragma unroll
        for (int it = 0; it < kEntIt; ++it)
            if (it < nv) atomicAdd(&sm.hist(gr)[ent[it] >> 16], ent[it] & 0xFFFFu);
    }
    for (int g = 0; more_ent && g < G; ++g) {  // entries past the batch (uniform loop; rare)
        int r, t;
        row_slice(g, nS, &r, &t);
        const int n = (int)ss.hdr[r][t][1];
        if (n <= cover || t == own) continue;
        const RowPart* P = part_u(f, unit, t, r);
        for (int x = cover + tid; x < n; x += kThreads) {
            const uint32_t e = ldnt(&P->ent[x]);
            atomicAdd(&sm.hist(r)[e >> 16], e & 0xFFFFu);
        }
    }
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
        const int rank = (int)wave_sum(cnt);
        const uint32_t nsp_all = wave_sum(nsp);
        const int ncand = (int)wave_sum(ntop);
        const bool xbad = __ballot(xcc != ss.hdr[r][0][7]) != 0;
        const int want = r ? want1 : want0;
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
            // too many specials, or more candidates than the stage holds: the general path
            rv.overflow = ((flo & 2u) || nsp_all > (uint32_t)kSpMerge || nS * want > kStageCap) ? 1 : 0;
            rv.has_special = nsp_all > 0u ? 1 : 0;
            rv.s_bits = ss.hdr[r][0][5];
            rv.rank_s = rank;
            rv.xcc_bad = xbad ? 1u : 0u;
            rv.e_s = 0.0;
            rv.m = 0.0f;
            rv.nm = min(ncand, want);
        }
    }
    for (int r = 0; r < rows; ++r) {  // specials (uniform loop; rows without them skip)
        const uint32_t nsp_all = r ? nsp1 : nsp0, flo = r ? fl1 : fl0;
        if (nsp_all == 0u || nsp_all > (uint32_t)kSpMerge || (flo & 3u)) continue;
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
    // candidate ranks in token order (key desc, id asc) over every slice's list of the row:
    // rank = staged order words above the candidate's (invalid slots hold 0, below every
    // listed candidate).  Up to 128 candidates, T = 2, 4 or 8 consecutive threads share one
    // candidate, each comparing it with every T-th pair of the stage, and their partial ranks
    // are summed across the group; beyond that each thread ranks its own two against the
    // whole stage in batches of 8.
    const int T = nst <= 32 ? 8 : nst <= 64 ? 4 : nst <= 128 ? 2 : 1;  // (uniform per wave)
    if (T > 1) {
        const int pc = cu / T, part = cu & (T - 1);
        const uint64_t o = pc < nst ? ss.stage[cr][pc] : 0ull;
        int rk = 0;
        if (o != 0ull) {
            const u64x2* sl2 = reinterpret_cast<const u64x2*>(ss.stage[cr]);
#pragma unroll 4
            for (int q = part; q < nst8 / 2; q += T) {
                const u64x2 v = sl2[q];
                rk += (v[0] > o ? 1 : 0) + (v[1] > o ? 1 : 0);
            }
        }
        rk += dpp<kDppQuadSwap1>(rk);
        if (T >= 4) rk += dpp<kDppQuadSwap2>(rk);
        if (T >= 8) rk += dpp<kDppRowHalfMirror>(rk);
        if (part == 0 && o != 0ull && rk < cwant) {
            ss.okey[cr][rk] = (uint32_t)(o >> 32);
            ss.oid[cr][rk] = (int32_t)~(uint32_t)o;
        }
    } else if (nst > 0 && (cord[0] != 0ull || cord[1] != 0ull)) {
        const uint64_t o0 = cord[0], o1 = cord[1];
        int r0 = 0, r1 = 0;
        const uint64_t* sl = ss.stage[cr];
#pragma unroll 2
        for (int q = 0; q < nst8; q += 8) {
            uint64_t v[8];
#pragma unroll
            for (int d = 0; d < 8; ++d) v[d] = sl[q + d];
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                r0 += v[d] > o0 ? 1 : 0;
                r1 += v[d] > o1 ? 1 : 0;
            }
        }
        if (o0 != 0ull && r0 < cwant) {
            ss.okey[cr][r0] = (uint32_t)(o0 >> 32);
            ss.oid[cr][r0] = (int32_t)~(uint32_t)o0;
        }
        if (o1 != 0ull && r1 < cwant) {
            ss.okey[cr][r1] = (uint32_t)(o1 >> 32);
            ss.oid[cr][r1] = (int32_t)~(uint32_t)o1;
        }
    }
    __syncthreads();

    // ---- pass A (counts): maximum, finite count, top-k cut, the compact list of occupied
    //      slots; threads [256 r, 256 r + 256), twelve consecutive slots each ----
    const int r = tid / kRowThreads;
    const int u = tid % kRowThreads;
    const bool live_row = r < rows;
    const int rr0 = live_row ? r : 0;
    RowView& rv = ss.rv[rr0];
    // this thread's slots, consecutive in slot (descending key) order and of one kind: thread 0
    // the huge positive values; threads 1 .. kBinThreads the positive bins (the last one the
    // remaining kBinTail); the next thread the tiny positive values, zero and the tiny negative
    // values; then the negative bins (the first thread the kBinTail highest); then the huge
    // negative values.  A bin thread reads its counts at fixed offsets from one address.
    const bool pos_t = u >= 1 && u <= kBinThreads;
    const bool neg_t = u >= kNegThread0 && u < kHugeNegThread;
    const int s0 = u == 0 ? kSlotHP
                 : pos_t ? 1 + kSlotsPer * (u - 1)
                 : u == kTinyThread ? kSlotTP
                 : neg_t ? (u == kNegThread0 ? kSlotTN + 1 : kSlotTN + 1 + kBinTail + kSlotsPer * (u - kNegThread0 - 1))
                 : u == kHugeNegThread ? kSlotHN : kSlots;
    const int nb = pos_t ? (u == kBinThreads ? kBinTail : kSlotsPer) : neg_t ? (u == kNegThread0 ? kBinTail : kSlotsPer) : 0;
    // bin of slot s0 (bins descend with the slot); bin - 11 >= 0 for every bin thread
    const int bb = pos_t ? kBins - s0 : neg_t ? kSlotHN - 1 - s0 : kSlotsPer - 1;
    // (flags read before the scan: single threads update them after it)
    // (read unconditionally and combined without short-circuits: no branch waits on each read)
    // (uniform in each wave: kept in scalar registers)
    const int f_bad = __builtin_amdgcn_readfirstlane(rv.bad), f_ovf = __builtin_amdgcn_readfirstlane(rv.overflow),
              f_gr = __builtin_amdgcn_readfirstlane(rv.greedy), f_hk = __builtin_amdgcn_readfirstlane(rv.has_k),
              f_hp = __builtin_amdgcn_readfirstlane(rv.has_p), f_hs = __builtin_amdgcn_readfirstlane(rv.has_special);
    const bool proc = live_row & (f_bad == 0) & (f_ovf == 0);  // uniform per row
    const bool greedy = live_row & (f_gr != 0);
    const bool has_k = live_row & (f_hk != 0), has_p = live_row & (f_hp != 0), has_sp = live_row & (f_hs != 0);
    uint32_t c[kSlotsPer];
    uint32_t nloc = 0, nz = 0;
    int first = -1;
    const uint32_t* hb = sm.hist(rr0) + (bb - (kSlotsPer - 1));
    const uint32_t a0 = ss.agg_n[rr0][0], a1 = ss.agg_n[rr0][1], a2 = ss.agg_n[rr0][2], a3 = ss.agg_n[rr0][3];
    const uint32_t cz = sm.hist(rr0)[kZeroBin];
#pragma unroll
    for (int i = 0; i < kSlotsPer; ++i) {
        uint32_t v = i < nb ? hb[kSlotsPer - 1 - i] : 0u;
        if (i == 0) v = u == 0 ? a0 : u == kTinyThread ? a1 : u == kHugeNegThread ? a3 : v;
        if (i == 1) v = u == kTinyThread ? cz : v;
        if (i == 2) v = u == kTinyThread ? a2 : v;
        c[i] = live_row ? v : 0u;
        nloc += c[i];
        nz += c[i] != 0u ? 1u : 0u;
        if (c[i] != 0u && first < 0) first = i;
    }
    uint64_t pinc, ptot;
    const uint64_t pexc = row_scan_u64(((uint64_t)nz << 32) | nloc, ss.wq, &pinc, &ptot);
    const uint32_t cexc = (uint32_t)pexc, cinc = (uint32_t)pinc, nfin = (uint32_t)ptot;
    const int zexc = (int)(pexc >> 32), n_occ = (int)(ptot >> 32);
    const int top_k = prm.top_k;
    const bool k_over = has_k && (uint32_t)top_k > nfin;
    if (live_row && u == 0) {
        rv.n_finite = nfin;
        if (nfin == 0u) rv.bad = 1;
        if (!greedy && k_over) rv.overflow = 1;  // -inf tokens would be kept
    }
    if (live_row && cexc == 0u && nloc != 0u) {  // the first occupied slot: the maximum
        const int s = s0 + first;
        const int b = slot_bin(s);
        rv.m = key16_value(b >= 0 ? bin_key(b) : ss.agg_key[r][slot_agg(s)]);
    }
    const bool cuts = proc && !greedy && nfin > 0u && !k_over;  // uniform per row
    // the thread whose counts hold the top_k-th element places the top-k cut from the list
    const bool k_thread = cuts && has_k && cexc < (uint32_t)top_k && cinc >= (uint32_t)top_k;
    // the compact list, written over the histogram row (every count is read by now)
    if (live_row) {
        int o = zexc;
#pragma unroll
        for (int i = 0; i < kSlotsPer; ++i)
            if (c[i] != 0u) sm.hist(r)[o++] = ((uint32_t)(s0 + i) << kListShift) | c[i];
    }
    __syncthreads();
    if (prm.top_k > 0 && prm.top_k < a.V) {  // (uniform: both rows take the request's top_k)
        if (k_thread) {
            uint32_t cum = cexc;
#pragma unroll 1
            for (int p = zexc; p < zexc + (int)nz; ++p) {
                const uint32_t le = sm.hist(r)[p];
                const uint32_t n = le & kListCount;
                if (cum + n >= (uint32_t)top_k) {
                    const int s = (int)(le >> kListShift);
                    const int b = slot_bin(s);
                    if (b < 0) {
                        rv.overflow = 1;  // the cut falls among specials: the general path
                    } else {
                        rv.ck = Cut{bin_key(b), (int)((uint32_t)top_k - cum), -1, 0, 0, (int)cum, s};
                        rv.n_kept = top_k;
                    }
                    break;
                }
                cum += n;
            }
        }
        __syncthreads();
    }

    // ---- the specials' masses (one wave per row with specials; rare) ----
    const bool any_sp = (ss.rv[0].has_special && !ss.rv[0].overflow) || (rows > 1 && ss.rv[1].has_special && !ss.rv[1].overflow);
    if (any_sp) {
        if (cuts && has_sp && (u >> 6) == 1) {
            const int n = min((int)ss.n_spm[r], kSpMerge);
            const float m = rv.m;
            const double invT = rv.invT;
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
    }

    // ---- the entries again for the owners of the cut ties (own slice included), in flight
    //      while the masses are summed ----
    uint32_t e2[kEntIt];
#pragma unroll
    for (int it = 0; it < kEntIt; it += 4) {
        const u32x4 v = ldnt(reinterpret_cast<const u32x4*>(ebase + e0 + it));
        e2[it] = v[0];
        e2[it + 1] = v[1];
        e2[it + 2] = v[2];
        e2[it + 3] = v[3];
    }

    // ---- pass B (masses): the compact list spread evenly over the row's threads ----
    const bool cuts2 = cuts && !rv.overflow;
    const int ks = (cuts2 && has_k) ? rv.ck.slot : kNone;
    const uint32_t take_k = (cuts2 && has_k) ? (uint32_t)rv.ck.take : 0u;
    const float m = live_row ? rv.m : 0.0f;
    const double invT = live_row ? rv.invT : 0.0;
    const int per = (n_occ + kRowThreads - 1) / kRowThreads;
    const int lo = min(u * per, n_occ), hi = min(lo + per, n_occ);
    double wloc = 0.0;
    uint32_t kloc = 0u;
    if (cuts2) {
#pragma unroll 1
        for (int p = lo; p < hi; ++p) {
            const uint32_t le = sm.hist(r)[p];
            const int s = (int)(le >> kListShift);
            if (s > ks) break;
            const uint32_t n = s == ks ? take_k : (le & kListCount);
            const int b = slot_bin(s);
            wloc += b >= 0 ? (double)n * mass_lean(key16_value(bin_key(b)), m, invT) : ss.agg_m[r][slot_agg(s)];
            kloc += n;
        }
    }
    // the drafted token's mass in each row (thread 255 of the row) and the masses of the draft
    // row's leading candidates (its last wave), for the final step
    const bool tok = dw && s_tok >= 0 && s_tok < a.V;
    if (tok && live_row && !greedy && u == kRowThreads - 1) {
        const uint32_t sb = rv.s_bits;  // exp((z_s - m) / T)
        rv.e_s = ((sb & 0x7FFFu) < 0x7F80u && nfin > 0u) ? mass_lean(__uint_as_float(sb << 16), m, invT) : 0.0;
    }
    if (dw && r == 1 && cuts2 && a.F > 0 && a.C < 1.0f && u >= kRowThreads - kWave) {  // (a whole wave)
        const int l = u - (kRowThreads - kWave);
        const double ec = l < min(a.F, rv.nm) ? mass_lean(key16_value(ss.okey[1][l]), m, invT) : 0.0;
        double ex;
        const double ei = wave_scan(ec, &ex);
        ss.cand_e[l] = ec;
        ss.cand_pre[l] = ei;
    }
    const Scan2 sc = row_scan2(wloc, kloc, ss);
    const double Skept = sc.wtot;
    const double need = (double)prm.top_p * Skept;
    if (cuts2 && u == 0) {
        rv.S_kept = Skept;
        if (!has_k) rv.n_kept = (int)nfin;
        if (!has_p) {
            rv.S = Skept;
            rv.n_nuc = has_k ? top_k : (int)nfin;
        }
    }
    // the one thread whose interval (exc, inc] holds top_p * S places the nucleus cut
    if (cuts2 && has_p && sc.wexc < need && need <= sc.winc) {
        double cum = sc.wexc;
        uint32_t ccum = sc.kexc;
        int pick_s = -1;
        double above = 0.0, pe = 0.0;
        uint32_t pn = 0u, pcab = 0u;
        bool partial = false;
#pragma unroll 1
        for (int p = lo; p < hi; ++p) {
            const uint32_t le = sm.hist(r)[p];
            const int s = (int)(le >> kListShift);
            if (s > ks) break;
            const uint32_t n = s == ks ? take_k : (le & kListCount);
            const int b = slot_bin(s);
            const double e = b >= 0 ? mass_lean(key16_value(bin_key(b)), m, invT) : 0.0;
            const double w = b >= 0 ? (double)n * e : ss.agg_m[r][slot_agg(s)];
            // the last kept slot stands in when rounding leaves the run short of need
            pick_s = s;
            above = cum;
            pe = e;
            pn = n;
            pcab = ccum;
            if (w > 0.0 && cum + w >= need) {
                partial = true;
                break;
            }
            cum += w;
            ccum += n;
        }
        const int b = pick_s >= 0 ? slot_bin(pick_s) : -1;
        if (b < 0) {
            rv.overflow = 1;  // the cut falls among specials (or nowhere): the general path
        } else {
            int take = (int)pn;
            if (partial && pe > 0.0) {
                const double q = ceil((need - above) / pe);
                take = q < 1.0 ? 1 : (q > (double)pn ? (int)pn : (int)q);
            }
            rv.cp = Cut{bin_key(b), take, -1, 0, 0, (int)pcab, pick_s};
            rv.S = above + (double)take * pe;
            rv.n_nuc = (int)pcab + take;
        }
        ss.crossed[r] = 1;
    }
    __syncthreads();

    // ---- owners of the cut ties: every slice's count at each cut bin; the downweighted set
    //      and the drafted token's probabilities ----
    auto cut_bin = [&](int rr, int cc) {
        const RowView& v = ss.rv[rr];
        const bool ok = rr < rows && !v.bad && !v.overflow && !v.greedy;
        const Cut& ct = cc ? v.cp : v.ck;
        return (ok && (cc ? v.has_p : v.has_k) && ct.key != 0u && ct.slot != kNone) ? bin_of_key(ct.key) : -1;
    };
    // (lane 2 rr + cc of every wave works out cut cc of row rr: one round of LDS reads, not four)
    const int cbl = lane < 4 ? cut_bin(lane >> 1, lane & 1) : -1;
    const int cb00 = __builtin_amdgcn_readlane(cbl, 0), cb01 = __builtin_amdgcn_readlane(cbl, 1),
              cb10 = __builtin_amdgcn_readlane(cbl, 2), cb11 = __builtin_amdgcn_readlane(cbl, 3);
#define CBIN(rr, cc) ((rr) ? ((cc) ? cb11 : cb10) : ((cc) ? cb01 : cb00))
    const bool any_cut = cb00 >= 0 || cb01 >= 0 || cb10 >= 0 || cb11 >= 0;
    if (any_cut && gi < G) {
        const int n = (int)ss.hdr[gr][gt][1];
        const int nv = min(max(n - x0 * kEntIt, 0), kEntIt);
        const int c0b = CBIN(gr, 0), c1b = CBIN(gr, 1);
        // a slice row lists a bin at most once and never with count 0: the count found at each
        // cut bin (0: none), without a branch per entry
        uint32_t h0 = 0u, h1 = 0u;
#pragma unroll
        for (int it = 0; it < kEntIt; ++it) {
            const uint32_t e = it < nv ? e2[it] : 0xFFFFFFFFu;  // (bin 0xFFFF is no cut bin)
            const int b = (int)(e >> 16);
            h0 = b == c0b ? (e & 0xFFFFu) : h0;
            h1 = b == c1b ? (e & 0xFFFFu) : h1;
        }
        if (h0 != 0u) ss.pc[gr][0][gt] = h0;
        if (h1 != 0u) ss.pc[gr][1][gt] = h1;
    }
    if (any_cut && more_ent) {
        for (int g = 0; g < G; ++g) {  // entries past the batch (uniform loop; rare)
            int rr, t;
            row_slice(g, nS, &rr, &t);
            const int n = (int)ss.hdr[rr][t][1];
            if (n <= cover || (CBIN(rr, 0) < 0 && CBIN(rr, 1) < 0)) continue;
            const RowPart* P = part_u(f, unit, t, rr);
            for (int x = cover + tid; x < n; x += kThreads) {
                const uint32_t e3 = ldnt(&P->ent[x]);
                const int b = (int)(e3 >> 16);
                if (b == CBIN(rr, 0)) ss.pc[rr][0][t] = e3 & 0xFFFFu;
                if (b == CBIN(rr, 1)) ss.pc[rr][1][t] = e3 & 0xFFFFu;
            }
        }
    }
    if (wave == 4 && rows > 1) {  // the draft row: downweighted set, then the token's probability
        RowView& v = ss.rv[1];
        // (every field read once, up front)
        const bool vok = !v.greedy && !v.bad && !v.overflow;
        const double S = v.S, e_s = v.e_s;
        const int n_nuc = v.n_nuc, nm = v.nm, rank_s = v.rank_s;
        const uint32_t sb = v.s_bits;
        const bool hk = v.has_k, hp = v.has_p;
        const uint32_t kk = v.ck.key, kp = v.cp.key;
        const int tk = v.ck.take, tp = v.cp.take;
        const bool want_set = dw && a.F > 0 && a.C < 1.0f && vok;
        int n = 0;
        double Cd = 1.0, Z = 1.0;
        uint32_t kF = 0xFFFFFFFFu;
        int idF = -1;
        bool degen = false;
        if (want_set) {
            const int n0 = min(min(a.F, n_nuc), nm);
            const double ec = lane < n0 ? ss.cand_e[lane] : 0.0;
            n = last_lane(__ballot(lane < n0 && ec > 0.0)) + 1;
            // (the masses fall in token order: the set is a prefix of the candidates)
            const double psum = n > 0 ? ss.cand_pre[n - 1] / S : 0.0;
            if (n > 0) {
                kF = ss.okey[1][n - 1];
                idF = ss.oid[1][n - 1];
                const double Zc = 1.0 - (1.0 - (double)a.C) * psum;
                if (Zc > 0.0) {
                    Cd = (double)a.C;
                    Z = Zc;
                } else {
                    degen = true;
                }
            }
        }
        if (lane == 0) {
            if (tok && !v.greedy) {
                const double p = prob_of_s(sb, rank_s, hk, kk, tk, hp, kp, tp, S, e_s);
                const double fct = (n > 0 && e_s > 0.0 && in_cut_id(kF, idF, key16(sb), s_tok)) ? Cd : 1.0;
                ss.ps = (p * fct) / Z;
            }
            if (want_set) {
                v.nset = n;
                v.kF = kF;
                v.idF = idF;
                v.C = Cd;
                v.Z = Z;
                v.degenerate = degen ? 1 : 0;
            }
        }
    }
    if (wave == 5 && tok && lane == 0 && !ss.rv[0].greedy) {  // the target row's probability
        const RowView& v = ss.rv[0];
        ss.qs = prob_of_s(v.s_bits, v.rank_s, v.has_k, v.ck.key, v.ck.take, v.has_p, v.cp.key, v.cp.take, v.S, v.e_s);
    }
    if (wave == 6 && lane < rows && ss.rv[lane].greedy) ss.rv[lane].argmax = ss.rv[lane].nm > 0 ? ss.oid[lane][0] : -1;
    __syncthreads();
    if (cuts2 && has_p && u == 0 && !ss.crossed[r]) rv.overflow = 1;  // (no thread placed it)
    if (wave < 4 && any_cut) {  // wave 2 rr + c settles row rr's cut c
        const int rr = wave >> 1, cc = wave & 1;
        if (CBIN(rr, cc) >= 0) {
            Cut& cut = cc ? ss.rv[rr].cp : ss.rv[rr].ck;
            const int nt = lane < nS ? (int)ss.pc[rr][cc][lane] : 0;
            int tex;
            const int tin = wave_scan(nt, &tex);
            const int own_l = first_lane(__ballot(lane < nS && tin >= cut.take));
            const int before = wave_bcast(tex, own_l < 0 ? 0 : own_l);
            if (lane == 0) {
                cut.owner = own_l < 0 ? nS - 1 : own_l;
                cut.owner_take = own_l < 0 ? 0 : cut.take - before;
            }
        }
    }
#undef CBIN
    __syncthreads();
}

}  // namespace fast
}  // namespace sv
