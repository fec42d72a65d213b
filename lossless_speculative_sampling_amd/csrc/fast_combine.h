// Settling one (request, position) unit from its slices' summaries: the exact processed
// distributions of the target and draft rows (temperature, top-k, softmax, nucleus; DeepMind
// speculative-sampling page, section 6), the Saguaro downweighted set of the draft row (SSD
// reading notes, section 4.4), and the processed probabilities of the draft token that the
// acceptance test compares.  Run by the last slice of a unit to finish counting.
#pragma once

#include "fast_common.h"

namespace sv {
namespace fast {

struct Cut {       // a cut in token order: keep key > key, and part of the elements at key
    uint32_t key;
    int take;         // histogram cut: elements kept at `key` (the first `take` in token order)
    int explicit_id;  // >= 0: explicit cut, the id of the last kept element at `key`
    int owner;        // histogram cut: slice holding the last kept element at `key`
    int owner_take;   // elements at `key` that slice keeps
    int count_above;  // elements with a larger key
};

struct RowView {   // the combined view of one row, identical in every slice of the unit
    int bad, overflow, greedy, argmax;
    float m;
    double invT;               // 1 / temperature
    double sc[kMaxSlices];     // per-slice rescale exp((m_t - m)/T)
    int n_top[kMaxSlices];     // per-slice candidate list lengths
    double seg_mass[kSegs];
    uint32_t seg_count[kSegs];
    uint32_t n_finite;
    int has_special;
    int want;                  // candidates each slice lists
    int total;                 // candidates all slices listed
    int nm;                    // merged candidates (okey / oid)
    double S_all, S_kept, S;
    int has_k, has_p, small_k; // top-k / nucleus active; top-k settled by the merged list
    Cut ck, cp;
    int n_kept;                // elements kept by top-k (or all finite)
    int n_nuc;                 // elements in the nucleus
    int nset;                  // downweighted set size (0: off)
    uint32_t kF;
    int idF;
    double C, Z;
    int degenerate;
    // draft token s: its value and its rank among the elements with its key (token order)
    uint32_t s_bits;
    double e_s;                // its mass exp((z_s - m)/T) (0 for -inf or no token)
    int rank_s;
    // a histogram cut in progress (0 none, 1 top-k count cut, 2 nucleus mass cut)
    int pend;
    int pend_seg;
    int early;                 // stage A ran before the candidate merge
    int early_g;               // the group whose per-slice counts were loaded then (-1: none)
    int pend_cnt_above;
    double pend_need;
    double pend_above;
    double pend_mass_above;
};

// LDS of the unit settle step (the last slice of a unit), laid over the histograms.
struct UnitSmem {
    RowView rv[2];
    uint32_t key[2][kMergeCap];   // every slice's candidate list, slice-major; specials staging
    int32_t id[2][kMergeCap];
    double qs, ps;                // the drafted token's processed probabilities
    uint32_t okey[2][kTop];       // merged candidates in token order
    int32_t oid[2][kTop];
    union {
        struct {                  // every slice's segment arrays, as loaded
            double mass[2][kMaxSlices][kSegs];
            uint32_t count[2][kMaxSlices][kSegs];
        } seg;
        struct {
            uint16_t fine_ps[2][kMaxSlices][kGroup];  // per-slice counts of a cut's group
            uint32_t spk[kMergeCap];                  // one segment's specials, merged
            int32_t spi[kMergeCap];
        };
    };
    int sp_n;
};

// ------------------------------------------------------------------------------------------
// Combining the slices' summaries (every slice of the unit derives the same view).  One round
// trip to L2 brings every slice header, segment array and candidate list of both rows; a
// second one, only when a cut falls inside a group of bins, brings that group's counts.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void init_row(RowView& rv, const VerifyArgs& a, const spec_params& prm) {
    rv.invT = inv_temperature(prm.temperature);
    rv.greedy = prm.temperature == 0.0f ? 1 : 0;
    rv.argmax = -1;
    rv.has_k = (prm.top_k > 0 && prm.top_k < a.V) ? 1 : 0;
    rv.has_p = ((double)prm.top_p < 1.0) ? 1 : 0;
    rv.small_k = rv.has_k && prm.top_k <= kTop;
    rv.ck = Cut{0u, 0, -1, 0, 0, 0};
    rv.cp = Cut{0u, 0, -1, 0, 0, 0};
    rv.nset = 0;
    rv.kF = 0xFFFFFFFFu;
    rv.idF = -1;
    rv.C = 1.0;
    rv.Z = 1.0;
    rv.degenerate = 0;
    rv.pend = 0;
}

__device__ __forceinline__ void stage_a(UnitSmem& us, int r, const spec_params& prm);

// Round trip 1 and what follows from it alone: row maxima, normalisers, flags, merged segment
// weights and merged candidate lists of both rows.
__device__ __forceinline__ void combine_load(const FastArgs& f, UnitSmem& us, int unit, int j, int rows, const spec_params& prm) {
    const VerifyArgs& a = f.a;
    const double T = (double)prm.temperature;
    const int nS = f.nS;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    int want[2];
    want[0] = list_len(a, prm, false);
    want[1] = rows > 1 ? draft_list_len(f, prm, j) : 0;
    // -- issue every load --
    // headers: wave r, one lane per slice (two 16-byte words and S)
    u32x4 h0 = {0, 0, 0, 0}, h1 = {0, 0, 0, 0};
    double St = 0.0;
    if (wave < rows && lane < nS) {
        const RowPart* P = part_of(f, unit, lane, wave);
        h0 = ldnt(reinterpret_cast<const u32x4*>(P));
        h1 = ldnt(reinterpret_cast<const u32x4*>(P) + 1);
        St = ldnt(&P->S);
    }
    // segment arrays, as loaded: 64 lanes per (row, slice), one word each
    constexpr int kPairs = 2 * kMaxSlices;                       // (row, slice)
    constexpr int kSegLoads = kPairs * kWave / kThreads;         // 4
    double ms[kSegLoads];
    uint32_t cs[kSegLoads];
#pragma unroll
    for (int it = 0; it < kSegLoads; ++it) {
        const int i = threadIdx.x + it * kThreads;
        const int r = i >> 10, t = (i >> 6) & (kMaxSlices - 1), sg = i & (kWave - 1);
        ms[it] = 0.0;
        cs[it] = 0u;
        if (r < rows && t < nS && sg < kSegs) {
            const RowPart* P = part_of(f, unit, t, r);
            ms[it] = ldnt(&P->seg_mass[sg]);
            cs[it] = ldnt(&P->seg_count[sg]);
        }
    }
    // candidate lists: 64 slots per (row, slice); entries past a slice's n_top are ignored
    uint32_t ck_[kSegLoads];
    int32_t ci_[kSegLoads];
#pragma unroll
    for (int it = 0; it < kSegLoads; ++it) {
        const int i = threadIdx.x + it * kThreads;
        const int r = i >> 10, t = (i >> 6) & (kMaxSlices - 1), x = i & (kWave - 1);
        ck_[it] = 0u;
        ci_[it] = 0;
        if (r < rows && t < nS && x < want[r]) {
            const RowPart* P = part_of(f, unit, t, r);
            ck_[it] = ldnt(&P->top_key[x]);
            ci_[it] = ldnt(&P->top_id[x]);
        }
    }
    // -- row headers (wave r) --
    int list_start = 0;  // wave r, lane t: where slice t's candidates start in the row's merge
    if (wave < rows) {
        RowView& rv = us.rv[wave];
        const float mt = lane < nS ? __uint_as_float(h0[0]) : -__builtin_inff();
        const uint32_t fl = h0[1], nf = h0[2], nsp = h0[3], ntop = h1[0], cnt = h1[1];
        const float m = wave_max(mt);
        const uint32_t flo = wave_or(fl);
        const uint32_t nfin = wave_sum(nf);
        const int rank = (int)wave_sum(cnt);
        const bool has_sp = __ballot(nsp > 0u) != 0;
        const double sc = (lane < nS && T > 0.0 && mt > -__builtin_inff()) ? mass_of(mt, m, inv_temperature(prm.temperature)) : 0.0;
        const double S = wave_sum(sc * St);
        const uint32_t sbits = wave_bcast(h1[2], 0);
        const int total = wave_scan(lane < nS ? (int)ntop : 0, &list_start);
        const int row_total = wave_bcast(total, kWave - 1);
        if (lane < kMaxSlices) {
            rv.sc[lane] = sc;
            rv.n_top[lane] = lane < nS ? (int)ntop : 0;
        }
        if (lane == 0) {
            init_row(rv, a, prm);
            rv.m = m;
            rv.bad = ((flo & 1u) || nfin == 0) ? 1 : 0;
            rv.overflow = (flo & 2u) ? 1 : 0;
            rv.n_finite = nfin;
            rv.has_special = has_sp ? 1 : 0;
            rv.S_all = S;
            rv.want = want[wave];
            rv.total = row_total;
            rv.s_bits = sbits;
            rv.rank_s = rank;
        }
    }
    // -- segment arrays and candidates to LDS --
#pragma unroll
    for (int it = 0; it < kSegLoads; ++it) {
        const int i = threadIdx.x + it * kThreads;
        const int r = i >> 10, t = (i >> 6) & (kMaxSlices - 1), x = i & (kWave - 1);
        if (r < rows && t < nS) {
            if (x < kSegs) {
                us.seg.mass[r][t][x] = ms[it];
                us.seg.count[r][t][x] = cs[it];
            }
            if (x < want[r]) {
                us.key[r][t * kTop + x] = ck_[it];
                us.id[r][t * kTop + x] = ci_[it];
            }
        }
    }
    __syncthreads();
    // -- merged segment weights (rescaled to the row maximum), slices in order --
    {
        const int r = threadIdx.x >> 6, sg = threadIdx.x & (kWave - 1);
        if (r < rows && sg < kSegs) {
            const RowView& rv = us.rv[r];
            double w = 0.0;
            uint32_t c = 0u;
            for (int t = 0; t < nS; ++t) {
                w += rv.sc[t] * us.seg.mass[r][t][sg];
                c += us.seg.count[r][t][sg];
            }
            us.rv[r].seg_mass[sg] = w;
            us.rv[r].seg_count[sg] = c;
        }
    }
    // -- early stage A: a row whose cuts need no merged candidate list (no greedy argmax, no
    //    top-k within the lists) settles them from the segments now (wave r, which merged the
    //    row's segments), and two other waves load the crossing group's per-slice counts while
    //    the lists merge --
    if (wave < rows) {
        RowView& rv = us.rv[wave];
        const bool early = !rv.greedy && !(rv.has_k && rv.small_k);
        if (early) stage_a(us, wave, prm);
        int g = -1;
        if (early && rv.pend != 0 && !rv.bad && !rv.overflow) g = group_of_seg(rv.pend_seg);
        if (lane == 0) {
            rv.early = early ? 1 : 0;
            rv.early_g = g;
        }
    }
    __syncthreads();
    if (wave >= 2 && wave < 2 + rows) {
        const int r = wave - 2;
        // the drafted token's mass, off the acceptance test's critical path
        if (lane == 0) {
            const uint32_t sb = us.rv[r].s_bits;
            us.rv[r].e_s = ((sb & 0x7FFFu) < 0x7F80u && T > 0.0) ? mass_of(__uint_as_float(sb << 16), us.rv[r].m, us.rv[r].invT) : 0.0;
        }
        const int g = us.rv[r].early_g;
        if (g >= 0) {
            // two counts per 32-bit word (fine counts start 4-byte aligned in a RowPart)
            static_assert(offsetof(RowPart, fine) % 4 == 0, "fine counts in 32-bit words");
            for (int i = lane; i < nS * (kGroup / 2); i += kWave) {
                const int t = i / (kGroup / 2), pr = i % (kGroup / 2);
                const uint32_t wd = ldnt(reinterpret_cast<const uint32_t*>(&part_of(f, unit, t, r)->fine[g * kGroup]) + pr);
                us.fine_ps[r][t][2 * pr] = (uint16_t)(wd & 0xFFFFu);
                us.fine_ps[r][t][2 * pr + 1] = (uint16_t)(wd >> 16);
            }
        }
    }
    // -- merged candidate lists --
    int total[2] = {0, 0};
#pragma unroll
    for (int r = 0; r < 2; ++r) total[r] = (r < rows && want[r] > 0) ? __builtin_amdgcn_readfirstlane(us.rv[r].total) : 0;
    // up to 64 candidates of a row: wave r holds one per lane and ranks each against all
    // others through lane reads
    if (wave < rows && want[wave] > 0 && total[wave] <= kWave) {
        const int r = wave;
        int t = 0, x = lane;
        for (int u = 0; u < nS; ++u) {
            const int st = wave_bcast(list_start, u);
            if (lane >= st) {
                t = u;
                x = lane - st;
            }
        }
        const bool live = lane < total[r];
        const uint32_t k = live ? us.key[r][t * kTop + x] : 0u;
        const int32_t id = live ? us.id[r][t * kTop + x] : 0;
        const uint64_t ord = ((uint64_t)k << 32) | (uint32_t)~id;  // token order (ids are non-negative)
        // lanes past the candidates hold key 0, below every candidate: reading them adds nothing
        int rank = 0;
        for (int y = 0; y < total[r]; y += 4) {
#pragma unroll
            for (int d = 0; d < 4; ++d) rank += wave_bcast(ord, y + d) > ord ? 1 : 0;
        }
        if (live && rank < want[r]) {
            us.okey[r][rank] = k;
            us.oid[r][rank] = id;
        }
    }
    // more: rank of every entry by branch-free binary searches in the other lists, up to 8
    // lists and both rows in lock-step so the LDS reads overlap
    if (total[0] > kWave || total[1] > kWave) {
        for (int i = threadIdx.x; i < nS * kTop; i += blockDim.x) {
            const int t = i >> 6, x = i & (kTop - 1);
            uint32_t k[2];
            int32_t id[2];
            uint64_t ord[2];
            int rank[2];
            bool live[2];
    #pragma unroll
            for (int r = 0; r < 2; ++r) {
                live[r] = r < rows && want[r] > 0 && total[r] > kWave && x < us.rv[r].n_top[t];
                k[r] = live[r] ? us.key[r][i] : 0u;
                id[r] = live[r] ? us.id[r][i] : 0;
                ord[r] = ((uint64_t)k[r] << 32) | (uint32_t)~id[r];
                rank[r] = x;
            }
            for (int tb = 0; tb < nS; tb += 8) {
                int pos[2][8], n[2][8];
                int nmax = 0;
    #pragma unroll
                for (int r = 0; r < 2; ++r)
    #pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int t2 = tb + u;
                        const int nt = (r < rows && want[r] > 0 && total[r] > kWave && t2 < nS) ? us.rv[r].n_top[t2] : 0;
                        nmax = max(nmax, nt);  // uniform: the same lists for every thread
                        pos[r][u] = 0;
                        n[r][u] = (live[r] && t2 != t) ? nt : 0;
                    }
                int step = 1;
                while (step * 2 <= nmax) step *= 2;
                for (; step > 0 && nmax > 0; step >>= 1) {
                    // every probe reads an address inside its list, so the reads need no branch
    #pragma unroll
                    for (int r = 0; r < 2; ++r)
    #pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            const int probe = pos[r][u] + step;
                            const int e = min(tb + u, kMaxSlices - 1) * kTop + min(probe, kTop) - 1;
                            // token order as one 64-bit comparison (ids are non-negative)
                            const uint64_t o2 = ((uint64_t)us.key[r][e] << 32) | (uint32_t)~us.id[r][e];
                            pos[r][u] = ((probe <= n[r][u]) & (o2 > ord[r])) ? probe : pos[r][u];
                        }
                }
    #pragma unroll
                for (int r = 0; r < 2; ++r)
    #pragma unroll
                    for (int u = 0; u < 8; ++u) rank[r] += pos[r][u];
            }
    #pragma unroll
            for (int r = 0; r < 2; ++r) {
                if (live[r] && rank[r] < want[r]) {
                    us.okey[r][rank[r]] = k[r];
                    us.oid[r][rank[r]] = id[r];
                }
            }
        }
    }
    if (threadIdx.x < (unsigned)rows) {
        const int r = threadIdx.x;
        us.rv[r].nm = min(total[r], want[r]);
    }
    __syncthreads();
}

// Wave-level: the crossing segment of a cut that keeps `need` weight (counts or masses) from
// the top of row rv, restricted to the `lim` cut when given; records it as rv's pending cut.
template <bool MASS>
__device__ __forceinline__ void seg_walk(RowView& rv, double need, bool has_lim, const Cut& lim) {
    const int lane = threadIdx.x & (kWave - 1);
    const int lim_seg = has_lim ? seg_of_key(lim.key) : kSegs;
    const bool live = lane < kSegs && lane < lim_seg;
    const uint32_t cnt = lane < kSegs ? rv.seg_count[lane] : 0u;
    const double ms = live ? rv.seg_mass[lane] : 0.0;
    const double w = live ? (MASS ? ms : (double)cnt) : 0.0;
    double wex, mex;
    int cex;
    const double win = wave_scan(w, &wex);
    wave_scan(ms, &mex);
    wave_scan(live ? (int)cnt : 0, &cex);
    // the walk stops at the limit's segment, which is resolved by the group walk
    const bool cross = lane < kSegs && (lane >= lim_seg || (cnt > 0u && win >= need));
    int pick = first_lane(__ballot(cross));
    if (pick < 0) {  // rounding left the target beyond the last segment: its last non-empty one
        pick = last_lane(__ballot(lane < kSegs && cnt > 0u));
        if (pick < 0) pick = kSegs - 1;
    }
    const double wa = wave_bcast(wex, pick);
    const double ma = wave_bcast(mex, pick);
    const int ca = wave_bcast(cex, pick);
    if (lane == 0) {
        rv.pend = MASS ? 2 : 1;
        rv.pend_seg = pick;
        rv.pend_need = need;
        rv.pend_above = wa;
        rv.pend_mass_above = ma;
        rv.pend_cnt_above = ca;
    }
}

// Wave-level: settles rv's pending cut inside its group from the per-slice counts in
// us.fine_ps[r]; writes *out and returns (weight kept, mass kept, elements kept) through
// the row view (S_kept / n_kept for a count cut, S / n_nuc for a mass cut).
template <bool MASS>
__device__ __forceinline__ void group_walk(const FastArgs& f, UnitSmem& us, int r, bool has_lim, const Cut& lim, Cut* out) {
    RowView& rv = us.rv[r];
    const int lane = threadIdx.x & (kWave - 1);
    const int g = group_of_seg(rv.pend_seg);
    const int bb = kGroup - 1 - lane;  // lane order = descending key
    const int bin = g * kGroup + bb;
    const uint32_t key = bin_key(bin);
    int n = 0;
    for (int t = 0; t < f.nS; ++t) n += us.fine_ps[r][t][bb];
    const bool at_lim = has_lim && key == lim.key;
    if (has_lim && key < lim.key) n = 0;
    if (at_lim) n = min(n, lim.take);
    const double e = n > 0 ? mass_of(key16_value(key), rv.m, rv.invT) : 0.0;
    const double w = MASS ? (double)n * e : (double)n;
    double wex, mex;
    int nex;
    const double win = wave_scan(w, &wex);
    wave_scan((double)n * e, &mex);
    wave_scan(n, &nex);
    const double need = rv.pend_need, above0 = rv.pend_above;
    const uint64_t hc = __ballot(n > 0 && (above0 + win >= need || at_lim));
    const bool done = hc != 0;
    // not done: rounding left the target just beyond the group; cut at its lowest bin
    const int sel = done ? first_lane(hc) : last_lane(__ballot(n > 0));
    Cut c{0u, 0, -1, 0, 0, rv.pend_cnt_above};
    double kept_w = above0, kept_m = rv.pend_mass_above;
    int kept_n = rv.pend_cnt_above;
    if (sel >= 0) {
        const double above = above0 + wave_bcast(wex, sel);
        const double e_s = wave_bcast(e, sel);
        const int n_s = wave_bcast(n, sel);
        const int nex_s = wave_bcast(nex, sel);
        int take = n_s;
        if (done && above + (MASS ? (double)n_s * e_s : (double)n_s) >= need) {
            if (MASS) {
                if (e_s > 0.0) {
                    const double q = ceil((need - above) / e_s);
                    take = q < 1.0 ? 1 : (q > (double)n_s ? n_s : (int)q);
                }
            } else {
                take = (int)(need - above);
                take = take < 1 ? 1 : (take > n_s ? n_s : take);
            }
        }
        c.key = bin_key(g * kGroup + (kGroup - 1 - sel));
        c.take = take;
        c.count_above = rv.pend_cnt_above + nex_s;
        kept_w = above + (MASS ? (double)take * e_s : (double)take);
        kept_m = rv.pend_mass_above + wave_bcast(mex, sel) + (double)take * e_s;
        kept_n = c.count_above + take;
        // the slice holding the last kept element at the cut key
        const int bsel = kGroup - 1 - sel;
        const int nt = lane < f.nS ? (int)us.fine_ps[r][lane][bsel] : 0;
        int tex;
        const int tin = wave_scan(nt, &tex);
        const int own = first_lane(__ballot(lane < f.nS && tin >= take));
        if (own < 0) {
            c.owner = f.nS - 1;
            c.owner_take = 0;
        } else {
            c.owner = own;
            c.owner_take = take - wave_bcast(tex, own);
        }
    }
    if (lane == 0) {
        *out = c;
        if (MASS) {
            rv.S = kept_w;
            rv.n_nuc = kept_n;
        } else {
            rv.S_kept = kept_m;
            rv.n_kept = kept_n;
        }
        rv.pend = 0;
    }
}

// Specials of segment sg of row r from every slice, sorted (key desc, id asc) into
// us.spk / spi; returns their number.  (Rare: finite values outside the exact bins.)
__device__ __forceinline__ int merge_specials(const FastArgs& f, UnitSmem& us, int unit, int r, int sg) {
    if (threadIdx.x == 0) us.sp_n = 0;
    __syncthreads();
    constexpr int kCap = kMergeCap;
    for (int i = threadIdx.x; i < f.nS * kSpecial; i += blockDim.x) {
        const RowPart* P = part_of(f, unit, i / kSpecial, r);
        const int x = i % kSpecial;
        if (x >= min((int)ldnt(&P->n_special), kSpecial)) continue;
        const uint32_t k = ldnt(&P->sp_key[x]);
        if (special_seg(k) != sg) continue;
        const int slot = atomicAdd(&us.sp_n, 1);
        if (slot < kCap) {
            us.key[0][slot] = k;  // staging (the candidate lists are no longer needed)
            us.id[0][slot] = ldnt(&P->sp_id[x]);
        }
    }
    __syncthreads();
    const int n = min(us.sp_n, kCap);
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const uint32_t k = us.key[0][i];
        const int id = us.id[0][i];
        int rank = 0;
        for (int x = 0; x < n; ++x) {
            const uint32_t k2 = us.key[0][x];
            rank += (k2 > k || (k2 == k && us.id[0][x] < id)) ? 1 : 0;
        }
        us.spk[rank] = k;
        us.spi[rank] = id;
    }
    __syncthreads();
    return n;
}

// Block-level (rare): settles rv's pending cut when it falls among the specials of a segment.
template <bool MASS>
__device__ __forceinline__ void special_walk(const FastArgs& f, UnitSmem& us, int unit, int r, bool has_lim, const Cut& lim,
                                             Cut* out) {
    RowView& rv = us.rv[r];
    const int n = merge_specials(f, us, unit, r, rv.pend_seg);
    if (threadIdx.x == 0) {
        double above = rv.pend_above, mass = rv.pend_mass_above;
        const double need = rv.pend_need;
        Cut c{0u, 0, -1, 0, 0, rv.pend_cnt_above};
        int i = 0;
        for (; i < n; ++i) {
            const uint32_t key = us.spk[i];
            if (has_lim && (key < lim.key || (key == lim.key && lim.explicit_id >= 0 && us.spi[i] > lim.explicit_id))) break;
            const double e = mass_of(key16_value(key), rv.m, rv.invT);
            above += MASS ? e : 1.0;
            mass += e;
            if (above >= need) {
                c.key = key;
                c.explicit_id = us.spi[i];
                ++i;
                break;
            }
        }
        if (c.explicit_id < 0 && i > 0) {  // the limit (or rounding) ends the walk
            c.key = us.spk[i - 1];
            c.explicit_id = us.spi[i - 1];
        }
        *out = c;
        if (MASS) {
            rv.S = above;
            rv.n_nuc = rv.pend_cnt_above + i;
        } else {
            rv.S_kept = mass;
            rv.n_kept = rv.pend_cnt_above + i;
        }
        rv.pend = 0;
    }
    __syncthreads();
}

// Wave-level step of row r after its top-k is settled: the nucleus, settled at once or left
// as a pending cut.
__device__ __forceinline__ void nucleus_step(UnitSmem& us, int r, const spec_params& prm) {
    RowView& rv = us.rv[r];
    const int lane = threadIdx.x & (kWave - 1);
    if (!rv.has_p) {
        if (lane == 0) {
            rv.S = rv.S_kept;
            rv.n_nuc = rv.n_kept;
        }
    } else if (rv.small_k) {  // inside the merged list
        const int kk = prm.top_k;
        const double need = (double)prm.top_p * rv.S_kept;
        const double e = lane < kk ? mass_of(key16_value(us.okey[r][lane]), rv.m, rv.invT) : 0.0;
        double ex;
        const double in = wave_scan(e, &ex);
        int i = first_lane(__ballot(lane < kk && in >= need));
        if (i < 0) i = kk - 1;
        const double cum = wave_bcast(in, i);
        if (lane == 0) {
            rv.cp = Cut{us.okey[r][i], 0, us.oid[r][i], 0, 0, 0};
            rv.S = cum;
            rv.n_nuc = i + 1;
        }
    } else {
        const bool use_lim = rv.has_k && rv.ck.key != 0u;
        seg_walk<true>(rv, (double)prm.top_p * rv.S_kept, use_lim, rv.ck);
    }
}

__device__ __forceinline__ bool cut_keeps_s(const RowView& rv, const Cut& c, uint32_t key_s, int s) {
    if (key_s > c.key) return true;
    if (key_s < c.key) return false;
    if (c.explicit_id >= 0) return s <= c.explicit_id;
    return rv.rank_s < c.take;
}

// Processed probability of token s in row r (after the combine).
__device__ __forceinline__ double prob_of_s(const UnitSmem& us, int r, int s, bool draft) {
    const RowView& rv = us.rv[r];
    const uint32_t h = rv.s_bits;
    if ((h & 0x7FFFu) >= 0x7F80u) return 0.0;
    const uint32_t key = key16(h);
    if (rv.has_k && !cut_keeps_s(rv, rv.ck, key, s)) return 0.0;
    if (rv.has_p && !cut_keeps_s(rv, rv.cp, key, s)) return 0.0;
    const double e = rv.e_s;
    const double p = e / rv.S;
    if (!draft) return p;
    const double fct = (rv.nset > 0 && e > 0.0 && in_cut_id(rv.kF, rv.idF, key, s)) ? rv.C : 1.0;
    return (p * fct) / rv.Z;
}

// Stage A of row r (wave r): top-k, then the nucleus where it needs no group counts; a cut
// that crosses a group is left pending.
__device__ __forceinline__ void stage_a(UnitSmem& us, int r, const spec_params& prm) {
    RowView& rv = us.rv[r];
    const int lane = threadIdx.x & (kWave - 1);
    if (rv.bad || rv.overflow) {
        // nothing to settle
    } else if (rv.greedy) {
        if (lane == 0) rv.argmax = rv.nm > 0 ? us.oid[r][0] : -1;
    } else if (rv.has_k && (uint32_t)prm.top_k > rv.n_finite) {  // -inf tokens would be kept
        if (lane == 0) rv.overflow = 1;
    } else {
        if (!rv.has_k) {
            if (lane == 0) {
                rv.S_kept = rv.S_all;
                rv.n_kept = (int)rv.n_finite;
            }
        } else if (rv.small_k) {
            const int kk = prm.top_k;
            const double e = lane < kk ? mass_of(key16_value(us.okey[r][lane]), rv.m, rv.invT) : 0.0;
            const double s = wave_sum(e);
            if (lane == 0) {
                rv.S_kept = s;
                rv.n_kept = kk;
                rv.ck = Cut{us.okey[r][kk - 1], 0, us.oid[r][kk - 1], 0, 0, 0};
            }
        } else {
            seg_walk<false>(rv, (double)prm.top_k, false, rv.ck);
        }
        if (rv.pend == 0) nucleus_step(us, r, prm);
    }
}

// Both rows' processed distributions: maxima, normalisers, top-k and nucleus cuts, and (dw)
// the draft row's downweighted set.  All threads.
__device__ __forceinline__ void combine(const FastArgs& f, UnitSmem& us, int unit, int j, int rows, const spec_params& prm,
                                        bool dw, int s_tok) {
    const VerifyArgs& a = f.a;
    combine_load(f, us, unit, j, rows, prm);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    // top-k, then the nucleus where it needs no group counts (wave r for row r), unless the
    // row settled them before the candidate merge
    if (wave < rows && !us.rv[wave].early) stage_a(us, wave, prm);
    __syncthreads();
    // pending histogram cuts: load their groups' per-slice counts, settle, repeat (a top-k cut
    // can leave a nucleus cut behind it)
    for (int round = 0; round < 2; ++round) {
        const bool p0 = us.rv[0].pend != 0;
        const bool p1 = rows > 1 && us.rv[1].pend != 0;
        if (!p0 && !p1) break;
        // (round 0: a row whose counts were loaded during the candidate merge has them already)
        const int g0 = (p0 && !(round == 0 && us.rv[0].early_g >= 0)) ? group_of_seg(us.rv[0].pend_seg) : -1;
        const int g1 = (p1 && !(round == 0 && us.rv[1].early_g >= 0)) ? group_of_seg(us.rv[1].pend_seg) : -1;
        for (int i = threadIdx.x; i < 2 * f.nS * kGroup; i += blockDim.x) {
            const int r = i / (f.nS * kGroup), t = (i / kGroup) % f.nS, bb = i % kGroup;
            const int g = r == 0 ? g0 : g1;
            if (g >= 0) us.fine_ps[r][t][bb] = (uint16_t)ldnt_u16(&part_of(f, unit, t, r)->fine[g * kGroup + bb]);
        }
        __syncthreads();
        // the rows' pending cuts as they stand before the walks
        bool count_cut[2], in_groups[2], pend[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            pend[r] = r == 0 ? p0 : p1;
            count_cut[r] = pend[r] && us.rv[r].pend == 1;
            in_groups[r] = pend[r] && group_of_seg(us.rv[r].pend_seg) >= 0;
        }
        // cuts inside an exact group: wave r walks row r, both rows at once
        if (wave < rows && in_groups[wave]) {
            RowView& rv = us.rv[wave];
            const Cut lim = rv.ck;
            if (count_cut[wave]) group_walk<false>(f, us, wave, false, lim, &rv.ck);
            else group_walk<true>(f, us, wave, rv.has_k && rv.ck.key != 0u, lim, &rv.cp);
        }
        // cuts among the special values: the whole workgroup, one row at a time
        for (int r = 0; r < rows; ++r) {
            if (!pend[r] || in_groups[r]) continue;
            RowView& rv = us.rv[r];
            const Cut lim = rv.ck;
            if (count_cut[r]) special_walk<false>(f, us, unit, r, false, lim, &rv.ck);
            else special_walk<true>(f, us, unit, r, rv.has_k && rv.ck.key != 0u, lim, &rv.cp);
        }
        __syncthreads();
        if (wave < rows && count_cut[wave]) nucleus_step(us, wave, prm);
        __syncthreads();
    }
    // downweighted set: the first F elements of the processed order that carry mass
    if (dw && rows > 1 && wave == 1) {
        RowView& rv = us.rv[1];
        const bool want_set = a.F > 0 && a.C < 1.0f && !rv.greedy && !rv.bad && !rv.overflow;
        if (want_set) {
            const int n0 = min(min(a.F, rv.n_nuc), rv.nm);
            const double e = lane < n0 ? mass_of(key16_value(us.okey[1][lane]), rv.m, rv.invT) : 0.0;
            const int n = last_lane(__ballot(lane < n0 && e > 0.0)) + 1;
            const double ps = wave_sum(lane < n ? e / rv.S : 0.0);
            if (lane == 0) {
                rv.nset = n;
                if (n > 0) {
                    rv.kF = us.okey[1][n - 1];
                    rv.idF = us.oid[1][n - 1];
                    const double Cd = (double)a.C;
                    const double Z = 1.0 - (1.0 - Cd) * ps;
                    if (Z > 0.0) {
                        rv.C = Cd;
                        rv.Z = Z;
                    } else {
                        rv.degenerate = 1;
                    }
                }
            }
        }
    }
    // the drafted token's processed probabilities for the acceptance test: lane 0 of wave 0
    // (target row) and of wave 1 (draft row, after its set; none for a uniform draft)
    if (dw && s_tok >= 0 && s_tok < a.V && wave < rows && lane == 0 && !us.rv[wave].greedy) {
        const double p = prob_of_s(us, wave, s_tok, wave == 1);
        if (wave == 0) us.qs = p;
        else us.ps = p;
    }
    __syncthreads();
}

}  // namespace fast
}  // namespace sv
