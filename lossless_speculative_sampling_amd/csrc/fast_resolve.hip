// Resolve kernel of the bf16 verification path: every slice of a unit combines the unit's
// slice summaries into the exact processed distributions, tests acceptance, sums the
// residual where the unit needs it, and the last workgroup of a request picks k and t*.
#include "fast_common.h"
#include "rowproc.h"

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
    double T;
    double sc[kMaxSlices];     // per-slice rescale exp((m_t - m)/T)
    int n_top[kMaxSlices];     // per-slice candidate list lengths
    double seg_mass[kSegs];
    uint32_t seg_count[kSegs];
    uint32_t n_finite;
    int has_special;
    int want;                  // candidates each slice lists
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
    int rank_s;
    // a histogram cut in progress (0 none, 1 top-k count cut, 2 nucleus mass cut)
    int pend;
    int pend_seg;
    int pend_cnt_above;
    double pend_need;
    double pend_above;
    double pend_mass_above;
};

struct Smem {
    UnitRec urec;
    union {
        double tab[2][kBins];      // residual tables
        struct {
            uint32_t key[2][kMergeCap];   // every slice's candidate list, slice-major
            int32_t id[2][kMergeCap];
            uint32_t okey[2][kTop];       // merged candidates in token order
            int32_t oid[2][kTop];
            uint16_t fine_ps[2][kMaxSlices][kGroup];  // per-slice counts of a cut's group
            uint32_t spk[kMergeCap / 2];  // one segment's specials, merged
            int32_t spi[kMergeCap / 2];
        } m;
        RowShared generic;
    } u;
    RowStats gst[2];
    int32_t scan[kWaves + 1];
    double redd[kWaves];
    int32_t redi[kWaves];
    RowView rv[2];
    int last;
    int found;
    int sp_n;
    int any_pend;
    uint32_t fin[2 * sizeof(RowFinal) / 4];
    int fk, ft, fmode, fc;
    uint32_t fstatus;
    double fW, ftarget, fbase;
};

// ------------------------------------------------------------------------------------------
// Combining the slices' summaries (every slice of the unit derives the same view).  One round
// trip to L2 brings every slice header, segment array and candidate list of both rows; a
// second one, only when a cut falls inside a group of bins, brings that group's counts.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void init_row(RowView& rv, const VerifyArgs& a, const spec_params& prm) {
    rv.T = (double)prm.temperature;
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
    rv.nm = 0;
}

// Round trip 1 and what follows from it alone: row maxima, normalisers, flags, merged segment
// weights and merged candidate lists of both rows.
__device__ __forceinline__ void combine_load(const FastArgs& f, Smem& sm, int unit, int rows, const spec_params& prm) {
    const VerifyArgs& a = f.a;
    const double T = (double)prm.temperature;
    const int nS = f.nS;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    int want[2];
    want[0] = list_len(a, prm, false);
    want[1] = rows > 1 ? list_len(a, prm, true) : 0;
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
    // segment arrays: eight lanes per (row, segment), slices t and t + 8 each
    constexpr int kSegItems = kSegs * 8;
    double ms[2][2];
    uint32_t cs[2][2];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int i = threadIdx.x + it * kThreads;
        const int r = i / kSegItems, sg = (i % kSegItems) / 8, t0 = i % 8;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int t = t0 + 8 * hh;
            ms[it][hh] = 0.0;
            cs[it][hh] = 0u;
            if (r < rows && t < nS) {
                const RowPart* P = part_of(f, unit, t, r);
                ms[it][hh] = ldnt(&P->seg_mass[sg]);
                cs[it][hh] = ldnt(&P->seg_count[sg]);
            }
        }
    }
    // candidate lists (entries past a slice's n_top are ignored later)
    uint32_t ck_[2][2];
    int32_t ci_[2][2];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int i = threadIdx.x + it * kThreads;
            ck_[r][it] = 0u;
            ci_[r][it] = 0;
            if (r < rows && i < nS * want[r]) {
                const RowPart* P = part_of(f, unit, i / want[r], r);
                ck_[r][it] = ldnt(&P->top_key[i % want[r]]);
                ci_[r][it] = ldnt(&P->top_id[i % want[r]]);
            }
        }
    // -- row headers (wave r) --
    if (wave < rows) {
        RowView& rv = sm.rv[wave];
        const float mt = lane < nS ? __uint_as_float(h0[0]) : -__builtin_inff();
        const uint32_t fl = h0[1], nf = h0[2], nsp = h0[3], ntop = h1[0], cnt = h1[1];
        const float m = wave_max(mt);
        const uint32_t flo = wave_or(fl);
        const uint32_t nfin = wave_sum(nf);
        const int rank = (int)wave_sum(cnt);
        const bool has_sp = __ballot(nsp > 0u) != 0;
        const double sc = (lane < nS && T > 0.0 && mt > -__builtin_inff()) ? exp(((double)mt - (double)m) / T) : 0.0;
        const double S = wave_sum(sc * St);
        const uint32_t sbits = wave_bcast(h1[2], 0);
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
            rv.s_bits = sbits;
            rv.rank_s = rank;
        }
    }
    // -- candidates to LDS --
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int i = threadIdx.x + it * kThreads;
            if (r < rows && i < nS * want[r]) {
                sm.u.m.key[r][i] = ck_[r][it];
                sm.u.m.id[r][i] = ci_[r][it];
            }
        }
    __syncthreads();
    // -- merged segment weights (rescaled to the row maximum) --
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int i = threadIdx.x + it * kThreads;
        const int r = i / kSegItems, sg = (i % kSegItems) / 8, t0 = i % 8;
        const bool live = r < rows;   // uniform over each group of eight lanes
        if (i < 2 * kSegItems) {
            const RowView& rv = sm.rv[live ? r : 0];
            double w = 0.0;
            if (live) {
                if (t0 < nS) w += rv.sc[t0] * ms[it][0];
                if (t0 + 8 < nS) w += rv.sc[t0 + 8] * ms[it][1];
            }
            const double wsum = group8_sum(w);
            const uint32_t csum = group8_sum(cs[it][0] + cs[it][1]);
            if (live && t0 == 0) {
                sm.rv[r].seg_mass[sg] = wsum;
                sm.rv[r].seg_count[sg] = csum;
            }
        }
    }
    // -- merged candidate lists: rank of every entry by binary search in the other lists --
    for (int r = 0; r < rows; ++r) {
        const int per = want[r];
        if (per == 0) continue;
        const RowView& rv = sm.rv[r];
        for (int i = threadIdx.x; i < nS * per; i += blockDim.x) {
            const int t = i / per, x = i % per;
            if (x >= rv.n_top[t]) continue;
            const uint32_t k = sm.u.m.key[r][i];
            const int id = sm.u.m.id[r][i];
            int rank = x;
            for (int t2 = 0; t2 < nS; ++t2) {
                if (t2 == t) continue;
                int lo = 0, hi = rv.n_top[t2];
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    const uint32_t k2 = sm.u.m.key[r][t2 * per + mid];
                    const bool before = k2 > k || (k2 == k && sm.u.m.id[r][t2 * per + mid] < id);
                    if (before) lo = mid + 1;
                    else hi = mid;
                }
                rank += lo;
            }
            if (rank < per) {
                sm.u.m.okey[r][rank] = k;
                sm.u.m.oid[r][rank] = id;
            }
        }
        if (threadIdx.x == 0) {
            int tot = 0;
            for (int t = 0; t < nS; ++t) tot += rv.n_top[t];
            sm.rv[r].nm = min(tot, per);
        }
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
// sm.u.m.fine_ps[r]; writes *out and returns (weight kept, mass kept, elements kept) through
// the row view (S_kept / n_kept for a count cut, S / n_nuc for a mass cut).
template <bool MASS>
__device__ __forceinline__ void group_walk(const FastArgs& f, Smem& sm, int r, bool has_lim, const Cut& lim, Cut* out) {
    RowView& rv = sm.rv[r];
    const int lane = threadIdx.x & (kWave - 1);
    const int g = group_of_seg(rv.pend_seg);
    const int bb = kGroup - 1 - lane;  // lane order = descending key
    const int bin = g * kGroup + bb;
    const uint32_t key = bin_key(bin);
    int n = 0;
    for (int t = 0; t < f.nS; ++t) n += sm.u.m.fine_ps[r][t][bb];
    const bool at_lim = has_lim && key == lim.key;
    if (has_lim && key < lim.key) n = 0;
    if (at_lim) n = min(n, lim.take);
    const double e = n > 0 ? mass_of(key16_value(key), rv.m, rv.T) : 0.0;
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
        const int nt = lane < f.nS ? (int)sm.u.m.fine_ps[r][lane][bsel] : 0;
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
// sm.u.m.spk / spi; returns their number.  (Rare: finite values outside the exact bins.)
__device__ __forceinline__ int merge_specials(const FastArgs& f, Smem& sm, int unit, int r, int sg) {
    if (threadIdx.x == 0) sm.sp_n = 0;
    __syncthreads();
    constexpr int kCap = kMergeCap / 2;
    for (int i = threadIdx.x; i < f.nS * kSpecial; i += blockDim.x) {
        const RowPart* P = part_of(f, unit, i / kSpecial, r);
        const int x = i % kSpecial;
        if (x >= min((int)ldnt(&P->n_special), kSpecial)) continue;
        const uint32_t k = ldnt(&P->sp_key[x]);
        if (special_seg(k) != sg) continue;
        const int slot = atomicAdd(&sm.sp_n, 1);
        if (slot < kCap) {
            sm.u.m.key[0][kCap + slot] = k;  // staging (the candidate lists are no longer needed)
            sm.u.m.id[0][kCap + slot] = ldnt(&P->sp_id[x]);
        }
    }
    __syncthreads();
    const int n = min(sm.sp_n, kCap);
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const uint32_t k = sm.u.m.key[0][kCap + i];
        const int id = sm.u.m.id[0][kCap + i];
        int rank = 0;
        for (int x = 0; x < n; ++x) {
            const uint32_t k2 = sm.u.m.key[0][kCap + x];
            rank += (k2 > k || (k2 == k && sm.u.m.id[0][kCap + x] < id)) ? 1 : 0;
        }
        sm.u.m.spk[rank] = k;
        sm.u.m.spi[rank] = id;
    }
    __syncthreads();
    return n;
}

// Block-level (rare): settles rv's pending cut when it falls among the specials of a segment.
template <bool MASS>
__device__ __forceinline__ void special_walk(const FastArgs& f, Smem& sm, int unit, int r, bool has_lim, const Cut& lim,
                                             Cut* out) {
    RowView& rv = sm.rv[r];
    const int n = merge_specials(f, sm, unit, r, rv.pend_seg);
    if (threadIdx.x == 0) {
        double above = rv.pend_above, mass = rv.pend_mass_above;
        const double need = rv.pend_need;
        Cut c{0u, 0, -1, 0, 0, rv.pend_cnt_above};
        int i = 0;
        for (; i < n; ++i) {
            const uint32_t key = sm.u.m.spk[i];
            if (has_lim && (key < lim.key || (key == lim.key && lim.explicit_id >= 0 && sm.u.m.spi[i] > lim.explicit_id))) break;
            const double e = mass_of(key16_value(key), rv.m, rv.T);
            above += MASS ? e : 1.0;
            mass += e;
            if (above >= need) {
                c.key = key;
                c.explicit_id = sm.u.m.spi[i];
                ++i;
                break;
            }
        }
        if (c.explicit_id < 0 && i > 0) {  // the limit (or rounding) ends the walk
            c.key = sm.u.m.spk[i - 1];
            c.explicit_id = sm.u.m.spi[i - 1];
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
__device__ __forceinline__ void nucleus_step(Smem& sm, int r, const spec_params& prm) {
    RowView& rv = sm.rv[r];
    const int lane = threadIdx.x & (kWave - 1);
    if (!rv.has_p) {
        if (lane == 0) {
            rv.S = rv.S_kept;
            rv.n_nuc = rv.n_kept;
        }
    } else if (rv.small_k) {  // inside the merged list
        const int kk = prm.top_k;
        const double need = (double)prm.top_p * rv.S_kept;
        const double e = lane < kk ? mass_of(key16_value(sm.u.m.okey[r][lane]), rv.m, rv.T) : 0.0;
        double ex;
        const double in = wave_scan(e, &ex);
        int i = first_lane(__ballot(lane < kk && in >= need));
        if (i < 0) i = kk - 1;
        const double cum = wave_bcast(in, i);
        if (lane == 0) {
            rv.cp = Cut{sm.u.m.okey[r][i], 0, sm.u.m.oid[r][i], 0, 0, 0};
            rv.S = cum;
            rv.n_nuc = i + 1;
        }
    } else {
        const bool use_lim = rv.has_k && rv.ck.key != 0u;
        seg_walk<true>(rv, (double)prm.top_p * rv.S_kept, use_lim, rv.ck);
    }
}

// Both rows' processed distributions: maxima, normalisers, top-k and nucleus cuts, and the
// draft row's downweighted set.  All threads.
__device__ __forceinline__ void combine(const FastArgs& f, Smem& sm, int unit, int rows, const spec_params& prm) {
    const VerifyArgs& a = f.a;
    combine_load(f, sm, unit, rows, prm);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    // top-k, then the nucleus where it needs no group counts (wave r for row r)
    if (wave < rows) {
        RowView& rv = sm.rv[wave];
        const int r = wave;
        if (rv.bad || rv.overflow) {
            // nothing to settle
        } else if (rv.greedy) {
            if (lane == 0) rv.argmax = rv.nm > 0 ? sm.u.m.oid[r][0] : -1;
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
                const double e = lane < kk ? mass_of(key16_value(sm.u.m.okey[r][lane]), rv.m, rv.T) : 0.0;
                const double s = wave_sum(e);
                if (lane == 0) {
                    rv.S_kept = s;
                    rv.n_kept = kk;
                    rv.ck = Cut{sm.u.m.okey[r][kk - 1], 0, sm.u.m.oid[r][kk - 1], 0, 0, 0};
                }
            } else {
                seg_walk<false>(rv, (double)prm.top_k, false, rv.ck);
            }
            if (rv.pend == 0) nucleus_step(sm, r, prm);
        }
    }
    __syncthreads();
    // pending histogram cuts: load their groups' per-slice counts, settle, repeat (a top-k cut
    // can leave a nucleus cut behind it)
    for (int round = 0; round < 2; ++round) {
        const bool p0 = sm.rv[0].pend != 0;
        const bool p1 = rows > 1 && sm.rv[1].pend != 0;
        if (!p0 && !p1) break;
        const int g0 = p0 ? group_of_seg(sm.rv[0].pend_seg) : -1;
        const int g1 = p1 ? group_of_seg(sm.rv[1].pend_seg) : -1;
        for (int i = threadIdx.x; i < 2 * f.nS * kGroup; i += blockDim.x) {
            const int r = i / (f.nS * kGroup), t = (i / kGroup) % f.nS, bb = i % kGroup;
            const int g = r == 0 ? g0 : g1;
            if (g >= 0) sm.u.m.fine_ps[r][t][bb] = (uint16_t)ldnt_u16(&part_of(f, unit, t, r)->fine[g * kGroup + bb]);
        }
        __syncthreads();
        for (int r = 0; r < rows; ++r) {
            RowView& rv = sm.rv[r];
            if (rv.pend == 0) continue;
            const bool count_cut = rv.pend == 1;
            const bool use_lim = !count_cut && rv.has_k && rv.ck.key != 0u;
            const Cut lim = rv.ck;
            if (group_of_seg(rv.pend_seg) >= 0) {
                if (wave == r) {
                    if (count_cut) group_walk<false>(f, sm, r, false, lim, &rv.ck);
                    else group_walk<true>(f, sm, r, use_lim, lim, &rv.cp);
                }
            } else {
                if (count_cut) special_walk<false>(f, sm, unit, r, false, lim, &rv.ck);
                else special_walk<true>(f, sm, unit, r, use_lim, lim, &rv.cp);
            }
            __syncthreads();
            if (count_cut && wave == r) nucleus_step(sm, r, prm);
        }
        __syncthreads();
    }
    // downweighted set: the first F elements of the processed order that carry mass
    if (rows > 1 && wave == 1) {
        RowView& rv = sm.rv[1];
        const bool want_set = a.F > 0 && a.C < 1.0f && !rv.greedy && !rv.bad && !rv.overflow;
        if (want_set) {
            const int n0 = min(min(a.F, rv.n_nuc), rv.nm);
            const double e = lane < n0 ? mass_of(key16_value(sm.u.m.okey[1][lane]), rv.m, rv.T) : 0.0;
            const int n = last_lane(__ballot(lane < n0 && e > 0.0)) + 1;
            const double ps = wave_sum(lane < n ? e / rv.S : 0.0);
            if (lane == 0) {
                rv.nset = n;
                if (n > 0) {
                    rv.kF = sm.u.m.okey[1][n - 1];
                    rv.idF = sm.u.m.oid[1][n - 1];
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
    __syncthreads();
}

// ------------------------------------------------------------------------------------------
// Per-element helpers shared by the slices and the finaliser
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ bool in_cut_id(uint32_t cut_key, int cut_id, uint32_t key, int col) {
    return key > cut_key || (key == cut_key && col <= cut_id);
}

// Processed probability of one element from the row's final statistics and true id cuts
// (same operation order as the slices' tables: ((e / S) * f) / Z).
__device__ __forceinline__ double final_prob(const RowFinal& rf, int idk, int idp, uint32_t h, int col, bool draft) {
    const uint32_t mag = h & 0x7FFFu;
    if (mag >= 0x7F80u) return 0.0;  // -inf (bad rows never reach here)
    if (rf.greedy) return col == rf.argmax ? 1.0 : 0.0;
    const uint32_t key = key16(h);
    if (!in_cut_id(rf.kk, idk, key, col) || !in_cut_id(rf.kp, idp, key, col)) return 0.0;
    const double e = mass_of(__uint_as_float(h << 16), rf.m, (double)rf.T);
    const double p = e / rf.S;
    if (!draft) return p;
    const double fct = (rf.nS > 0 && e > 0.0 && in_cut_id(rf.kF, rf.idF, key, col)) ? rf.C : 1.0;
    return (p * fct) / rf.Z;
}

// The n-th (1-based) element of this slice, in token order, whose key equals `key`.
__device__ __forceinline__ int local_nth_at_key(Smem& sm, const u32x4 (&v)[kLoads], int c0, int V, uint32_t key, int n) {
    if (threadIdx.x == 0) sm.found = -1;
    __syncthreads();
    int base = 0;
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
        if (base >= n) break;  // uniform
        uint32_t mq = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int col = col_of(c0, q, e);
            const uint32_t w = v[q][e >> 1];
            const uint32_t h = (e & 1) ? (w >> 16) : (w & 0xFFFFu);
            if (col < V && (h & 0x7FFFu) < 0x7F80u && key16(h) == key) mq |= 1u << e;
        }
        int total;
        const int before = block_exclusive_scan<int>(__popc(mq), sm.scan, &total);
        if (base + before < n && base + before + __popc(mq) >= n) {
            int k = base + before;
            for (int e = 0; e < 8; ++e)
                if ((mq & (1u << e)) && ++k == n) {
                    sm.found = col_of(c0, q, e);
                    break;
                }
        }
        base += total;
    }
    __syncthreads();
    const int r = sm.found;
    __syncthreads();
    return r;
}

// This slice's id cut at a cut's key: all ties (V-1), none (-1), or the owner's exact id.
__device__ __forceinline__ int effective_id(Smem& sm, const Cut& c, int slice, const u32x4 (&v)[kLoads], int c0, int V) {
    if (c.explicit_id >= 0) return c.explicit_id;
    if (c.key == 0) return V - 1;
    if (slice < c.owner) return V - 1;
    if (slice > c.owner) return -1;
    return local_nth_at_key(sm, v, c0, V, c.key, c.owner_take);
}

__device__ __forceinline__ bool cut_keeps_s(const RowView& rv, const Cut& c, uint32_t key_s, int s) {
    if (key_s > c.key) return true;
    if (key_s < c.key) return false;
    if (c.explicit_id >= 0) return s <= c.explicit_id;
    return rv.rank_s < c.take;
}

// Processed probability of token s in row r (after the combine).
__device__ __forceinline__ double prob_of_s(const Smem& sm, int r, int s, bool draft) {
    const RowView& rv = sm.rv[r];
    const uint32_t h = rv.s_bits;
    if ((h & 0x7FFFu) >= 0x7F80u) return 0.0;
    const uint32_t key = key16(h);
    if (rv.has_k && !cut_keeps_s(rv, rv.ck, key, s)) return 0.0;
    if (rv.has_p && !cut_keeps_s(rv, rv.cp, key, s)) return 0.0;
    const double e = mass_of(__uint_as_float(h << 16), rv.m, rv.T);
    const double p = e / rv.S;
    if (!draft) return p;
    const double fct = (rv.nset > 0 && e > 0.0 && in_cut_id(rv.kF, rv.idF, key, s)) ? rv.C : 1.0;
    return (p * fct) / rv.Z;
}

// Residual (rejected draft position) or target (bonus position) mass of this slice over
// 512-column chunks, in token order.
__device__ __forceinline__ void residual_chunks(const FastArgs& f, Smem& sm, int unit, int slice, int c0, bool two,
                                const u32x4 (&vq)[kLoads], const u32x4 (&vp)[kLoads], const int (&eff)[2][2]) {
    const VerifyArgs& a = f.a;
    const RowView& rq = sm.rv[0];
    const RowView& rp = sm.rv[1];
    // per-bin values: q = e / S, p' = ((e / S) * f) / Z; ties at a cut key are settled per element
    for (int b = threadIdx.x; b < kBins; b += blockDim.x) {
        const uint32_t key = bin_key(b);
        const float z = key16_value(key);
        {
            const bool in = (!rq.has_k || key >= rq.ck.key) && (!rq.has_p || key >= rq.cp.key);
            sm.u.tab[0][b] = in ? mass_of(z, rq.m, rq.T) / rq.S : 0.0;
        }
        if (two) {
            const bool in = (!rp.has_k || key >= rp.ck.key) && (!rp.has_p || key >= rp.cp.key);
            double pv = in ? mass_of(z, rp.m, rp.T) / rp.S : 0.0;
            if (rp.nset > 0 && key == rp.kF) {
                // raw e / S; the set membership of ties is settled per element
            } else {
                const double fct = (rp.nset > 0 && pv > 0.0 && key > rp.kF) ? rp.C : 1.0;
                pv = (pv * fct) / rp.Z;
            }
            sm.u.tab[1][b] = pv;
        }
    }
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    double* out = reinterpret_cast<double*>(f.ws + f.L.chunks) + ((size_t)unit * f.nS + slice) * kChunks;
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
        double acc = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int col = col_of(c0, q, e);
            if (col >= a.V) continue;
            double qv = 0.0, pv = 0.0;
            {
                const uint32_t w = vq[q][e >> 1];
                const uint32_t h = (e & 1) ? (w >> 16) : (w & 0xFFFFu);
                int bin;
                const int kind = classify(h, &bin);
                const uint32_t key = key16(h);
                if (kind == kKindBin) {
                    qv = sm.u.tab[0][bin];
                    if (qv != 0.0 && ((rq.has_k && key == rq.ck.key && col > eff[0][0]) ||
                                      (rq.has_p && key == rq.cp.key && col > eff[0][1])))
                        qv = 0.0;
                } else if (kind == kKindSpecial) {
                    if (in_cut_id(rq.has_k ? rq.ck.key : 0u, eff[0][0], key, col) &&
                        in_cut_id(rq.has_p ? rq.cp.key : 0u, eff[0][1], key, col))
                        qv = mass_of(__uint_as_float(h << 16), rq.m, rq.T) / rq.S;
                }
            }
            if (two) {
                const uint32_t w = vp[q][e >> 1];
                const uint32_t h = (e & 1) ? (w >> 16) : (w & 0xFFFFu);
                int bin;
                const int kind = classify(h, &bin);
                const uint32_t key = key16(h);
                bool in = false;
                double p = 0.0;
                if (kind == kKindBin) {
                    p = sm.u.tab[1][bin];
                    in = p != 0.0 && !((rp.has_k && key == rp.ck.key && col > eff[1][0]) ||
                                       (rp.has_p && key == rp.cp.key && col > eff[1][1]));
                    if (in && rp.nset > 0 && key == rp.kF) p = (p * (col <= rp.idF ? rp.C : 1.0)) / rp.Z;
                } else if (kind == kKindSpecial) {
                    in = in_cut_id(rp.has_k ? rp.ck.key : 0u, eff[1][0], key, col) &&
                         in_cut_id(rp.has_p ? rp.cp.key : 0u, eff[1][1], key, col);
                    if (in) {
                        const double e2 = mass_of(__uint_as_float(h << 16), rp.m, rp.T);
                        const double pp = e2 / rp.S;
                        const double fct = (rp.nset > 0 && e2 > 0.0 && in_cut_id(rp.kF, rp.idF, key, col)) ? rp.C : 1.0;
                        p = (pp * fct) / rp.Z;
                    }
                }
                pv = in ? p : 0.0;
                const double d = qv - pv;
                acc += d > 0.0 ? d : 0.0;
            } else {
                acc += qv;
            }
        }
        acc = wave_sum(acc);
        if (lane == 0) out[q * kWaves + wave] = acc;
    }
}

// The general algorithm for one unit (out of line: a rare path).  The arguments come by
// value so that no pointer to the kernel's own arguments escapes (which would move them to
// scratch memory for the whole kernel).
__device__ __noinline__ void fallback_unit(VerifyArgs a, int b, int j, Smem& sm) {
    unit_verify(a, b, j, &sm.urec, sm.u.generic, sm.gst[0], sm.gst[1]);
}

// ------------------------------------------------------------------------------------------
// Finaliser: the last workgroup of a request picks k and t*
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void finalize_request(const FastArgs& f, Smem& sm, int b) {
    const VerifyArgs& a = f.a;
    const int K = a.K;
    const UnitFast* U = reinterpret_cast<const UnitFast*>(f.ws + f.L.units) + (size_t)b * (K + 1);
    const int32_t* IC = reinterpret_cast<const int32_t*>(f.ws + f.L.idcut);
    const int lane = threadIdx.x & (kWave - 1);
    // 1. the verdicts of the request's K + 1 units (one lane each): status and k
    if (threadIdx.x < kWave) {
        uint32_t st = 0;
        int acc = 1;
        if (lane <= K) {
            st = ldnt(&U[lane].status);
            acc = ldnt(&U[lane].accept);
        }
        const uint32_t any = wave_or(st);
        const uint32_t deg = wave_or(lane < K ? (st & kStDegenerate) : 0u);
        int k = first_lane(__ballot(lane < K && !acc));
        if (k < 0) k = K;
        const uint32_t outside = wave_or((lane < K && lane <= k) ? (st & kStOutside) : 0u);
        uint32_t status;
        bool normal = false;
        if (any & kStBadParam) {
            status = kStBadParam;
        } else if (any & kStBadLogit) {
            status = kStBadLogit;
        } else if (any & kStBadToken) {
            status = deg | kStBadToken;
        } else {
            status = deg | outside;
            normal = true;
        }
        if (lane == 0) {
            sm.fk = normal ? k : 0;
            sm.fstatus = status;
            sm.fmode = normal ? -1 : 0;
            sm.ft = -1;
            sm.fW = 0.0;
        }
    }
    __syncthreads();
    const int k = sm.fk;
    int mode = 0;  // 0: done, 1: scan of one chunk, 2: empty residual (scan of the target row)
    if (sm.fmode < 0) {
        const UnitFast* uk = &U[k];
        const int fb = ldnt(&uk->fallback);
        const int greedy = ldnt(&uk->rq.greedy);
        if (fb) {
            if (threadIdx.x == 0) {
                sm.ft = ldnt(&uk->tcand);
                sm.fW = k == K ? 0.0 : (double)ldnt(&uk->W);
                sm.fstatus |= ldnt(&uk->status) & kStEmptyResidual;
            }
        } else if (greedy) {
            if (threadIdx.x == 0) sm.ft = ldnt(&uk->rq.argmax);
        } else {
            // the unit's chunk sums in token order, two per thread
            const double* ch = reinterpret_cast<const double*>(f.ws + f.L.chunks) + (size_t)(b * (K + 1) + k) * f.nS * kChunks;
            const int n = f.nS * kChunks;
            const int c0 = 2 * threadIdx.x;
            const double x0 = c0 < n ? ldnt(&ch[c0]) : 0.0;
            const double x1 = c0 + 1 < n ? ldnt(&ch[c0 + 1]) : 0.0;
            double W;
            const double before = block_exclusive_scan<double>(x0 + x1, sm.redd, &W);
            const double v = uniform_at(a.seed, a.round, (uint64_t)b, (uint64_t)k, 1);
            if (W > 0.0) {
                // the last chunk with mass whose preceding mass is <= v * W
                const double target = v * W;
                int pick = -1;
                if (x0 > 0.0 && before <= target) pick = c0;
                if (x1 > 0.0 && before + x0 <= target) pick = c0 + 1;
                pick = block_max<int>(pick, sm.redi);
                if (pick >= 0 && (pick >> 1) == (int)threadIdx.x) sm.fbase = (pick & 1) ? before + x0 : before;
                if (threadIdx.x == 0) {
                    sm.fc = pick;
                    sm.ftarget = target;
                    sm.fW = k == K ? 0.0 : W;
                }
                mode = 1;
            } else {
                if (threadIdx.x == 0) {
                    sm.fstatus |= kStEmptyResidual;
                    sm.ftarget = v;
                    sm.fW = 0.0;
                }
                mode = 2;
            }
        }
    }
    __syncthreads();
    if (mode != 0) {
        const int unit = b * (K + 1) + k;
        // the row statistics of unit k (published by its slice 0), staged through LDS
        constexpr int kWords = (int)(sizeof(RowFinal) / 4);
        if ((int)threadIdx.x < 2 * kWords)
            sm.fin[threadIdx.x] = ldnt(reinterpret_cast<const uint32_t*>(&U[k].rq) + threadIdx.x);
        __syncthreads();
        RowFinal rq, rp;
        {
            uint32_t* dq = reinterpret_cast<uint32_t*>(&rq);
            uint32_t* dp = reinterpret_cast<uint32_t*>(&rp);
#pragma unroll
            for (int i = 0; i < kWords; ++i) {
                dq[i] = sm.fin[i];
                dp[i] = sm.fin[kWords + i];
            }
        }
        const int idk_q = ldnt(&IC[unit * 4 + 0]), idp_q = ldnt(&IC[unit * 4 + 1]);
        const int idk_p = ldnt(&IC[unit * 4 + 2]), idp_p = ldnt(&IC[unit * 4 + 3]);
        const size_t stride = (size_t)a.V;
        const uint16_t* trow = static_cast<const uint16_t*>(a.target) + ((size_t)b * (K + 1) + k) * stride;
        const uint16_t* drow = k < K ? static_cast<const uint16_t*>(a.draft) + ((size_t)b * a.draft_rows + k) * stride : nullptr;
        // columns to scan: the picked chunk (mode 1) or the whole target row (mode 2)
        int lo, hi;
        double base;
        if (mode == 1) {
            const int c = sm.fc;
            const int slice = c / kChunks, within = c % kChunks;
            lo = slice * kSliceCols + (within / kWaves) * (kThreads * 8) + (within % kWaves) * kChunkCols;
            hi = min(lo + kChunkCols, a.V);
            base = sm.fbase;
        } else {
            lo = 0;
            hi = a.V;
            base = 0.0;
        }
        // mode 2 needs the total of q first
        double total_q = 0.0;
        if (mode == 2) {
            double acc = 0.0;
            for (int col = threadIdx.x; col < a.V; col += blockDim.x)
                acc += final_prob(rq, idk_q, idp_q, trow[col], col, false);
            total_q = block_sum<double>(acc, sm.redd);
        }
        const double tgt = mode == 1 ? sm.ftarget : sm.ftarget * total_q;
        int best = 0x7FFFFFFF, last = -1;
        for (int c0 = lo; c0 < hi; c0 += blockDim.x) {
            const int col = c0 + threadIdx.x;
            double w = 0.0;
            if (col < hi) {
                const double qv = final_prob(rq, idk_q, idp_q, trow[col], col, false);
                if (mode == 1 && drow) {
                    const double pv = final_prob(rp, idk_p, idp_p, drow[col], col, true);
                    w = qv > pv ? qv - pv : 0.0;
                } else {
                    w = qv;
                }
            }
            double tot;
            const double before = block_exclusive_scan<double>(w, sm.redd, &tot);
            const double cum = base + before + w;
            if (w > 0.0 && cum > tgt) best = min(best, col);
            if (w > 0.0) last = max(last, col);
            base += tot;
            const int bmin = block_min<int>(best, sm.redi);
            if (bmin != 0x7FFFFFFF) {
                best = bmin;
                break;
            }
        }
        last = block_max<int>(last, sm.redi);
        if (threadIdx.x == 0) sm.ft = best != 0x7FFFFFFF ? best : last;
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        a.out_k[b] = k;
        a.out_t[b] = sm.ft;
        if (a.out_W) a.out_W[b] = (float)sm.fW;
        if (a.out_status) a.out_status[b] = sm.fstatus;
        // leave the request's counter zeroed for the next call
        *reinterpret_cast<unsigned*>(f.ws + f.L.req + (size_t)b * 128) = 0u;
    }
}

// ------------------------------------------------------------------------------------------
// Resolve kernel: every slice combines its unit's summaries into the exact processed
// distributions (redundantly), tests acceptance and, where the unit needs it, re-reads its
// columns to sum the residual over 512-column chunks; the last workgroup of a request to
// finish picks k and t*.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void fast_resolve_kernel(FastArgs f) {
    __shared__ Smem sm;
    const VerifyArgs& a = f.a;
    const Place P = place_of(f);
    if (P.b >= a.B) return;
    const int b = P.b, j = P.j, slice = P.slice, unit = P.unit;
    const int c0 = slice * kSliceCols;
    const bool two = j < a.K;
    const spec_params prm = a.params[b];
    const bool param_ok = params_ok(prm);
    const size_t stride = (size_t)a.V;
    const uint16_t* trow = static_cast<const uint16_t*>(a.target) + ((size_t)b * (a.K + 1) + j) * stride;
    const uint16_t* drow = two ? static_cast<const uint16_t*>(a.draft) + ((size_t)b * a.draft_rows + j) * stride : nullptr;
    const int s_tok = two ? a.tokens[(size_t)b * a.K + j] : -1;
    const bool tok_ok = !two || (s_tok >= 0 && s_tok < a.V);
    UnitFast* U = reinterpret_cast<UnitFast*>(f.ws + f.L.units) + unit;
    int32_t* IC = reinterpret_cast<int32_t*>(f.ws + f.L.idcut) + unit * 4;

    uint32_t status = 0;
    int accept = 0;
    bool need_resid = false;
    bool fb_unit = false;
    if (!param_ok) {
        status = kStBadParam;
    } else {
        combine(f, sm, unit, two ? 2 : 1, prm);
        const bool bad = sm.rv[0].bad || (two && sm.rv[1].bad);
        fb_unit = !bad && (sm.rv[0].overflow || (two && sm.rv[1].overflow));
        if (bad) {
            status = kStBadLogit;
        } else if (fb_unit) {
            // rare shapes the counts cannot settle: the general algorithm, by slice 0 alone (below)
        } else {
            if (two && sm.rv[1].degenerate) status |= kStDegenerate;
            if (!tok_ok) {
                status |= kStBadToken;
            } else if (two) {
                if (sm.rv[0].greedy) {
                    accept = (s_tok == sm.rv[0].argmax) ? 1 : 0;
                } else {
                    const double ps = prob_of_s(sm, 1, s_tok, true);
                    const double qs = prob_of_s(sm, 0, s_tok, false);
                    if (!(ps > 0.0)) status |= kStOutside;
                    const double u = uniform_at(a.seed, a.round, (uint64_t)b, (uint64_t)j, 0);
                    accept = (u * ps < qs) ? 1 : 0;
                }
            } else {
                accept = 1;  // bonus position
            }
            need_resid = tok_ok && (!accept || !two) && !sm.rv[0].greedy;
            if (slice == 0 && threadIdx.x == 0) {
                for (int r = 0; r < 2; ++r) {
                    const RowView& rv = sm.rv[r];
                    RowFinal rf;
                    rf.m = rv.m;
                    rf.T = (float)rv.T;
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
                    // explicit and trivial id cuts (histogram cuts are written by their owner)
                    if (!rv.has_k || rv.ck.key == 0) IC[r * 2 + 0] = a.V - 1;
                    else if (rv.ck.explicit_id >= 0) IC[r * 2 + 0] = rv.ck.explicit_id;
                    if (!rv.has_p || rv.cp.key == 0) IC[r * 2 + 1] = a.V - 1;
                    else if (rv.cp.explicit_id >= 0) IC[r * 2 + 1] = rv.cp.explicit_id;
                }
                U->fallback = 0;
                U->tcand = -1;
                U->W = 0.0f;
            }
        }
    }
    if (slice == 0 && threadIdx.x == 0 && !fb_unit) {
        U->accept = accept;
        U->status = status;
    }
    if (need_resid) {
        u32x4 vq[kLoads], vp[kLoads];
        load_slice(trow, c0, a.V, vq);
        if (two) load_slice(drow, c0, a.V, vp);
        int eff[2][2];
        for (int r = 0; r < (two ? 2 : 1); ++r) {
            const RowView& rv = sm.rv[r];
            const u32x4(&v)[kLoads] = r == 0 ? vq : vp;
            eff[r][0] = rv.has_k ? effective_id(sm, rv.ck, slice, v, c0, a.V) : a.V - 1;
            eff[r][1] = rv.has_p ? effective_id(sm, rv.cp, slice, v, c0, a.V) : a.V - 1;
            if (threadIdx.x == 0) {
                if (rv.has_k && rv.ck.key != 0 && rv.ck.explicit_id < 0 && slice == rv.ck.owner) IC[r * 2 + 0] = eff[r][0];
                if (rv.has_p && rv.cp.key != 0 && rv.cp.explicit_id < 0 && slice == rv.cp.owner) IC[r * 2 + 1] = eff[r][1];
            }
        }
        if (!two) {
            eff[1][0] = eff[1][1] = a.V - 1;
        }
        __syncthreads();
        residual_chunks(f, sm, unit, slice, c0, two, vq, vp, eff);
    }

    if (fb_unit && slice == 0) {
        fallback_unit(a, b, j, sm);
        if (threadIdx.x == 0) {
            U->accept = sm.urec.accept;
            U->status = sm.urec.status;
            U->fallback = 1;
            U->tcand = sm.urec.tcand;
            U->W = sm.urec.W;
        }
    }

    // ---- request rendezvous: the last workgroup of the request finalises it ----
    drain_stores();
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned* rc = reinterpret_cast<unsigned*>(f.ws + f.L.req + (size_t)b * 128);
        const unsigned old = l2_fetch_add(rc, 1u);
        sm.last = (old + 1 == (unsigned)P.per_req) ? 1 : 0;
    }
    __syncthreads();
    if (sm.last) finalize_request(f, sm, b);
}

void launch_resolve(const FastArgs& f, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(fast_resolve_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, f);
}

}  // namespace fast
}  // namespace sv
