// Resolve kernel of the bf16 verification path.  The count kernel has decided every request:
// its first rejected position k (or K) and whether a residual is still to be drawn.  Here
// the slices of unit k sum the residual (q_k - p'_k)+ (or the target q_K at the bonus
// position) over 512-column chunks, and the last of them draws t* by inverse CDF in token
// order (DeepMind speculative-sampling page, sections 1 and 3; SSD reading notes, section
// 2.2).  Requests whose units the counts could not settle run the general algorithm.
#include "fast_common.h"

#include <atomic>
#include "rowproc.h"

namespace sv {
namespace fast {

// A bin at which this slice decides elements one by one: its table entry holds the value of
// the elements up to column thr; later elements of the bin take alt (0 past a cut, the value
// outside the downweighted set past its boundary).
struct TieRole {
    uint32_t off;  // byte offset of the bin's table entry (kNoTie: none)
    int thr;
    double alt;
};
constexpr uint32_t kNoTie = 0xFFFFFFFFu;


struct ResSmem {
    union {
        double tab[2][kHistRow];   // per-bin values of q and p' in the padded histogram layout
        RowShared generic;
        struct {
            RowShared rs;
            CacheShared cs;
        } cache;
    } u;
    RowStats gst[2];
    UnitRec urec;
    RowFinal rf[2];
    double inv[2][2];              // [row][1 / S, 1 / Z]
    TieRole tie[2][3];             // [row][set boundary, top-k tie, top-p tie] this slice decides
    UnitCut cut[2][2];
    uint32_t flags[2];             // this slice's RowPart flags of each row
    int eff[2][2];                 // this slice's id cut at each cut key (V-1 all, -1 none)
    uint64_t nth_scan[kWaves][4];  // per-wave match counts of the owned cut keys
    int32_t scan[kWaves + 1];
    double redd[kWaves];
    int32_t redi[kWaves];
    int last;
    int misplaced;  // the request's workgroups arrived from more than one XCD
    int fc;
    int fscan[kWaves];
    double ftarget, fbase, fW;
    double u_res;                  // the draw for t*
};

// This slice's id cut at every cut key of both rows (row r, cut c): V - 1 (keeps all), -1
// (keeps none), the explicit id, or, at a histogram cut this slice owns, the column of the
// owner_take-th element at the cut key in token order.  The owned cuts share one pass: packed
// bf16 comparisons count each thread's matches per 16-byte load, one workgroup scan of four
// 64-bit words (one per cut, four 16-bit load counts each) orders them, and the threads
// holding the wanted elements report their columns.
__device__ __forceinline__ void slice_id_cuts(ResSmem& sm, const u32x4 (&vq)[kLoads], const u32x4 (&vp)[kLoads], int c0, int V,
                                              int slice, bool two) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    bool own[4];
    int res[4];
    uint32_t masks[4];
    uint64_t packed[4];
    bool any = false;
    // elements per load that lie inside the row (the tail slice is zero-filled past V)
    uint32_t valid[kLoads];
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
        const int left = V - col_of(c0, q, 0);
        valid[q] = left >= 8 ? 0xFFu : (left <= 0 ? 0u : ((1u << left) - 1u));
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int r = x >> 1;
        const UnitCut uc = sm.cut[r][x & 1];
        own[x] = false;
        res[x] = V - 1;
        masks[x] = 0u;
        packed[x] = 0u;
        if (uc.key == 0u || (r == 1 && !two)) continue;
        if (uc.explicit_id >= 0) res[x] = uc.explicit_id;
        else if (slice > uc.owner) res[x] = -1;
        else if (slice == uc.owner) own[x] = true;
        if (!own[x]) continue;
        any = true;
        // the key's bf16 pattern; zero's key stands for both signed zeros
        const uint32_t k = uc.key;
        const uint32_t hk = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
        const uint32_t keep = hk == 0u ? 0x7FFF7FFFu : 0xFFFFFFFFu;
        const uint32_t pat = hk * 0x10001u;
        const u32x4(&v)[kLoads] = r == 0 ? vq : vp;
#pragma unroll
        for (int q = 0; q < kLoads; ++q) {
            uint32_t mq = 0;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t y = (v[q][d] & keep) ^ pat;
                mq |= ((y & 0xFFFFu) == 0u ? 1u : 0u) << (2 * d);
                mq |= ((y >> 16) == 0u ? 1u : 0u) << (2 * d + 1);
            }
            mq &= valid[q];
            masks[x] |= mq << (8 * q);
            packed[x] |= (uint64_t)__popc(mq) << (16 * q);
        }
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
        if ((int)threadIdx.x == x) sm.eff[x >> 1][x & 1] = own[x] ? -1 : res[x];  // -1: fewer matches than wanted
    if (any) {
        uint64_t before[4], total[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            uint64_t exc;
            const uint64_t inc = wave_scan(packed[x], &exc);
            before[x] = exc;
            if (lane == kWave - 1) sm.nth_scan[wave][x] = inc;
        }
        __syncthreads();
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            total[x] = 0u;
            for (int w = 0; w < kWaves; ++w) {
                const uint64_t t = sm.nth_scan[w][x];
                if (w < wave) before[x] += t;
                total[x] += t;
            }
        }
        // token order is (load q, thread, element): the loads before q contribute their totals
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            if (!own[x]) continue;
            const int n = sm.cut[x >> 1][x & 1].owner_take;
            int base = 0;
#pragma unroll
            for (int q = 0; q < kLoads; ++q) {
                const uint32_t mq = (masks[x] >> (8 * q)) & 0xFFu;
                const int bq = base + (int)((before[x] >> (16 * q)) & 0xFFFFu);
                if (bq < n && bq + __popc(mq) >= n) {
                    // the (n - bq)-th set bit of mq
                    uint32_t m = mq;
                    for (int skip = n - bq - 1; skip > 0; --skip) m &= m - 1u;
                    sm.eff[x >> 1][x & 1] = col_of(c0, q, __builtin_ctz(m));
                }
                base += (int)((total[x] >> (16 * q)) & 0xFFFFu);
            }
        }
    }
}

// Processed probability of one element from the row's final statistics, id cuts and its mass
// e: q = e / S, p' = ((e / S) * f) / Z, the divisions taken as products with 1 / S and 1 / Z.
__device__ __forceinline__ double prob_from_mass(const RowFinal& rf, const double (&inv)[2], int idk, int idp, uint32_t key,
                                                 int col, double e, bool draft) {
    if (!in_cut_id(rf.kk, idk, key, col) || !in_cut_id(rf.kp, idp, key, col)) return 0.0;
    const double p = e * inv[0];
    if (!draft) return p;
    const double fct = (rf.nS > 0 && e > 0.0 && in_cut_id(rf.kF, rf.idF, key, col)) ? rf.C : 1.0;
    return (p * fct) * inv[1];
}

__device__ __forceinline__ double final_prob(const RowFinal& rf, const double (&inv)[2], int idk, int idp, uint32_t h, int col,
                                             bool draft) {
    const uint32_t mag = h & 0x7FFFu;
    if (mag >= 0x7F80u) return 0.0;  // -inf (rows with NaN or +inf never get here)
    if (rf.greedy) return col == rf.argmax ? 1.0 : 0.0;
    return prob_from_mass(rf, inv, idk, idp, key16(h), col, mass_of(__uint_as_float(h << 16), rf.m, rf.invT), draft);
}

// Whether this slice's elements at a cut key are kept: all (before the owner), none (after),
// or decided per element (the owner itself).
__device__ __forceinline__ bool slice_keeps(const UnitCut& c, int slice) { return slice <= c.owner; }

// Table entries that stand for "decide this element exactly": large enough that any 512-
// column partial sum containing one exceeds kMarkSeen, which no true sum of probabilities can.
constexpr double kMarkQ = 1e300;    // in the target table: (q - p)+ and q become huge
constexpr double kMarkP = -1e300;   // in the draft table: (q - p)+ becomes huge
constexpr double kMarkSeen = 1e299;

// What the table entries of one row depend on, read once into registers (the entries are
// written to LDS, so values left in LDS would be re-read after every entry).
struct RowTab {
    uint32_t klow, kmax;      // below the cuts / above the maximum
    uint32_t kk, kp;          // cut keys (0: none)
    bool keep_k, keep_p;      // this slice keeps its elements at the cut keys
    uint32_t own_k, own_p;    // cut keys this slice decides one by one (kNoTie: none)
    uint32_t own_F;           // the set boundary key when this slice decides it (kNoTie: none)
    uint32_t kF;
    bool set_on, keep_F;      // the downweighted set exists / this slice's boundary ties are in it
    int idF;
    double inv_S, inv_Z, C;
};

__device__ __forceinline__ RowTab row_tab(const ResSmem& sm, int r, int slice, int ownerF) {
    const RowFinal& rf = sm.rf[r];
    const UnitCut& ck = sm.cut[r][0];
    const UnitCut& cp = sm.cut[r][1];
    RowTab t;
    t.klow = max(ck.key, cp.key);
    t.kmax = key16(__float_as_uint(rf.m) >> 16);
    t.kk = ck.key;
    t.kp = cp.key;
    t.keep_k = slice_keeps(ck, slice);
    t.keep_p = slice_keeps(cp, slice);
    t.own_k = (ck.key != 0u && ck.owner == slice) ? ck.key : kNoTie;
    t.own_p = (cp.key != 0u && cp.owner == slice) ? cp.key : kNoTie;
    t.own_F = (r == 1 && ownerF == slice) ? rf.kF : kNoTie;
    t.kF = rf.kF;
    t.set_on = r == 1 && rf.nS > 0;
    t.keep_F = slice <= ownerF;
    t.idF = rf.idF;
    t.inv_S = sm.inv[r][0];
    t.inv_Z = sm.inv[r][1];
    t.C = rf.C;
    return t;
}

// The table entry of one bin of row r as this slice sees it: q = e / S, p' = ((e / S) * f) / Z
// (as final_prob), with every cut key resolved as this slice sees it.  Where this slice decides
// elements of the bin one by one (it holds the last kept element at a cut key, or the draft
// row's downweighted-set boundary) the entry holds the value of the earliest elements and a tie
// role records where and how the later ones differ.
__device__ __forceinline__ void bin_entry(ResSmem& sm, int r, const RowTab& t, int bin, double e) {
    const uint32_t key = bin_key(bin);
    // zero never reaches its group's bins (the packed offsets send it to the padding words)
    const bool real = bin / kGroup != kZeroGroup;
    double v = 0.0;
    if (key >= t.klow && key <= t.kmax && (key > t.kk || t.keep_k) && (key > t.kp || t.keep_p)) {
        const double pv = e * t.inv_S;
        v = pv;
        if (r == 1) {
            const bool in_set = t.set_on && e > 0.0 && (key > t.kF || (key == t.kF && t.keep_F));
            v = (pv * (in_set ? t.C : 1.0)) * t.inv_Z;
        }
        if (real && (key == t.own_F || key == t.own_k || key == t.own_p)) {
            const uint32_t off = 8u * (uint32_t)(kHistLead + bin);
            if (key == t.own_F) sm.tie[r][0] = TieRole{off, t.idF, pv * t.inv_Z};
            if (key == t.own_k) sm.tie[r][1] = TieRole{off, 0, 0.0};
            if (key == t.own_p) sm.tie[r][2] = TieRole{off, 0, 0.0};
        }
    }
    sm.u.tab[r][kHistLead + bin] = v;
}

// The residual's tables from the slice's own occupied bins: the (bin, count) entries the count
// kernel published for it (ent0, ent1: entries t % 256 and t % 256 + 256 of row t / 256, loaded
// with the slice's columns; n_ent: that row's entry count).  Every element of the slice falls in
// one of them (or is a value outside the bins, which the padding words' markers send to the exact
// formula), so no other entry is read: one exp per occupied bin instead of one per bin of every
// group the slice holds between the cuts and the maximum.
constexpr int kHalf = kThreads / 2;  // a row's share of the workgroup

struct SliceEnt {     // this thread's share of the slice's entries (see sparse_tables)
    const RowPart* pr;  // the record of row threadIdx.x / kHalf
    uint32_t n, e0, e1; // that row's entry count; entries threadIdx.x % kHalf and that + kHalf
};
__device__ __forceinline__ SliceEnt load_slice_ent(const FastArgs& f, int unit, int slice) {
    SliceEnt e;
    e.pr = part_of(f, unit, slice, (int)threadIdx.x / kHalf);
    e.n = ldnt(&e.pr->n_ent);
    e.e0 = ldnt(&e.pr->ent[threadIdx.x % kHalf]);
    e.e1 = ldnt(&e.pr->ent[threadIdx.x % kHalf + kHalf]);
    return e;
}
__device__ __forceinline__ void sparse_tables(ResSmem& sm, bool two, int slice, const RowPart* pr, uint32_t n_ent,
                                              uint32_t ent0, uint32_t ent1) {
    const int r = (int)threadIdx.x / kHalf, i = (int)threadIdx.x % kHalf;
    const int ownerF = (two && sm.rf[1].nS > 0) ? sm.rf[1].idF / kSliceCols : -1;
    if (r == 0 || two) {
        const RowTab t = row_tab(sm, r, slice, ownerF);
        const float m = sm.rf[r].m;
        const double invT = sm.rf[0].invT;
        const int n = (int)min(n_ent, (uint32_t)kBins);
        if (i < n) bin_entry(sm, r, t, (int)(ent0 >> 16), mass_of(key16_value(bin_key((int)(ent0 >> 16))), m, invT));
        if (i + kHalf < n)
            bin_entry(sm, r, t, (int)(ent1 >> 16), mass_of(key16_value(bin_key((int)(ent1 >> 16))), m, invT));
        for (int x = i + 2 * kHalf; x < n; x += kHalf) {  // (rare: over 512 occupied bins)
            const int bin = (int)(ldnt(&pr->ent[x]) >> 16);
            bin_entry(sm, r, t, bin, mass_of(key16_value(bin_key(bin)), m, invT));
        }
    }
    // padding words: values outside the exact bins
    if ((int)threadIdx.x < (two ? 4 : 2)) {
        const int rr = threadIdx.x >> 1;
        const double v = (sm.flags[rr] & 4u) ? (rr == 0 ? kMarkQ : kMarkP) : 0.0;
        sm.u.tab[rr][(threadIdx.x & 1) ? kHistLead + kBins : kHistLead - 1] = v;
    }
}

// The tie roles of a row as the workgroup reads them: uniform values.
struct Ties {
    uint32_t off[3];
    int thr[3];
    double alt[3];
    int any;
};
__device__ __forceinline__ Ties load_ties(const ResSmem& sm, int r) {
    Ties t;
    t.any = 0;
#pragma unroll
    for (int x = 0; x < 3; ++x) {
        t.off[x] = __builtin_amdgcn_readfirstlane(sm.tie[r][x].off);
        // the boundary's threshold is its id; a cut's is this slice's id cut at the cut key
        t.thr[x] = __builtin_amdgcn_readfirstlane(x == 0 ? sm.tie[r][x].thr : sm.eff[r][x - 1]);
        const double alt = sm.tie[r][x].alt;
        t.alt[x] = __hiloint2double(__builtin_amdgcn_readfirstlane(__double2hiint(alt)),
                                    __builtin_amdgcn_readfirstlane(__double2loint(alt)));
        t.any |= t.off[x] != kNoTie;
    }
    return t;
}
// Applies the roles (boundary first, then the cuts) to the values v0, v1 of the two elements
// at table offsets o (low, high half) and columns col, col + 1.
__device__ __forceinline__ void apply_ties(const Ties& t, uint32_t o, int col, double& v0, double& v1) {
#pragma unroll
    for (int x = 0; x < 3; ++x) {
        if (t.off[x] == kNoTie || col + 1 <= t.thr[x]) continue;
        if ((o & 0xFFFFu) == t.off[x] && col > t.thr[x]) v0 = t.alt[x];
        if ((o >> 16) == t.off[x]) v1 = t.alt[x];
    }
}
__device__ __forceinline__ double apply_ties1(const Ties& t, uint32_t o16, int col, double v) {
#pragma unroll
    for (int x = 0; x < 3; ++x)
        if (o16 == t.off[x] && col > t.thr[x]) v = t.alt[x];
    return v;
}

// Byte offsets of the two fp64 table entries of the bf16 values packed in w.
__device__ __forceinline__ uint32_t tab_offsets2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, hist_offsets2(w)) << (u16x2)(uint16_t)1);
}
__device__ __forceinline__ double tab_at(const char* base, uint32_t off) {
    return *reinterpret_cast<const double*>(base + off);
}

// Residual of unit k over this workgroup's half of the slice (its half of the loads), per
// 512-column chunk: table lookups for every element; a thread's 8 columns of one chunk that
// met a marker are recomputed exactly.
__device__ __forceinline__ void residual_slice(const FastArgs& f, ResSmem& sm, int b, int slice, int half, int halves, int c0, bool two,
                                               bool uni, const u32x4 (&vq)[kLoads], const u32x4 (&vp)[kLoads]) {
    const double pu = 1.0 / (double)f.a.V;  // the uniform draft's probability
    const VerifyArgs& a = f.a;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const char* tq = reinterpret_cast<const char*>(&sm.u.tab[0][0]);
    const char* tp = reinterpret_cast<const char*>(&sm.u.tab[1][0]);
    double* out = reinterpret_cast<double*>(f.ws + f.L.chunks) + ((size_t)b * f.nS + slice) * kChunks;
    const Ties tiq = load_ties(sm, 0);
    const Ties tip = load_ties(sm, 1);
    static_assert(kLoads % 2 == 0, "halves of a slice");
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
        if (halves == 2 && q / (kLoads / 2) != half) continue;
        double s = 0.0;
        const int cq = col_of(c0, q, 0);
        if (cq < a.V) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t oq = tab_offsets2(vq[q][d]);
                double q0 = tab_at(tq, oq & 0xFFFFu), q1 = tab_at(tq, oq >> 16);
                if (tiq.any) apply_ties(tiq, oq, cq + 2 * d, q0, q1);
                if (two) {
                    const uint32_t op = tab_offsets2(vp[q][d]);
                    double p0 = tab_at(tp, op & 0xFFFFu), p1 = tab_at(tp, op >> 16);
                    if (tip.any) apply_ties(tip, op, cq + 2 * d, p0, p1);
                    s += max(q0 - p0, 0.0);
                    s += max(q1 - p1, 0.0);
                } else if (uni) {
                    s += max(q0 - pu, 0.0);
                    s += max(q1 - pu, 0.0);
                } else {
                    s += q0;
                    s += q1;
                }
            }
            if (s > kMarkSeen) {  // rare: values outside the exact bins, decided exactly
                s = 0.0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int col = cq + e;
                    const uint32_t wq = vq[q][e >> 1];
                    const uint32_t hq = (e & 1) ? (wq >> 16) : (wq & 0xFFFFu);
                    const uint32_t oq = tab_offsets2(hq) & 0xFFFFu;
                    double qe = tab_at(tq, oq);
                    qe = qe > kMarkSeen ? final_prob(sm.rf[0], sm.inv[0], sm.eff[0][0], sm.eff[0][1], hq, col, false)
                                        : apply_ties1(tiq, oq, col, qe);
                    if (two) {
                        const uint32_t wp = vp[q][e >> 1];
                        const uint32_t hp = (e & 1) ? (wp >> 16) : (wp & 0xFFFFu);
                        const uint32_t op = tab_offsets2(hp) & 0xFFFFu;
                        double pe = tab_at(tp, op);
                        pe = pe < -kMarkSeen ? final_prob(sm.rf[1], sm.inv[1], sm.eff[1][0], sm.eff[1][1], hp, col, true)
                                             : apply_ties1(tip, op, col, pe);
                        s += max(qe - pe, 0.0);
                    } else if (uni) {
                        s += max(qe - pu, 0.0);
                    } else {
                        s += qe;
                    }
                }
            }
        }
        const double sq = wave_sum(s);
        if (lane == 0) out[q * kWaves + wave] = sq;
    }
}

// One block of up to blockDim.x consecutive columns of the inverse-CDF scan, each thread one
// column with weight w: the first column whose cumulative weight (base + preceding weights +
// its own) exceeds tgt, the last column with weight, and the block's total (two barriers: wave
// scans, then the waves' totals).
__device__ __forceinline__ void scan_block(ResSmem& sm, double w, int col, double base, double tgt, int* first, int* last,
                                           double* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    double excl;
    const double incl = wave_scan(w, &excl);
    if (lane == kWave - 1) sm.redd[wave] = incl;
    __syncthreads();
    double before = base, all = 0.0;
    for (int v = 0; v < kWaves; ++v) {
        const double t = sm.redd[v];
        if (v < wave) before += t;
        all += t;
    }
    const uint64_t hit = __ballot(w > 0.0 && before + incl > tgt);
    const uint64_t pos = __ballot(w > 0.0);
    if (lane == 0) {
        sm.scan[wave] = hit ? col - lane + first_lane(hit) : 0x7FFFFFFF;
        sm.fscan[wave] = pos ? col - lane + last_lane(pos) : -1;
    }
    __syncthreads();
    int f = 0x7FFFFFFF, l = -1;
    for (int v = 0; v < kWaves; ++v) {
        f = min(f, sm.scan[v]);
        l = max(l, sm.fscan[v]);
    }
    *first = f;
    *last = l;
    *total = all;
    __syncthreads();  // sm.redd / sm.scan / sm.fscan are reused by the next block
}

// The outcome-cache lookup of request b's verified outcome (k, t*), fused into this kernel
// (saguaro_cache_lookup mode 0; SSD reading notes, section 7.1): the slot of t* in the cache's
// depth-k list, or a miss, added into the batch's hit count and all-hit flag.  One thread.
// The first eight entries of request b's depth-k cache list (-1 past the list), loaded ahead.
struct LookupHead {
    int32_t v[8];
};
__device__ __forceinline__ LookupHead lookup_head(const FastArgs& f, int b, int k) {
    LookupHead h;
    const bool ok = k >= 0 && k <= f.a.K;
    const int32_t* c = f.out_cache + (size_t)b * f.budget + (ok ? f.fan.off[k] : 0);
    const int n = ok ? f.fan.f[k] : 0;
#pragma unroll
    for (int d = 0; d < 8; ++d) h.v[d] = d < n ? ldnt(c + d) : -1;
    return h;
}
__device__ __forceinline__ void lookup_request(const FastArgs& f, int b, int k, int t, const LookupHead& head) {
    const VerifyArgs& a = f.a;
    int res = -1;
    if (k >= 0 && k <= a.K && t >= 0) {
        // the depth-k list in batches of eight independent loads, the first batch loaded ahead
        // (rows written by this kernel's workgroups of the request reach L2 before their arrival)
        const int32_t* c = f.out_cache + (size_t)b * f.budget + f.fan.off[k];
        const int n = f.fan.f[k];
#pragma unroll
        for (int d = 7; d >= 0; --d)
            if (head.v[d] == t) res = f.fan.off[k] + d;
        for (int f0 = 8; f0 < n && res < 0; f0 += 8) {
            int32_t v[8];
#pragma unroll
            for (int d = 0; d < 8; ++d) v[d] = f0 + d < n ? ldnt(c + f0 + d) : -1;
#pragma unroll
            for (int d = 7; d >= 0; --d)
                if (v[d] == t) res = f.fan.off[k] + f0 + d;
        }
    }
    f.out_slot[b] = res;
    f.out_hit[b] = res >= 0 ? 1 : 0;
    // the batch's hit count and all-hit flag, which the count kernel set to {0, 1}: added into at
    // system scope (the requests' workgroups run on every XCD), results unused (no round trip)
    if (f.out_batch) {
        (void)__hip_atomic_fetch_add(&f.out_batch[0], res >= 0 ? 1 : 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        if (res < 0) (void)__hip_atomic_fetch_and(&f.out_batch[1], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

// The last workgroup of the request draws t* by inverse CDF over the residual (or q_K), in
// token order: one wave picks the 512-column chunk from the chunk sums (each lane sums up to 8
// consecutive chunks), then the workgroup scans that chunk's exact values.  u is the draw.
__device__ __forceinline__ void finalize_residual(const FastArgs& f, ResSmem& sm, int b, int k, uint32_t status, double v) {
    const VerifyArgs& a = f.a;
    // the fused lookup's first cache entries, loaded while t* is drawn
    LookupHead head{};
    if (f.lookup && threadIdx.x == 0) head = lookup_head(f, b, k);
    const int K = a.K;
    const int n = f.nS * kChunks;
    const double* ch = reinterpret_cast<const double*>(f.ws + f.L.chunks) + (size_t)b * f.nS * kChunks;
    const int32_t* IC = reinterpret_cast<const int32_t*>(f.ws + f.L.idcut) + b * 4;
    const int lane = threadIdx.x & (kWave - 1);
    const int idk_q = ldnt(&IC[0]), idp_q = ldnt(&IC[1]), idk_p = ldnt(&IC[2]), idp_p = ldnt(&IC[3]);
    if (threadIdx.x < kWave) {
        static_assert(kMaxSlices * kChunks <= 8 * kWave, "eight chunks per lane");
        double x[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int i = lane * 8 + c;
            x[c] = i < n ? ldnt(&ch[i]) : 0.0;
        }
        double mine = 0.0;
#pragma unroll
        for (int c = 0; c < 8; ++c) mine += x[c];
        double before;
        const double incl = wave_scan(mine, &before);
        const double W = wave_bcast(incl, kWave - 1);
        const double target = v * W;
        // the last chunk with mass whose preceding mass is <= target
        int pick = -1;
        double pbase = 0.0, run = before;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            if (x[c] > 0.0 && run <= target) {
                pick = lane * 8 + c;
                pbase = run;
            }
            run += x[c];
        }
        const int best = max(wave_max(pick), 0);  // (W > 0 always picks a chunk; a guard for NaN sums)
        if (pick == best && best >= 0) sm.fbase = pbase;
        if (lane == 0) {
            sm.fc = best;
            sm.ftarget = W > 0.0 ? target : v;
            sm.fW = W;
        }
    }
    __syncthreads();
    const double W = sm.fW;
    const int mode = W > 0.0 ? 1 : 2;
    if (mode == 2) status |= kStEmptyResidual;
    const RowFinal& rq = sm.rf[0];
    const RowFinal& rp = sm.rf[1];
    const size_t stride = (size_t)a.V;
    const uint16_t* trow = static_cast<const uint16_t*>(a.target) + ((size_t)b * (K + 1) + k) * stride;
    const bool uni = k < K && f.uniform;
    const uint16_t* drow =
        (k < K && !f.uniform) ? static_cast<const uint16_t*>(a.draft) + ((size_t)b * a.draft_rows + k) * stride : nullptr;
    const double pu = 1.0 / (double)a.V;
    // columns to scan: the picked chunk (mode 1) or the whole target row (mode 2)
    int lo, hi;
    double base;
    if (mode == 1) {
        lo = (sm.fc / kChunks) * kSliceCols + (sm.fc % kChunks) * kChunkCols;
        hi = min(lo + kChunkCols, a.V);
        base = sm.fbase;
    } else {
        lo = 0;
        hi = a.V;
        base = 0.0;
    }
    double total_q = 0.0;
    if (mode == 2) {
        double acc = 0.0;
        for (int col = threadIdx.x; col < a.V; col += blockDim.x) acc += final_prob(rq, sm.inv[0], idk_q, idp_q, trow[col], col, false);
        total_q = block_sum<double>(acc, sm.redd);
    }
    const double tgt = mode == 1 ? sm.ftarget : sm.ftarget * total_q;
    int best = 0x7FFFFFFF, last = -1;
    for (int c0 = lo; c0 < hi; c0 += blockDim.x) {
        const int col = c0 + threadIdx.x;
        double w = 0.0;
        if (col < hi) {
            const double qv = final_prob(rq, sm.inv[0], idk_q, idp_q, trow[col], col, false);
            if (mode == 1 && drow) {
                const double pv = final_prob(rp, sm.inv[1], idk_p, idp_p, drow[col], col, true);
                w = qv > pv ? qv - pv : 0.0;
            } else if (mode == 1 && uni) {
                w = qv > pu ? qv - pu : 0.0;
            } else {
                w = qv;
            }
        }
        int fb, lb;
        double tot;
        scan_block(sm, w, col, base, tgt, &fb, &lb, &tot);
        last = max(last, lb);
        base += tot;
        if (fb != 0x7FFFFFFF) {
            best = fb;
            break;
        }
    }
    if (threadIdx.x == 0) {
        const int t = best != 0x7FFFFFFF ? best : last;
        a.out_k[b] = k;
        a.out_t[b] = t;
        if (a.out_W) a.out_W[b] = k == K ? 0.0f : (float)W;
        if (a.out_status) a.out_status[b] = status | (sm.misplaced ? kStPlacement : 0u);
        if (f.lookup) lookup_request(f, b, k, t, head);
    }
}

// The general algorithm for one unit (out of line: a rare path).  The arguments come by
// value so that no pointer to the kernel's own arguments escapes (which would move them to
// scratch memory for the whole kernel).
__device__ __forceinline__ void fallback_unit(const VerifyArgs& a, int b, int j, ResSmem& sm) {
    unit_verify<1>(a, b, j, &sm.urec, sm.u.generic, sm.gst[0], sm.gst[1]);  // (no loads ahead: registers)
}

// Request arrival in the XCD's L2; true for the last of `expected` workgroups (which resets
// the counter for the next call).  The 64-bit counter holds the arrivals (bits 0-7) and, in
// seven bits per XCD from bit 8, the arrivals from each XCD: when the last arriver's own XCD
// did not see every arrival, the request's workgroups did not share one L2 and sm.misplaced
// is set (the outputs then carry kStPlacement).
__device__ __forceinline__ bool arrive_last(const FastArgs& f, ResSmem& sm, int b, int expected) {
    drain_stores();
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t* rc = reinterpret_cast<uint64_t*>(f.ws + f.L.res_ctr + (size_t)b * 128);
        const uint32_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0x7u;  // XCC_ID
        const uint64_t add = 1ull + (1ull << (8 + 7 * xcc));
        const uint64_t now = l2_fetch_add64(rc, add) + add;
        sm.last = ((now & 0xFFull) == (uint64_t)expected) ? 1 : 0;
        sm.misplaced = ((now >> (8 + 7 * xcc)) & 0x7Full) != (uint64_t)expected ? 1 : 0;
        if (sm.last) *rc = 0ull;
    }
    __syncthreads();
    return sm.last != 0;
}

// The general algorithm for every unit of request b, and the request's outcome from them.
__device__ __forceinline__ void general_request(const FastArgs& f, ResSmem& sm, int b, int j, uint32_t extra) {
    const VerifyArgs& a = f.a;
    UnitRec* G = reinterpret_cast<UnitRec*>(f.ws + f.L.gen) + (size_t)b * (a.K + 1);
    fallback_unit(a, b, j, sm);
    if (threadIdx.x == 0) G[j] = sm.urec;
    if (!arrive_last(f, sm, b, a.K + 1)) return;
    if (threadIdx.x != 0) return;
    uint32_t any = 0, deg = 0;
    for (int x = 0; x <= a.K; ++x) {
        const uint32_t st = ldnt(&G[x].status);
        any |= st;
        if (x < a.K) deg |= st & kStDegenerate;
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
        for (int x = 0; x < a.K; ++x) {
            st |= ldnt(&G[x].status) & kStOutside;
            if (!ldnt(&G[x].accept)) {
                k = x;
                break;
            }
        }
        t = ldnt(&G[k].tcand);
        W = ldnt(&G[k].W);
        st |= ldnt(&G[k].status) & kStEmptyResidual;
    }
    a.out_k[b] = k;
    a.out_t[b] = t;
    if (a.out_W) a.out_W[b] = W;
    if (a.out_status) a.out_status[b] = st | extra | (sm.misplaced ? kStPlacement : 0u);
    if (f.lookup) lookup_request(f, b, k, t, lookup_head(f, b, k));
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void fast_resolve_kernel(FastArgs f) {
    __shared__ ResSmem sm;
    const VerifyArgs& a = f.a;
    // placement as in the count kernel (request b on XCD b % 8), R = max(H nS, K + 1)
    // workgroups per request (H = f.halves); workgroup w of a request is half w % H of slice
    // w / H of unit k (residual) or unit w (general algorithm, cache rows)
    const int H = f.halves;
    const int R = max(H * f.nS, a.K + 1);
    const int x = blockIdx.x % kXcd, l = blockIdx.x / kXcd;
    const int b = (l / R) * kXcd + x, w = l % R;
    if (b >= a.B) return;
    // what the residual needs of every unit (k picks one): row statistics, cuts, this slice's
    // flags and the draw, one 32-bit word per thread, issued before the decision's own load
    // (the slice's group masks are not among them: its tables come from its entries)
    static_assert(offsetof(UnitFast, rp) == offsetof(UnitFast, rq) + sizeof(RowFinal), "rq, rp adjacent");
    constexpr int kRf = (int)(sizeof(RowFinal) / 4), kCut = (int)(sizeof(UnitCut) / 4);
    constexpr int kWCut = 2 * kRf, kWFlag = kWCut + 4 * kCut, kWDraw = kWFlag + 2, kWEnd = kWDraw + 2, kRecWords = 64;
    static_assert(kWEnd <= kRecWords, "one unit's words in a wave");
    const bool pre = (a.K + 1) * kRecWords <= kThreads;  // otherwise loaded once k is known
    const int pj = (int)threadIdx.x / kRecWords, pw = (int)threadIdx.x % kRecWords;
    uint32_t pre_word = 0u;
    const int wslice = H == 2 ? w >> 1 : w;  // the slice of the residual this workgroup sums
    if (pre && pj <= a.K && wslice < f.nS) {
        const int uj = b * (a.K + 1) + pj;
        const UnitFast* Uj = reinterpret_cast<const UnitFast*>(f.ws + f.L.units) + uj;
        if (pw < kWCut) pre_word = ldnt(reinterpret_cast<const uint32_t*>(&Uj->rq) + pw);
        else if (pw < kWFlag) pre_word = ldnt(reinterpret_cast<const uint32_t*>(&Uj->cut[0][0]) + (pw - kWCut));
        else if (pw < kWDraw) pre_word = ldnt(&part_of(f, uj, wslice, pw - kWFlag)->flags);
        else if (pw < kWEnd) pre_word = ldnt(reinterpret_cast<const uint32_t*>(&Uj->u_res) + (pw - kWDraw));
    }
    // the request's decision and this unit's cache flag, loaded together
    static_assert(sizeof(ReqFast) == 16, "one 16-byte record");
    const u32x4 req = ldnt(reinterpret_cast<const u32x4*>(f.ws + f.L.reqs) + b);
    const bool cache_here = f.cache && w <= a.K;
    const int32_t cgen_word = ldnt(reinterpret_cast<const int32_t*>(f.ws + f.L.cache_gen) + b * (a.K + 1) + min(w, a.K));
    const int32_t cgen = cache_here ? cgen_word : 0;
    // outcome-cache rows the count kernel's candidate lists could not settle
    if (cgen) {
        CacheArgs c{a.draft, a.dtype, a.B, a.K, a.V, a.tokens, f.budget, f.fan, f.out_cache};
        cache_row<1>(c, b, w, f.fan.f[w], f.fan.off[w], sm.u.cache.rs, sm.gst[0], sm.u.cache.cs);
        __syncthreads();
    }
    const int mode = (int)req[0];
    if (mode == 0) {  // decided by the count kernel
        // the fused lookup once every cache row of the request is written (units w <= K)
        if (f.lookup && w <= a.K && arrive_last(f, sm, b, a.K + 1) && threadIdx.x == 0)
        {
            const int k = ldnt(&a.out_k[b]);
            lookup_request(f, b, k, ldnt(&a.out_t[b]), lookup_head(f, b, k));
        }
        return;
    }
    if (mode == 2) {
        if (w <= a.K) general_request(f, sm, b, w, req[2]);
        return;
    }
    // mode 1: the residual of unit k, slice w / 2; each half of the slice's loads is summed by
    // its own workgroup (both load the whole slice: the owner of a cut orders its ties over it)
    const int k = (int)req[1];
    const int slice = wslice, half = H == 2 ? w & 1 : 0;
    if (slice >= f.nS) return;
    const int unit = b * (a.K + 1) + k;
    const uint32_t status = req[2];
    const bool two = k < a.K && !f.uniform;   // a draft row at the rejected position
    const bool uni = k < a.K && f.uniform;    // the uniform draft there (residual (q - 1/V)+)
    const int c0 = slice * kSliceCols;
    const size_t stride = (size_t)a.V;
    const uint16_t* trow = static_cast<const uint16_t*>(a.target) + ((size_t)b * (a.K + 1) + k) * stride;
    const uint16_t* drow = two ? static_cast<const uint16_t*>(a.draft) + ((size_t)b * a.draft_rows + k) * stride : nullptr;
    // without the preload: the unit's record (row statistics and cuts), this slice's flags and
    // the draw for t* (taken by the count kernel with the position's acceptance draw), loaded
    // before the slice itself so that waiting for them does not wait for the slice
    uint32_t rec_word = pre_word;
    int rec_slot = pj == k ? pw : -1;
    if (!pre) {
        rec_slot = (int)threadIdx.x < kWEnd ? (int)threadIdx.x : -1;
        const UnitFast* U = reinterpret_cast<const UnitFast*>(f.ws + f.L.units) + unit;
        const int x = (int)threadIdx.x;
        if (x < kWCut) rec_word = ldnt(reinterpret_cast<const uint32_t*>(&U->rq) + x);
        else if (x < kWFlag) rec_word = ldnt(reinterpret_cast<const uint32_t*>(&U->cut[0][0]) + (x - kWCut));
        else if (x < kWDraw) rec_word = ldnt(&part_of(f, unit, slice, x - kWFlag)->flags);
        else if (x < kWEnd) rec_word = ldnt(reinterpret_cast<const uint32_t*>(&U->u_res) + (x - kWDraw));
    }
    // (without a draft row the second set re-reads the target and goes unused: unconditional
    // loads keep the waits above exact)
    // the slice's occupied bins of each row (thread t: row t / 256, entries t % 256 and t % 256 + 256;
    // within the record's entry array whatever the count, which is checked where they are used),
    // issued ahead of the columns: loads complete in order, so the tables wait only for these
    const RowPart* pr = part_of(f, unit, slice, (int)threadIdx.x / kHalf);
    const uint32_t n_ent = ldnt(&pr->n_ent);
    const uint32_t ent0 = ldnt(&pr->ent[threadIdx.x % kHalf]);
    const uint32_t ent1 = ldnt(&pr->ent[threadIdx.x % kHalf + kHalf]);
    u32x4 vq[kLoads], vp[kLoads];
    load_slice(trow, c0, a.V, vq);
    load_slice(two ? drow : trow, c0, a.V, vp);
    // the record into LDS; without a draft row its cuts keep everything and its flags are 0
    if (rec_slot >= 0) {
        if (rec_slot < kWCut) {
            reinterpret_cast<uint32_t*>(&sm.rf[0])[rec_slot] = rec_word;
        } else if (rec_slot < kWFlag) {
            const int x = rec_slot - kWCut;
            const bool keep_all = !two && x >= 2 * kCut;  // UnitCut{0, -1, 0, 0}
            reinterpret_cast<uint32_t*>(&sm.cut[0][0])[x] = keep_all ? (x % kCut == 1 ? 0xFFFFFFFFu : 0u) : rec_word;
        } else if (rec_slot < kWDraw) {
            sm.flags[rec_slot - kWFlag] = (rec_slot == kWFlag || two) ? rec_word : 0u;
        } else if (rec_slot < kWEnd) {
            reinterpret_cast<uint32_t*>(&sm.u_res)[rec_slot - kWDraw] = rec_word;
        }
    }
    if (threadIdx.x >= kWave && threadIdx.x < kWave + 6) sm.tie[(threadIdx.x - kWave) / 3][(threadIdx.x - kWave) % 3].off = kNoTie;
    __syncthreads();
    if (threadIdx.x < 2) {
        const int r = threadIdx.x;
        sm.inv[r][0] = 1.0 / sm.rf[r].S;
        sm.inv[r][1] = 1.0 / sm.rf[r].Z;
    }
    __syncthreads();  // 1 / S and 1 / Z
    // the tables need no column of the slice: they are built while its loads are in flight
    sparse_tables(sm, two, slice, pr, n_ent, ent0, ent1);
    // this slice's id cut at each cut key; the owner of a histogram cut publishes its id for
    // the finaliser (explicit cuts and no cut come from slice 0)
    slice_id_cuts(sm, vq, vp, c0, a.V, slice, two);
    __syncthreads();
    if (threadIdx.x < 4) {
        const int r = threadIdx.x >> 1, c = threadIdx.x & 1;
        const UnitCut uc = sm.cut[r][c];
        const bool writer = (uc.key == 0u || uc.explicit_id >= 0) ? slice == 0 : slice == uc.owner;
        if (writer && half == 0) reinterpret_cast<int32_t*>(f.ws + f.L.idcut)[b * 4 + threadIdx.x] = sm.eff[r][c];
    }
    residual_slice(f, sm, b, slice, half, H, c0, two, uni, vq, vp);
    if (!arrive_last(f, sm, b, H * f.nS)) return;
    finalize_residual(f, sm, b, k, status, sm.u_res);
}

// ------------------------------------------------------------------------------------------
// Fuzzy acceptance (PyramidSD notes, key design 1): a drafted token passes when the Jensen-
// Shannon divergence (bits) of the processed verifier row q_j and drafter row p'_j is at most
// the request's threshold; elsewhere the lossless test the count kernel already ran decides.
// For every request the count kernel left pending, one workgroup per slice of each drafted
// position sums the divergence over the slice with the same exact per-element values as the
// residual; the last of a position's workgroups totals it, and the last position of the
// request finds k and hands the request to the resolve kernel.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ double div_term(double q, double p) {
    const double m = 0.5 * (p + q);
    double d = 0.0;
    if (p > 0.0) d += 0.5 * p * log2(p / m);
    if (q > 0.0) d += 0.5 * q * log2(q / m);
    return d;
}
// v log2 v, 0 at v = 0.
__device__ __forceinline__ double xlog2x(double v) { return v > 0.0 ? v * log2(v) : 0.0; }

// Base-2 logarithm of the per-element and per-bin terms.  x = 2^e f with f in [1/2, 1); the
// 8 fraction bits below f's leading one pick an interval of width 2^-9 with centre c_i, and
// log2 f = log2 c_i + log2(1 + r) with r = f / c_i - 1 (|r| <= 2^-9, one fma with the
// tabulated 1 / c_i) and log2(1 + r) from the first five terms of its series.  Absolute error
// about 2e-16 on (0, 1] (about 12 fp64 operations against the library's ~60): each term
// v log2 v is off by at most v times that, so a sum over a distribution by under 1e-15.
struct LogTab {
    double2 e[256];  // {1 / c_i, log2 c_i}
};
__device__ __forceinline__ void build_logtab(LogTab& lt) {
    for (int i = (int)threadIdx.x; i < 256; i += (int)blockDim.x) {
        const double r = 1.0 / (0.5 + (i + 0.5) / 512.0);
        lt.e[i] = make_double2(r, -log2(r));
    }
}
__device__ __forceinline__ double log2_tab(double x, const LogTab& lt) {
    const double f = __builtin_amdgcn_frexp_mant(x);
    const int e = __builtin_amdgcn_frexp_exp(x);
    const double2 t = lt.e[(__double2hiint(f) >> 12) & 0xFF];
    const double r = fma(f, t.x, -1.0);
    double p = fma(r, 0.2, -0.25);
    p = fma(r, p, 1.0 / 3.0);
    p = fma(r, p, -0.5);
    p = fma(r, p, 1.0);
    return fma(r * p, 1.4426950408889634, t.y) + (double)e;
}
__device__ __forceinline__ double xlog2x_tab(double v, const LogTab& lt) { return v > 0.0 ? v * log2_tab(v, lt) : 0.0; }

// This thread's share of the divergence over the slice, every element's term whole (two
// logarithms each): the way a slice with more than kDivList elements outside the exact bins
// takes.  It loads the slice again (from cache), so that the caller's copy is dead here.
__device__ __forceinline__ double divergence_slice_whole(const FastArgs& f, ResSmem& sm, int c0, bool two,
                                                        const uint16_t* trow, const uint16_t* drow) {
    // fresh addresses: reusing the first load's would keep them live over the whole kernel
    asm volatile("" : "+s"(trow), "+s"(drow), "+s"(c0));
    u32x4 vq[kLoads], vp[kLoads];
    load_slice(trow, c0, f.a.V, vq);
    load_slice(drow, c0, f.a.V, vp);
    const double pu = 1.0 / (double)f.a.V;
    const VerifyArgs& a = f.a;
    const char* tq = reinterpret_cast<const char*>(&sm.u.tab[0][0]);
    const char* tp = reinterpret_cast<const char*>(&sm.u.tab[1][0]);
    const Ties tiq = load_ties(sm, 0);
    const Ties tip = load_ties(sm, 1);
    double tot = 0.0;
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
        const int cq = col_of(c0, q, 0);
        if (cq >= a.V) continue;
        double s = 0.0;
        bool mark = false;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t oq = tab_offsets2(vq[q][d]);
            double q0 = tab_at(tq, oq & 0xFFFFu), q1 = tab_at(tq, oq >> 16);
            if (tiq.any) apply_ties(tiq, oq, cq + 2 * d, q0, q1);
            double p0 = pu, p1 = pu;
            if (two) {
                const uint32_t op = tab_offsets2(vp[q][d]);
                p0 = tab_at(tp, op & 0xFFFFu);
                p1 = tab_at(tp, op >> 16);
                if (tip.any) apply_ties(tip, op, cq + 2 * d, p0, p1);
            }
            mark |= q0 > kMarkSeen || q1 > kMarkSeen || p0 < -kMarkSeen || p1 < -kMarkSeen;
            if (!mark) s += div_term(q0, p0) + div_term(q1, p1);
        }
        if (mark) {  // rare: values outside the exact bins, decided exactly
            s = 0.0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int col = cq + e;
                const uint32_t wq = vq[q][e >> 1];
                const uint32_t hq = (e & 1) ? (wq >> 16) : (wq & 0xFFFFu);
                const uint32_t oq = tab_offsets2(hq) & 0xFFFFu;
                double qe = tab_at(tq, oq);
                qe = qe > kMarkSeen ? final_prob(sm.rf[0], sm.inv[0], sm.eff[0][0], sm.eff[0][1], hq, col, false)
                                    : apply_ties1(tiq, oq, col, qe);
                double pe = pu;
                if (two) {
                    const uint32_t wp = vp[q][e >> 1];
                    const uint32_t hp = (e & 1) ? (wp >> 16) : (wp & 0xFFFFu);
                    const uint32_t op = tab_offsets2(hp) & 0xFFFFu;
                    pe = tab_at(tp, op);
                    pe = pe < -kMarkSeen ? final_prob(sm.rf[1], sm.inv[1], sm.eff[1][0], sm.eff[1][1], hp, col, true)
                                         : apply_ties1(tip, op, col, pe);
                }
                s += div_term(qe, pe);
            }
        }
        tot += s;
    }
    return tot;
}

constexpr int kDivList = 1024;  // elements outside the exact bins a slice lists

// Where the divergence pass keeps the listed elements: their columns in the slice, and each
// row's value (table value with the ties applied), or -(h + 1) for a marker entry (h the bf16
// logit, whose value final_prob forms).
struct DivList {
    double q[kDivList];
    double p[kDivList];
    uint16_t col[kDivList];
};

// This thread's share of the divergence over the slice.  Each element's term is split as
// (q log2 q + p log2 p) / 2 - m log2 m with m = (q + p) / 2: the first pass sums -m log2 m per
// element; the tables then turn in place into per-bin v log2 v, which the second pass sums.
// One logarithm (log2_tab) per element instead of two, and no division.  Elements whose
// value lies outside the exact bins (a marker entry) take the exact term instead: the first
// pass lists them in thread order (a workgroup scan), and the workgroup shares the list out
// once the slice is no longer needed in registers, so that a wave is not held up by its few
// lanes that hold one.
__device__ __forceinline__ double divergence_slice(const FastArgs& f, ResSmem& sm, int c0, bool two,
                                                  const u32x4 (&vq)[kLoads], const u32x4 (&vp)[kLoads],
                                                  DivList& dl, const LogTab& lt, const uint16_t* trow,
                                                  const uint16_t* drow, const SliceEnt& ent) {
    const double pu = 1.0 / (double)f.a.V;
    const VerifyArgs& a = f.a;
    const char* tq = reinterpret_cast<const char*>(&sm.u.tab[0][0]);
    const char* tp = reinterpret_cast<const char*>(&sm.u.tab[1][0]);
    Ties tiq = load_ties(sm, 0);
    Ties tip = load_ties(sm, 1);
    double tot = 0.0;
    uint32_t odd = 0u;  // bit 8 q + e: element e of load q is outside the exact bins
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
        const int cq = col_of(c0, q, 0);
        if (cq >= a.V) continue;
        double s = 0.0;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t oq = tab_offsets2(vq[q][d]);
            double q0 = tab_at(tq, oq & 0xFFFFu), q1 = tab_at(tq, oq >> 16);
            if (tiq.any) apply_ties(tiq, oq, cq + 2 * d, q0, q1);
            double p0 = pu, p1 = pu;
            if (two) {
                const uint32_t op = tab_offsets2(vp[q][d]);
                p0 = tab_at(tp, op & 0xFFFFu);
                p1 = tab_at(tp, op >> 16);
                if (tip.any) apply_ties(tip, op, cq + 2 * d, p0, p1);
            }
            const bool x0 = q0 > kMarkSeen || p0 < -kMarkSeen, x1 = q1 > kMarkSeen || p1 < -kMarkSeen;
            odd |= ((x0 ? 1u : 0u) | (x1 ? 2u : 0u)) << (8 * q + 2 * d);
            s -= xlog2x_tab(x0 ? 0.0 : 0.5 * (q0 + p0), lt) + xlog2x_tab(x1 ? 0.0 : 0.5 * (q1 + p1), lt);
        }
        tot += s;
    }
    int n_all;
    const int base = block_exclusive_scan<int>(__popc(odd), sm.redi, &n_all);
    if (n_all > kDivList) return divergence_slice_whole(f, sm, c0, two, trow, drow);
    if (odd) {
        int i = base;
#pragma unroll
        for (int q = 0; q < kLoads; ++q) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (!((odd >> (8 * q + e)) & 1u)) continue;
                const int col = col_of(c0, q, e);
                const uint32_t hq = (vq[q][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                const uint32_t oq = tab_offsets2(hq) & 0xFFFFu;
                const double qv = tab_at(tq, oq);
                double pv = pu;
                if (two) {
                    const uint32_t hp = (vp[q][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                    const uint32_t op = tab_offsets2(hp) & 0xFFFFu;
                    pv = tab_at(tp, op);
                    pv = pv < -kMarkSeen ? -(double)(hp + 1u) : apply_ties1(tip, op, col, pv);
                }
                dl.q[i] = qv > kMarkSeen ? -(double)(hq + 1u) : apply_ties1(tiq, oq, col, qv);
                dl.p[i] = pv;
                dl.col[i] = (uint16_t)(col - c0);
                ++i;
            }
        }
    }
    // every value an element inside the exact bins reads is the entry of one of the slice's own
    // occupied bins (each listed once per row: every entry turns exactly once; 0 stays 0), or a
    // tie's alternative
    __syncthreads();
    {
        const int r = (int)threadIdx.x / kHalf, i = (int)threadIdx.x % kHalf;
        if (r == 0 || two) {
            const int n = (int)min(ent.n, (uint32_t)kBins);
            double* tab = sm.u.tab[r] + kHistLead;
            if (i < n) tab[ent.e0 >> 16] = xlog2x_tab(tab[ent.e0 >> 16], lt);
            if (i + kHalf < n) tab[ent.e1 >> 16] = xlog2x_tab(tab[ent.e1 >> 16], lt);
            for (int x = i + 2 * kHalf; x < n; x += kHalf) {  // (rare: over 512 occupied bins)
                const uint32_t bin = ldnt(&ent.pr->ent[x]) >> 16;
                tab[bin] = xlog2x_tab(tab[bin], lt);
            }
        }
    }
#pragma unroll
    for (int x = 0; x < 3; ++x) {
        tiq.alt[x] = xlog2x(tiq.alt[x]);
        tip.alt[x] = xlog2x(tip.alt[x]);
    }
    __syncthreads();
    const double lpu = xlog2x(pu);  // p log2 p of every element, uniform draft
    double half = 0.0;
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
        const int cq = col_of(c0, q, 0);
        if (cq >= a.V) continue;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t oq = tab_offsets2(vq[q][d]);
            double q0 = tab_at(tq, oq & 0xFFFFu), q1 = tab_at(tq, oq >> 16);
            if (tiq.any) apply_ties(tiq, oq, cq + 2 * d, q0, q1);
            double p0 = lpu, p1 = lpu;
            if (two) {
                const uint32_t op = tab_offsets2(vp[q][d]);
                p0 = tab_at(tp, op & 0xFFFFu);
                p1 = tab_at(tp, op >> 16);
                if (tip.any) apply_ties(tip, op, cq + 2 * d, p0, p1);
            }
            const uint32_t x = odd >> (8 * q + 2 * d);
            half += ((x & 1u) ? 0.0 : q0 + p0) + ((x & 2u) ? 0.0 : q1 + p1);
        }
    }
    for (int i = (int)threadIdx.x; i < n_all; i += kThreads) {
        const int col = c0 + (int)dl.col[i];
#pragma unroll 1
        for (int r = 0; r < 2; ++r) {  // the marker entries' values, in place
            double* v = r ? &dl.p[i] : &dl.q[i];
            if (*v < 0.0) *v = final_prob(sm.rf[r], sm.inv[r], sm.eff[r][0], sm.eff[r][1], (uint32_t)(-*v) - 1u, col, r == 1);
        }
        tot += div_term(dl.q[i], dl.p[i]);
    }
    return tot + 0.5 * half;
}

// The last position of a pending request: k from the fuzzy passes and the units' own tests.
__device__ __forceinline__ void decide_fuzzy(const FastArgs& f, int b) {
    const VerifyArgs& a = f.a;
    const int K = a.K;
    const int lane = threadIdx.x & (kWave - 1);
    const UnitFast* U = reinterpret_cast<const UnitFast*>(f.ws + f.L.units) + (size_t)b * (K + 1);
    const double* D = reinterpret_cast<const double*>(f.ws + f.L.div) + (size_t)f.units * f.nS +
                      (size_t)b * (K + 1);
    uint32_t st = 0;
    int acc = 1;
    bool pass = false;
    if (lane < K) {
        st = ldnt(&U[lane].status);
        acc = ldnt(&U[lane].accept);
        pass = ldnt(&D[lane]) <= (double)a.tau[b];
    }
    const uint32_t deg = wave_or(st & kStDegenerate);
    int k = first_lane(__ballot(lane < K && !pass && !acc));
    if (k < 0) k = K;
    // a position that passed on its divergence never took the lossless test
    const uint32_t outside = wave_or((lane < K && lane <= k && !pass) ? (st & kStOutside) : 0u);
    if (lane == 0) {
        ReqFast* Rq = reinterpret_cast<ReqFast*>(f.ws + f.L.reqs) + b;
        Rq->mode = 1;
        Rq->k = k;
        Rq->status = deg | outside;
    }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void fast_diverge_kernel(FastArgs f) {
    __shared__ ResSmem sm;
    __shared__ DivList dl;
    __shared__ LogTab lt;
    const VerifyArgs& a = f.a;
    // placement as in the count kernel (request b on XCD b % 8); workgroup w of a request is
    // slice w % nS of drafted position w / nS
    const int R = f.nS * a.K;
    const int x = blockIdx.x % kXcd, l = blockIdx.x / kXcd;
    const int b = (l / R) * kXcd + x, w = l % R;
    if (b >= a.B) return;
    const u32x4 req = ldnt(reinterpret_cast<const u32x4*>(f.ws + f.L.reqs) + b);
    if ((int)req[0] != 3) return;
    const int j = w / f.nS, slice = w % f.nS;
    const int unit = b * (a.K + 1) + j;
    const bool two = !f.uniform;
    constexpr int kRf = (int)(sizeof(RowFinal) / 4), kCut = (int)(sizeof(UnitCut) / 4);
    constexpr int kWCut = 2 * kRf, kWFlag = kWCut + 4 * kCut, kWEnd = kWFlag + 2;
    static_assert(kWEnd <= kThreads, "one record word per thread");
    const UnitFast* U = reinterpret_cast<const UnitFast*>(f.ws + f.L.units) + unit;
    const int t = (int)threadIdx.x;
    uint32_t rec_word = 0u;
    if (t < kWCut) rec_word = ldnt(reinterpret_cast<const uint32_t*>(&U->rq) + t);
    else if (t < kWFlag) rec_word = ldnt(reinterpret_cast<const uint32_t*>(&U->cut[0][0]) + (t - kWCut));
    else if (t < kWEnd) rec_word = ldnt(&part_of(f, unit, slice, t - kWFlag)->flags);
    const int c0 = slice * kSliceCols;
    const size_t stride = (size_t)a.V;
    const uint16_t* trow = static_cast<const uint16_t*>(a.target) + ((size_t)b * (a.K + 1) + j) * stride;
    const uint16_t* drow = two ? static_cast<const uint16_t*>(a.draft) + ((size_t)b * a.draft_rows + j) * stride : trow;
    // the slice's occupied bins, ahead of its columns (the tables wait only for them)
    const SliceEnt ent = load_slice_ent(f, unit, slice);
    u32x4 vq[kLoads], vp[kLoads];
    load_slice(trow, c0, a.V, vq);
    load_slice(drow, c0, a.V, vp);
    build_logtab(lt);
    if (t < kWCut) {
        reinterpret_cast<uint32_t*>(&sm.rf[0])[t] = rec_word;
    } else if (t < kWFlag) {
        const int y = t - kWCut;
        const bool keep_all = !two && y >= 2 * kCut;  // no draft row: UnitCut{0, -1, 0, 0}
        reinterpret_cast<uint32_t*>(&sm.cut[0][0])[y] = keep_all ? (y % kCut == 1 ? 0xFFFFFFFFu : 0u) : rec_word;
    } else if (t < kWEnd) {
        sm.flags[t - kWFlag] = (t == kWFlag || two) ? rec_word : 0u;
    }
    if (t >= kWave && t < kWave + 6) sm.tie[(t - kWave) / 3][(t - kWave) % 3].off = kNoTie;
    __syncthreads();
    if (t < 2) {
        sm.inv[t][0] = 1.0 / sm.rf[t].S;
        sm.inv[t][1] = 1.0 / sm.rf[t].Z;
    }
    __syncthreads();  // 1 / S and 1 / Z
    // the tables need no column of the slice: they are built while its loads are in flight
    sparse_tables(sm, two, slice, ent.pr, ent.n, ent.e0, ent.e1);
    slice_id_cuts(sm, vq, vp, c0, a.V, slice, two);
    __syncthreads();
    const double part = block_sum<double>(divergence_slice(f, sm, c0, two, vq, vp, dl, lt, trow, drow, ent), sm.redd);
    double* parts = reinterpret_cast<double*>(f.ws + f.L.div);
    if (t == 0) parts[(size_t)unit * f.nS + slice] = part;
    // the position's arrival (its nS workgroups), then the request's (its K positions)
    drain_stores();
    __syncthreads();
    if (t == 0) {
        unsigned* uc = reinterpret_cast<unsigned*>(f.ws + f.L.unit_ctr + (size_t)unit * 128);
        const unsigned old = l2_fetch_add(uc, 1u);
        sm.last = (old + 1 == (unsigned)f.nS) ? 1 : 0;
        if (sm.last) *uc = 0u;
    }
    __syncthreads();
    if (!sm.last) return;
    if (t < kWave) {
        const double v = t < f.nS ? ldnt(&parts[(size_t)unit * f.nS + t]) : 0.0;
        const double Dj = wave_sum(v);  // fixed order: the same bits on every run
        if (t == 0) {
            reinterpret_cast<double*>(f.ws + f.L.div)[(size_t)f.units * f.nS + unit] = Dj;
            if (a.out_div) a.out_div[(size_t)b * a.K + j] = (float)Dj;
        }
    }
    drain_stores();
    __syncthreads();
    if (t == 0) {
        unsigned* rc = reinterpret_cast<unsigned*>(f.ws + f.L.req_ctr + (size_t)b * 128);
        const unsigned old = l2_fetch_add(rc, 1u);
        sm.last = (old + 1 == (unsigned)a.K) ? 1 : 0;
        if (sm.last) *rc = 0u;
    }
    __syncthreads();
    if (!sm.last || t >= kWave) return;
    decide_fuzzy(f, b);
}

void launch_diverge(const FastArgs& f, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(fast_diverge_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, f);
}

void launch_resolve(const FastArgs& f, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(fast_resolve_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, f);
}

int resolve_resident() {
    // per device, worked out once (0 until then: a failed query keeps two workgroups per slice)
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 1 << 30;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fast_resolve_kernel, kThreads, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu <= 0 || cus <= 0)
        return 1 << 30;
    v = per_cu * cus;
    cached[dev].store(v, std::memory_order_relaxed);
    return v;
}

}  // namespace fast
}  // namespace sv
