// Register-resident bf16 verification path: see fastpath.h for the structure.
//
// What is computed is the same as the general path (generic.hip): temperature, top-k, softmax
// and nucleus processing of draft and target rows (DeepMind speculative-sampling page, section
// 6), Saguaro sigma_{F,C} on the draft (SSD reading notes, section 4.4; hyper.ai summary,
// Method), the min(1, q/p) acceptance test with first-rejection cutoff and the residual /
// bonus sampling (DeepMind page, sections 1 and 3; SSD reading notes, section 2.2).
//
// How it is computed differs: bf16 logits take few distinct values, so a row's processed
// distribution is fixed by the count of every distinct value.  Counting replaces the
// per-element exp: masses are count * exp((z - m)/T) in fp64, one exp per distinct value.
#include "fastpath.h"
#include "rowproc.h"

namespace sv {
namespace fast {

// ------------------------------------------------------------------------------------------
// bf16 values, bins and segments
// ------------------------------------------------------------------------------------------
enum : int { kKindBin = 0, kKindSpecial = 1, kKindNegInf = 2, kKindBad = 3 };

__device__ __forceinline__ int classify(uint32_t h, int* bin) {
    const uint32_t mag = h & 0x7FFFu;
    const uint32_t e = mag >> 7;
    if (e >= (uint32_t)kExpLo && e < (uint32_t)kExpHi) {
        const int off = (int)mag - (kExpLo << 7);
        *bin = (h & 0x8000u) ? (kNegBins - 1 - off) : (kPosBase + off);
        return kKindBin;
    }
    if (mag == 0) {
        *bin = kZeroBin;
        return kKindBin;
    }
    if (mag < 0x7F80u) return kKindSpecial;
    if (mag == 0x7F80u && (h & 0x8000u)) return kKindNegInf;
    return kKindBad;  // +inf or NaN
}

// 16-bit order key of a bf16 value (grows with the value; -0 folded onto +0).
__device__ __forceinline__ uint32_t key16(uint32_t h) {
    if (h == 0x8000u) h = 0;
    return (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
}
__device__ __forceinline__ float key16_value(uint32_t k) {
    const uint32_t h = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
    return __uint_as_float(h << 16);
}
__device__ __forceinline__ uint32_t bin_key(int bin) {
    if (bin < kNegBins) return key16(0x8000u | (uint32_t)((kExpLo << 7) + (kNegBins - 1 - bin)));
    if (bin < kPosBase) return 0x8000u;
    return key16((uint32_t)((kExpLo << 7) + (bin - kPosBase)));
}
// bin of an order key known to be in the exact range (or zero)
__device__ __forceinline__ int key_bin(uint32_t k) {
    const uint32_t h = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
    int b = -1;
    classify(h, &b);
    return b;
}
__device__ __forceinline__ bool key_is_binned(uint32_t k) {
    const uint32_t h = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
    int b;
    return classify(h, &b) == kKindBin;
}
__host__ __device__ constexpr int seg_of_group(int g) {
    return g < kNegGroups ? (kSegTinyNeg + 1 + (kNegGroups - 1 - g)) : (g == kZeroGroup ? kSegZero : 1 + (kGroups - 1 - g));
}
__host__ __device__ constexpr int group_of_seg(int s) {
    return (s >= 1 && s < kSegTinyPos) ? (kGroups - s)
           : (s == kSegZero ? kZeroGroup : ((s > kSegTinyNeg && s < kSegHugeNeg) ? (kNegGroups - 1 - (s - kSegTinyNeg - 1)) : -1));
}
static_assert(group_of_seg(seg_of_group(0)) == 0, "segment map");
static_assert(group_of_seg(seg_of_group(kNegGroups - 1)) == kNegGroups - 1, "segment map");
static_assert(group_of_seg(seg_of_group(kZeroGroup)) == kZeroGroup, "segment map");
static_assert(group_of_seg(seg_of_group(kZeroGroup + 1)) == kZeroGroup + 1, "segment map");
static_assert(group_of_seg(seg_of_group(kGroups - 1)) == kGroups - 1, "segment map");
static_assert(seg_of_group(kGroups - 1) == 1 && seg_of_group(kNegGroups - 1) == kSegTinyNeg + 1, "segment order");
static_assert(seg_of_group(0) == kSegHugeNeg - 1, "segment order");

// segment of a special (finite, outside the exact bins) key
__device__ __forceinline__ int special_seg(uint32_t k) {
    const bool pos = (k & 0x8000u) != 0;
    const uint32_t h = pos ? (k & 0x7FFFu) : (~k & 0xFFFFu);
    const bool huge = ((h & 0x7FFFu) >> 7) >= (uint32_t)kExpHi;
    return pos ? (huge ? kSegHugePos : kSegTinyPos) : (huge ? kSegHugeNeg : kSegTinyNeg);
}

// ------------------------------------------------------------------------------------------
// Workspace records
// ------------------------------------------------------------------------------------------
struct RowPart {  // one slice of one row, published before the unit barrier
    float m;            // largest finite logit of the slice, -inf when none
    uint32_t maxkey;
    uint32_t flags;     // 1: NaN or +inf seen, 2: special list overflow
    uint32_t n_neginf;
    uint32_t n_finite;
    uint32_t n_special;
    uint32_t n_top;
    uint32_t rank_s;    // (slice owning s) elements with key == key(s) and id < s
    double S;           // sum of exp((z - m)/T) over the slice's finite elements
    double seg_mass[kSegs];
    uint32_t seg_count[kSegs];
    uint32_t top_key[kTop];
    int32_t top_id[kTop];
    uint32_t sp_key[kSpecial];
    int32_t sp_id[kSpecial];
    uint16_t fine[kBins];
};

struct RowFinal {  // enough to evaluate any element's processed probability
    float m;
    float T;
    double S;      // normaliser of the processed distribution
    double C;      // factor on the downweighted set (1 when off)
    double Z;      // normaliser after the downweight (1 when off)
    uint32_t kk;   // top-k cut key (id cut in UnitFast::idcut[.][0])
    uint32_t kp;   // nucleus cut key (id cut in UnitFast::idcut[.][1])
    uint32_t kF;   // downweighted set: key > kF, or key == kF and id <= idF (nS > 0)
    int32_t idF;
    int32_t nS;
    int32_t argmax;
    int32_t greedy;
    int32_t has_special;  // slices hold finite values outside the bins (finalizer recomputes them)
};

struct UnitFast {
    int32_t accept;
    uint32_t status;
    int32_t fallback;   // processed by the general algorithm: tcand / W are final
    int32_t tcand;
    float W;
    int32_t pad;
    RowFinal rq, rp;
};

struct Layout {
    size_t req, parts, units, idcut, chunks, total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

__host__ __device__ inline Layout layout(int B, int units, int nS) {
    Layout L;
    size_t o = 0;
    L.req = o;    o += align256((size_t)B * 128);               // request arrival counters
    L.parts = o;  o += align256((size_t)units * nS * 2 * sizeof(RowPart));
    L.units = o;  o += align256((size_t)units * sizeof(UnitFast));
    L.idcut = o;  o += align256((size_t)units * 4 * sizeof(int32_t));
    L.chunks = o; o += align256((size_t)units * nS * kChunks * sizeof(double));
    L.total = o;
    return L;
}

struct FastArgs {
    VerifyArgs a;
    int nS;
    int units;
    char* ws;
    Layout L;
};

// ------------------------------------------------------------------------------------------
// Request arrival counter in the XCD's L2 (every workgroup of a request runs on one XCD)
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ unsigned l2_fetch_add(unsigned* p, unsigned v) {
    unsigned old;
    asm volatile("s_waitcnt vmcnt(0)\n\tglobal_atomic_add %0, %1, %2, off sc0\n\ts_waitcnt vmcnt(0)"
                 : "=v"(old) : "v"(p), "v"(v) : "memory");
    return old;
}

// Every wave waits until its own global stores have reached L2; __syncthreads() alone orders
// only LDS traffic, so this must precede the workgroup barrier in front of an arrival.
__device__ __forceinline__ void drain_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ------------------------------------------------------------------------------------------
// Loads of data published by other workgroups (non-temporal: bypass L1, served by L2)
// ------------------------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ T ldnt(const T* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint32_t ldnt_u16(const uint16_t* p) {
    // u16 via the enclosing aligned dword
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const uint32_t w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(a & ~(uintptr_t)3));
    return (a & 2) ? (w >> 16) : (w & 0xFFFFu);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Columns of a slice are held as: load q, thread t, element e  ->  c0 + q*kThreads*8 + t*8 + e,
// so (q, t, e) in lexicographic order is token-id order.
__device__ __forceinline__ int col_of(int c0, int q, int e) { return c0 + q * kThreads * 8 + (int)threadIdx.x * 8 + e; }

// ------------------------------------------------------------------------------------------
// Shared memory
// ------------------------------------------------------------------------------------------
constexpr int kWaves = kThreads / kWave;
constexpr int kMergeCap = 1024;   // merged candidates (top lists or one segment's specials)

struct Cut {       // a cut in token order: keep key > key, and the first `take` elements at key
    uint32_t key;
    int take;      // elements taken at `key` (histogram cuts)
    int explicit_id;  // >= 0: the id of the last kept element (explicit cuts); -1: histogram cut
    int owner;     // histogram cut: slice holding the last kept tie
    int owner_take;   // ties the owner keeps
    int eff;       // this slice's id cut at `key` (V - 1: all, -1: none, else an id)
    int count_above;  // elements with key > cut key (histogram cuts)
};

struct RowView {   // the combined view of one row, identical in every slice of the unit
    int bad, overflow, greedy, argmax;
    float m;
    double T;
    double seg_mass[kSegs];
    uint32_t seg_count[kSegs];
    double sc[32];         // per-slice rescale exp((m_t - m)/T)
    uint32_t n_finite;
    double S_all, S_kept, S;
    int has_k, has_p;      // top-k / nucleus active
    Cut ck, cp;
    int n_kept;            // elements kept by top-k (or all finite)
    int n_nuc;             // elements in the nucleus
    int nset;              // downweighted set size (0: off)
    uint32_t kF;
    int idF;
    double C, Z;
    int degenerate;
    int has_special;
    // token s of this row
    uint32_t key_s;
    float z_s;
    double prob_s;
};

struct Smem {
    double segm[kSegs];
    uint32_t segc[kSegs];
    UnitRec urec;
    union {
        uint32_t hist[2][kBins];
        double tab[2][kBins];
        struct {
            uint32_t key[kMergeCap];
            int32_t id[kMergeCap];
            uint32_t okey[kTop];
            int32_t oid[kTop];
            uint32_t fine[kGroup];
            uint32_t fine8[kWaves][kGroup];
            int32_t toff[32];
            int32_t tcnt[32];
            int32_t ttotal;
        } m;
        RowShared generic;
    } u;
    RowStats gst[2];
    uint32_t sp_key[2][kSpecial];
    int32_t sp_id[2][kSpecial];
    uint32_t n_sp[2];
    uint32_t top_key[kTop];
    int32_t top_id[kTop];
    uint32_t n_top;
    uint32_t flags[2];
    uint32_t neginf[2];
    int32_t scan[kWaves + 1];
    double redd[kWaves];
    int32_t redi[kWaves];
    RowView rv[2];
    uint32_t s_bits[2];   // bf16 bits of token s in each row
    // values handed between the steps of one helper
    uint32_t tau;
    int need;
    int cut_seg;
    int cut_cnt_above;
    int cut_nin;
    double cut_above;
    double cut_mass_above;
    double cut_w;
    double cut_mass;
    int last;
    int found;
    uint32_t fin[2 * sizeof(RowFinal) / 4];
    int fk, ft, fmode, fc;
    uint32_t fstatus;
    double fW, ftarget, fbase;
};

__device__ __forceinline__ RowPart* part_of(const FastArgs& f, int unit, int slice, int r) {
    return reinterpret_cast<RowPart*>(f.ws + f.L.parts) + ((size_t)unit * f.nS + slice) * 2 + r;
}

// e of a finite value relative to the row's largest logit
__device__ __forceinline__ double mass_of(float z, float m, double T) { return exp(((double)z - (double)m) / T); }

// key of any finite bf16 (bin or special)
__device__ __forceinline__ bool cut_keeps(const Cut& c, uint32_t key, int col) {
    return key > c.key || (key == c.key && col <= c.eff);
}

// ------------------------------------------------------------------------------------------
// Phase A helpers
// ------------------------------------------------------------------------------------------
// Segment of any finite order key.
__device__ __forceinline__ int seg_of_key(uint32_t k) {
    return key_is_binned(k) ? seg_of_group(key_bin(k) / kGroup) : special_seg(k);
}

// Bin of lane `lane` in a walk over group g in descending key order.
__device__ __forceinline__ int bin_of_sel(int g, int lane) { return g * kGroup + (kGroup - 1 - lane); }

// ------------------------------------------------------------------------------------------
// Phase C: combining the slices' summaries of one row (every slice computes the same view)
// ------------------------------------------------------------------------------------------
// Merged candidates of the unit's slices for row r, sorted (key desc, id asc), into
// sm.u.m.okey / oid; returns their number (<= want).  Source: each slice's top list.
__device__ __forceinline__ int merge_tops(const FastArgs& f, Smem& sm, int unit, int r, int want) {
    const int lane = threadIdx.x & (kWave - 1);
    if (threadIdx.x < kWave) {  // list lengths and offsets, one lane per slice
        const int nt = lane < f.nS ? (int)ldnt(&part_of(f, unit, lane, r)->n_top) : 0;
        int ex;
        const int in = wave_scan(nt, &ex);
        if (lane < f.nS) {
            sm.u.m.toff[lane] = ex;
            sm.u.m.tcnt[lane] = nt;
        }
        const int tot = __shfl(in, kWave - 1, kWave);
        if (lane == 0) sm.u.m.ttotal = tot;
    }
    __syncthreads();
    const int n = min(sm.u.m.ttotal, kMergeCap);
    for (int i = threadIdx.x; i < f.nS * kTop; i += blockDim.x) {  // all entries at once
        const int t = i / kTop, x = i % kTop;
        if (x < sm.u.m.tcnt[t]) {
            const int d = sm.u.m.toff[t] + x;
            if (d < kMergeCap) {
                const RowPart* P = part_of(f, unit, t, r);
                sm.u.m.key[d] = ldnt(&P->top_key[x]);
                sm.u.m.id[d] = ldnt(&P->top_id[x]);
            }
        }
    }
    __syncthreads();
    // rank every entry; keep those with rank < want
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const uint32_t k = sm.u.m.key[i];
        const int id = sm.u.m.id[i];
        int rank = 0;
        for (int x = 0; x < n; ++x) {
            const uint32_t k2 = sm.u.m.key[x];
            rank += (k2 > k || (k2 == k && sm.u.m.id[x] < id)) ? 1 : 0;
        }
        if (rank < want && rank < kTop) {
            sm.u.m.okey[rank] = k;
            sm.u.m.oid[rank] = id;
        }
    }
    __syncthreads();
    return min(n, min(want, kTop));
}

// Specials of segment sg of row r from every slice, sorted (key desc, id asc) into sm.u.m
// key/id; returns their number.
__device__ __forceinline__ int merge_specials(const FastArgs& f, Smem& sm, int unit, int r, int sg) {
    __shared__ int s_n;
    if (threadIdx.x == 0) s_n = 0;
    __syncthreads();
    for (int t = 0; t < f.nS; ++t) {
        const RowPart* P = part_of(f, unit, t, r);
        const int ns = min((int)ldnt(&P->n_special), kSpecial);
        for (int i = threadIdx.x; i < ns; i += blockDim.x) {
            const uint32_t k = ldnt(&P->sp_key[i]);
            if (special_seg(k) != sg) continue;
            const int slot = atomicAdd(&s_n, 1);
            if (slot < kMergeCap / 2) {
                sm.u.m.key[kMergeCap / 2 + slot] = k;
                sm.u.m.id[kMergeCap / 2 + slot] = ldnt(&P->sp_id[i]);
            }
        }
    }
    __syncthreads();
    const int n = min(s_n, kMergeCap / 2);
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const uint32_t k = sm.u.m.key[kMergeCap / 2 + i];
        const int id = sm.u.m.id[kMergeCap / 2 + i];
        int rank = 0;
        for (int x = 0; x < n; ++x) {
            const uint32_t k2 = sm.u.m.key[kMergeCap / 2 + x];
            rank += (k2 > k || (k2 == k && sm.u.m.id[kMergeCap / 2 + x] < id)) ? 1 : 0;
        }
        sm.u.m.key[rank] = k;
        sm.u.m.id[rank] = id;
    }
    __syncthreads();
    return n;
}

// Fine counts of group g of row r summed over the slices into sm.u.m.fine[64]: wave w reads
// slices w, w + 8, ...; the eight partial sums are added in a fixed order.
__device__ __forceinline__ void merge_fine(const FastArgs& f, Smem& sm, int unit, int r, int g) {
    const int bb = threadIdx.x & (kGroup - 1);
    const int w = threadIdx.x / kGroup;
    uint32_t c = 0;
    for (int t = w; t < f.nS; t += kWaves) c += ldnt_u16(&part_of(f, unit, t, r)->fine[g * kGroup + bb]);
    sm.u.m.fine8[w][bb] = c;
    __syncthreads();
    if (threadIdx.x < kGroup) {
        uint32_t s = 0;
#pragma unroll
        for (int x = 0; x < kWaves; ++x) s += sm.u.m.fine8[x][threadIdx.x];
        sm.u.m.fine[threadIdx.x] = s;
    }
    __syncthreads();
}

// Wave 0: the slice holding the take-th element (token order) of bin `bin` of row r, and how
// many of that bin's elements it keeps: c.owner, c.owner_take (one lane per slice).
__device__ __forceinline__ void tie_owner(const FastArgs& f, int unit, int r, int bin, Cut& c) {
    const int lane = threadIdx.x & (kWave - 1);
    const int take = c.take;
    const int n = lane < f.nS ? (int)ldnt_u16(&part_of(f, unit, lane, r)->fine[bin]) : 0;
    int ex;
    const int in = wave_scan(n, &ex);
    const int t = first_lane(__ballot(lane < f.nS && in >= take));
    if (t < 0) {
        if (lane == 0) {
            c.owner = f.nS - 1;
            c.owner_take = 0;
        }
    } else if (lane == t) {
        c.owner = t;
        c.owner_take = take - ex;
    }
}

// The cut where the running weight over row r, walked from the largest key down, first
// reaches `need`.  Weights are counts (MASS false) or masses cnt * e (MASS true); elements
// are restricted to the `lim` cut when given (nucleus inside a top-k set).  The walk is a
// prefix scan over the 49 segments, then over the 64 bins of the crossing group (or the
// specials of the crossing segment).  Results: *out (LDS), sm.cut_w (weight kept),
// sm.cut_mass (mass kept), sm.cut_nin (elements kept).
template <bool MASS>
__device__ __forceinline__ void find_cut(const FastArgs& f, Smem& sm, int unit, int r, double need, bool has_lim,
                                         const Cut lim_cut, Cut* out) {
    const Cut* lim = has_lim ? &lim_cut : nullptr;
    const RowView& rv = sm.rv[r];
    const int lane = threadIdx.x & (kWave - 1);
    const bool w0 = threadIdx.x < kWave;
    // 1. crossing segment; the walk stops at the limit's segment, which is resolved below
    if (w0) {
        const int lim_seg = lim ? seg_of_key(lim->key) : kSegs;
        const bool live = lane < kSegs && lane < lim_seg;
        const uint32_t cnt = lane < kSegs ? rv.seg_count[lane] : 0u;
        const double ms = live ? rv.seg_mass[lane] : 0.0;
        const double w = live ? (MASS ? ms : (double)cnt) : 0.0;
        double wex, mex;
        int cex;
        const double win = wave_scan(w, &wex);
        wave_scan(ms, &mex);
        wave_scan(live ? (int)cnt : 0, &cex);
        const bool cross = lane < kSegs && (lane >= lim_seg || (cnt > 0 && win >= need));
        int pick = first_lane(__ballot(cross));
        if (pick < 0) {  // rounding left the target beyond the last segment: its last non-empty one
            pick = last_lane(__ballot(lane < kSegs && cnt > 0));
            if (pick < 0) pick = kSegs - 1;
        }
        const double wa = __shfl(wex, pick, kWave);
        const double ma = __shfl(mex, pick, kWave);
        const int ca = __shfl(cex, pick, kWave);
        if (lane == 0) {
            sm.cut_seg = pick;
            sm.cut_above = wa;
            sm.cut_mass_above = ma;
            sm.cut_cnt_above = ca;
        }
    }
    __syncthreads();
    const int sg = sm.cut_seg;
    const int g = group_of_seg(sg);
    if (g >= 0) {
        merge_fine(f, sm, unit, r, g);
        if (w0) {
            const int bb = kGroup - 1 - lane;  // lane order = descending key
            const int bin = g * kGroup + bb;
            const uint32_t key = bin_key(bin);
            int n = (int)sm.u.m.fine[bb];
            const bool at_lim = lim && key == lim->key;
            if (lim && key < lim->key) n = 0;
            if (at_lim) n = min(n, lim->take);
            const double e = n > 0 ? mass_of(key16_value(key), rv.m, rv.T) : 0.0;
            const double w = MASS ? (double)n * e : (double)n;
            double wex, mex;
            int nex;
            const double win = wave_scan(w, &wex);
            wave_scan((double)n * e, &mex);
            wave_scan(n, &nex);
            const double above0 = sm.cut_above;
            const uint64_t hc = __ballot(n > 0 && (above0 + win >= need || at_lim));
            const bool done = hc != 0;
            // not done: rounding left the target just beyond the group; cut at its lowest bin
            const int sel = done ? first_lane(hc) : last_lane(__ballot(n > 0));
            if (lane == sel) {
                const double above = above0 + wex;
                int take = n;
                if (done && above + w >= need) {
                    if (MASS) {
                        if (e > 0.0) {
                            const double q = ceil((need - above) / e);
                            take = q < 1.0 ? 1 : (q > (double)n ? n : (int)q);
                        }
                    } else {
                        take = (int)(need - above);
                        take = take < 1 ? 1 : (take > n ? n : take);
                    }
                }
                Cut c;
                c.key = key;
                c.take = take;
                c.explicit_id = -1;
                c.owner = 0;
                c.owner_take = 0;
                c.eff = 0;
                c.count_above = sm.cut_cnt_above + nex;
                *out = c;
                sm.cut_w = above + (MASS ? (double)take * e : (double)take);
                sm.cut_mass = sm.cut_mass_above + mex + (double)take * e;
                sm.cut_nin = c.count_above + take;
            }
            if (sel < 0 && lane == 0) {
                Cut c;
                c.key = 0u;
                c.take = 0;
                c.explicit_id = -1;
                c.owner = 0;
                c.owner_take = 0;
                c.eff = 0;
                c.count_above = sm.cut_cnt_above;
                *out = c;
                sm.cut_w = above0;
                sm.cut_mass = sm.cut_mass_above;
                sm.cut_nin = sm.cut_cnt_above;
            }
            if (sel >= 0) tie_owner(f, unit, r, bin_of_sel(g, sel), *out);
        }
        __syncthreads();
    } else {
        const int n = merge_specials(f, sm, unit, r, sg);
        if (threadIdx.x == 0) {  // rare: finite values outside the exact bins
            double above = sm.cut_above, mass = sm.cut_mass_above;
            Cut c;
            c.key = 0u;
            c.take = 0;
            c.explicit_id = -1;
            c.owner = 0;
            c.owner_take = 0;
            c.eff = 0;
            c.count_above = sm.cut_cnt_above;
            int i = 0;
            for (; i < n; ++i) {
                const uint32_t key = sm.u.m.key[i];
                if (lim && (key < lim->key || (key == lim->key && lim->explicit_id >= 0 && sm.u.m.id[i] > lim->explicit_id))) break;
                const double e = mass_of(key16_value(key), rv.m, rv.T);
                above += MASS ? e : 1.0;
                mass += e;
                if (above >= need) {
                    c.key = key;
                    c.explicit_id = sm.u.m.id[i];
                    ++i;
                    break;
                }
            }
            if (c.explicit_id < 0 && i > 0) {  // the limit (or rounding) ends the walk
                c.key = sm.u.m.key[i - 1];
                c.explicit_id = sm.u.m.id[i - 1];
            }
            *out = c;
            sm.cut_w = above;
            sm.cut_mass = mass;
            sm.cut_nin = sm.cut_cnt_above + i;
        }
        __syncthreads();
    }
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

// Global rank (0-based, token order) of token s among the elements of row r with
// key == key_s.  Wave-level: every wave computes it, one lane per preceding slice.
__device__ __forceinline__ int global_rank_s(const FastArgs& f, int unit, int r, uint32_t key_s, int s) {
    const int lane = threadIdx.x & (kWave - 1);
    const int owner = s / kSliceCols;
    int acc = 0;
    if (lane < owner && lane < f.nS) {
        const RowPart* P = part_of(f, unit, lane, r);
        if (key_is_binned(key_s)) {
            acc = (int)ldnt_u16(&P->fine[key_bin(key_s)]);
        } else {
            const int ns = min((int)ldnt(&P->n_special), kSpecial);
            for (int i = 0; i < ns; ++i) acc += (ldnt(&P->sp_key[i]) == key_s) ? 1 : 0;
        }
    }
    return wave_sum(acc) + (int)ldnt(&part_of(f, unit, owner, r)->rank_s);
}

__device__ __forceinline__ bool cut_keeps_s(const FastArgs& f, int unit, int r, const Cut& c, uint32_t key_s, int s) {
    if (key_s > c.key) return true;
    if (key_s < c.key) return false;
    if (c.explicit_id >= 0) return s <= c.explicit_id;
    return global_rank_s(f, unit, r, key_s, s) < c.take;
}

// ------------------------------------------------------------------------------------------
// Combine one row (all threads; every slice of the unit derives the same view)
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void combine_row(const FastArgs& f, Smem& sm, int unit, int r, const spec_params& prm, bool draft) {
    RowView& rv = sm.rv[r];
    const VerifyArgs& a = f.a;
    const double T = (double)prm.temperature;
    const int lane = threadIdx.x & (kWave - 1);
    const bool w0 = threadIdx.x < kWave;
    if (w0) {  // slice headers, one lane per slice
        float mt = -__builtin_inff();
        uint32_t fl = 0, nf = 0, nsp = 0;
        double St = 0.0;
        if (lane < f.nS) {
            const RowPart* P = part_of(f, unit, lane, r);
            mt = ldnt(&P->m);
            fl = ldnt(&P->flags);
            nf = ldnt(&P->n_finite);
            nsp = ldnt(&P->n_special);
            St = ldnt(&P->S);
        }
        const float m = wave_max(mt);
        const uint32_t flo = wave_or(fl);
        const uint32_t nfin = wave_sum(nf);
        const bool has_sp = __ballot(nsp > 0) != 0;
        const double sc = (lane < f.nS && T > 0.0 && mt > -__builtin_inff()) ? exp(((double)mt - (double)m) / T) : 0.0;
        const double S = wave_sum(sc * St);
        if (lane < 32) rv.sc[lane] = sc;
        if (lane == 0) {
            rv.m = m;
            rv.T = T;
            rv.bad = ((flo & 1u) || nfin == 0) ? 1 : 0;
            rv.overflow = (flo & 2u) ? 1 : 0;
            rv.n_finite = nfin;
            rv.greedy = prm.temperature == 0.0f ? 1 : 0;
            rv.has_special = has_sp ? 1 : 0;
            rv.argmax = -1;
            rv.S_all = S;
            rv.has_k = (prm.top_k > 0 && prm.top_k < a.V) ? 1 : 0;
            rv.has_p = ((double)prm.top_p < 1.0) ? 1 : 0;
            rv.ck = Cut{0, 0, -1, 0, 0, a.V - 1, 0};
            rv.cp = Cut{0, 0, -1, 0, 0, a.V - 1, 0};
            rv.nset = 0;
            rv.kF = 0xFFFFFFFFu;
            rv.idF = -1;
            rv.C = 1.0;
            rv.Z = 1.0;
            rv.degenerate = 0;
        }
    }
    __syncthreads();
    if (rv.bad || rv.overflow) return;
    // how many leading elements of the merged order are needed explicitly
    const bool small_k = rv.has_k && prm.top_k <= kTop;
    const bool want_set = draft && a.F > 0 && a.C < 1.0f && !rv.greedy;
    int want = rv.greedy ? 1 : 0;
    if (small_k) want = max(want, prm.top_k);
    if (want_set) want = max(want, a.F);
    int nm = 0;
    if (want > 0) nm = merge_tops(f, sm, unit, r, want);
    if (rv.greedy) {
        if (threadIdx.x == 0) rv.argmax = nm > 0 ? sm.u.m.oid[0] : -1;
        __syncthreads();
        return;
    }
    if (rv.has_k && (uint32_t)prm.top_k > rv.n_finite) {  // -inf tokens would be kept
        __syncthreads();
        if (threadIdx.x == 0) rv.overflow = 1;
        __syncthreads();
        return;
    }
    // merged segment weights: eight lanes per segment, slices t, t + 8, ... each
    {
        const int sg = threadIdx.x / 8, t0 = threadIdx.x % 8;
        double ms = 0.0;
        uint32_t cs = 0;
        if (sg < kSegs) {
            for (int t = t0; t < f.nS; t += 8) {
                const RowPart* P = part_of(f, unit, t, r);
                ms += rv.sc[t] * ldnt(&P->seg_mass[sg]);
                cs += ldnt(&P->seg_count[sg]);
            }
        }
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) {
            ms += __shfl_xor(ms, o, kWave);
            cs += __shfl_xor(cs, o, kWave);
        }
        if (sg < kSegs && t0 == 0) {
            rv.seg_mass[sg] = ms;
            rv.seg_count[sg] = cs;
        }
    }
    __syncthreads();
    // top-k
    if (!rv.has_k) {
        if (threadIdx.x == 0) {
            rv.S_kept = rv.S_all;
            rv.n_kept = (int)rv.n_finite;
        }
    } else if (small_k) {
        if (w0) {
            const int kk = prm.top_k;
            const double e = lane < kk ? mass_of(key16_value(sm.u.m.okey[lane]), rv.m, T) : 0.0;
            const double s = wave_sum(e);
            if (lane == 0) {
                rv.S_kept = s;
                rv.n_kept = kk;
                rv.ck = Cut{sm.u.m.okey[kk - 1], 0, sm.u.m.oid[kk - 1], 0, 0, sm.u.m.oid[kk - 1], 0};
            }
        }
    } else {
        find_cut<false>(f, sm, unit, r, (double)prm.top_k, false, rv.ck, &rv.ck);
        if (threadIdx.x == 0) {
            rv.S_kept = sm.cut_mass;
            rv.n_kept = sm.cut_nin;
        }
    }
    __syncthreads();
    // nucleus
    if (!rv.has_p) {
        if (threadIdx.x == 0) {
            rv.S = rv.S_kept;
            rv.n_nuc = rv.n_kept;
        }
    } else if (small_k) {
        if (w0) {
            const int kk = prm.top_k;
            const double need = (double)prm.top_p * rv.S_kept;
            const double e = lane < kk ? mass_of(key16_value(sm.u.m.okey[lane]), rv.m, T) : 0.0;
            double ex;
            const double in = wave_scan(e, &ex);
            int i = first_lane(__ballot(lane < kk && in >= need));
            if (i < 0) i = kk - 1;
            const double cum = __shfl(in, i, kWave);
            if (lane == 0) {
                rv.cp = Cut{sm.u.m.okey[i], 0, sm.u.m.oid[i], 0, 0, sm.u.m.oid[i], 0};
                rv.S = cum;
                rv.n_nuc = i + 1;
            }
        }
    } else {
        const Cut lim = rv.ck;
        const bool use_lim = rv.has_k && lim.key != 0;
        find_cut<true>(f, sm, unit, r, (double)prm.top_p * rv.S_kept, use_lim, lim, &rv.cp);
        if (threadIdx.x == 0) {
            rv.S = sm.cut_w;
            rv.n_nuc = sm.cut_nin;
        }
    }
    __syncthreads();
    // downweighted set: the first F elements of the processed order that carry mass
    if (want_set) {
        if (w0) {
            const int n0 = min(min(a.F, rv.n_nuc), nm);
            const double e = lane < n0 ? mass_of(key16_value(sm.u.m.okey[lane]), rv.m, T) : 0.0;
            const int n = last_lane(__ballot(lane < n0 && e > 0.0)) + 1;
            const double ps = wave_sum(lane < n ? e / rv.S : 0.0);
            if (lane == 0) {
                rv.nset = n;
                if (n > 0) {
                    rv.kF = sm.u.m.okey[n - 1];
                    rv.idF = sm.u.m.oid[n - 1];
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
        __syncthreads();
    }
}

// Processed probability of token s in row r (after the combine; wave-level).
__device__ __forceinline__ double prob_of_s(const FastArgs& f, Smem& sm, int unit, int r, int s, bool draft) {
    const RowView& rv = sm.rv[r];
    const uint32_t h = sm.s_bits[r];
    if ((h & 0x7FFFu) >= 0x7F80u) return 0.0;
    const uint32_t key = key16(h);
    if (rv.has_k && !cut_keeps_s(f, unit, r, rv.ck, key, s)) return 0.0;
    if (rv.has_p && !cut_keeps_s(f, unit, r, rv.cp, key, s)) return 0.0;
    const double e = mass_of(__uint_as_float(h << 16), rv.m, rv.T);
    const double p = e / rv.S;
    if (!draft) return p;
    const double fct = (rv.nset > 0 && e > 0.0 && in_cut_id(rv.kF, rv.idF, key, s)) ? rv.C : 1.0;
    return (p * fct) / rv.Z;
}

// ------------------------------------------------------------------------------------------
// Number of leading candidates each slice lists for a row (identical in phase A and combine)
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ int list_len(const VerifyArgs& a, const spec_params& prm, bool draft) {
    const bool greedy = prm.temperature == 0.0f;
    int want = greedy ? 1 : 0;
    if (!greedy && prm.top_k > 0 && prm.top_k < a.V && prm.top_k <= kTop) want = max(want, prm.top_k);
    if (!greedy && draft && a.F > 0 && a.C < 1.0f) want = max(want, a.F);
    return want;
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
// Placement: request b runs on XCD b % 8 (workgroup index modulo 8 picks the XCD); its
// (K + 1) units x nS slices follow in order.  Both kernels use the same map, so a slice's
// summary is written and read through one L2.
// ------------------------------------------------------------------------------------------
struct Place {
    int b, j, slice, unit, per_req;
};
__device__ __forceinline__ Place place_of(const FastArgs& f) {
    Place p;
    const int x = blockIdx.x % kXcd;
    const int l = blockIdx.x / kXcd;
    p.per_req = (f.a.K + 1) * f.nS;
    p.b = (l / p.per_req) * kXcd + x;
    p.j = (l / f.nS) % (f.a.K + 1);
    p.slice = l % f.nS;
    p.unit = p.b * (f.a.K + 1) + p.j;
    return p;
}

__device__ __forceinline__ bool params_ok(const spec_params& prm) {
    return prm.temperature >= 0.0f && !isinf(prm.temperature) && prm.top_p > 0.0f;
}

// Columns [c0, c0 + kSliceCols) of a row, 16 bytes per load (zero past the row's end).
__device__ __forceinline__ void load_slice(const uint16_t* row, int c0, int V, u32x4 (&v)[kLoads]) {
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
        const int col = col_of(c0, q, 0);
        v[q] = col < V ? *reinterpret_cast<const u32x4*>(row + col) : u32x4{0, 0, 0, 0};
    }
}

// ------------------------------------------------------------------------------------------
// Count kernel: every slice of every unit loads its columns, counts them and publishes its
// summaries (no waiting on other workgroups).
// ------------------------------------------------------------------------------------------
struct CountSmem {
    double segm[kSegs];
    uint32_t segc[2][kSegs];
    union {
        uint32_t hist[2][kBins];
    } u;
    uint32_t sp_key[2][kSpecial];
    int32_t sp_id[2][kSpecial];
    uint32_t n_sp[2];
    uint32_t top_key[2][kTop];
    int32_t top_id[2][kTop];
    uint32_t n_top[2];
    uint32_t rank_s[2];
    uint32_t flags[2];
    uint32_t neginf[2];
    int32_t scan[kWaves + 1];
    double redd[kWaves];
    int32_t redi[kWaves];
    uint32_t s_bits[2];
    uint32_t tau;
    int need;
};

// Per-segment element counts of row r into sm.segc[r]: one wave per group of 64 bins, the
// last wave also sorts the specials into their four segments.  (Callers synchronise.)
__device__ __forceinline__ void seg_counts(CountSmem& sm, int r) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
#pragma unroll 1
    for (int g = wave; g < kGroups; g += kWaves) {
        const uint32_t cs = wave_sum(sm.u.hist[r][g * kGroup + lane]);
        if (lane == 0) sm.segc[r][seg_of_group(g)] = cs;
    }
    if (wave == kWaves - 1) {
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

// Wave 0: the key of the L-th element (token order) of row r in this slice, and how many
// elements at that key are taken, into sm.tau / sm.need; (0, 0) when the slice holds fewer
// than L finite elements.  Scans the segment counts, then the 64 bins of the crossing group,
// or the specials of the crossing segment.
__device__ __forceinline__ void local_threshold(CountSmem& sm, int r, int L) {
    const int lane = threadIdx.x & (kWave - 1);
    if (lane == 0) {
        sm.tau = 0u;
        sm.need = 0;
    }
    const int c = lane < kSegs ? (int)sm.segc[r][lane] : 0;
    int cex;
    const int cin = wave_scan(c, &cex);
    const uint64_t hit = __ballot(lane < kSegs && cin >= L);
    if (hit == 0) return;
    const int sg = first_lane(hit);
    const int rem = L - __shfl(cex, sg, kWave);
    const int g = group_of_seg(sg);
    if (g >= 0) {
        const int bin = bin_of_sel(g, lane);  // lane order = descending key
        const int n = (int)sm.u.hist[r][bin];
        int nex;
        const int nin = wave_scan(n, &nex);
        const int i = first_lane(__ballot(nin >= rem));
        if (lane == i) {
            sm.tau = bin_key(bin);
            sm.need = rem - nex;
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
    // every element strictly above tau (fewer than L of them), any order
    uint32_t tiemask = 0;
#pragma unroll
    for (int q = 0; q < kLoads; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int col = col_of(c0, q, e);
            const uint32_t w = v[q][e >> 1];
            const uint32_t h = (e & 1) ? (w >> 16) : (w & 0xFFFFu);
            if (col >= V || (h & 0x7FFFu) >= 0x7F80u) continue;  // past the row, inf, NaN
            const uint32_t k = key16(h);
            if (k > tau) {
                const int slot = (int)atomicAdd(&sm.n_top[r], 1u);
                if (slot < kTop) {
                    sm.top_key[r][slot] = k;
                    sm.top_id[r][slot] = col;
                }
            } else if (k == tau && need > 0) {
                tiemask |= 1u << (q * 8 + e);
            }
        }
    __syncthreads();
    int base = min((int)sm.n_top[r], kTop);
    int need_left = need;
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

// Rank of the draft token among the elements of row r with its key that precede it in this
// slice (the slice holding the token only), into sm.rank_s[r].
__device__ __forceinline__ void local_rank(CountSmem& sm, int r, int c0, int s_tok, const u32x4 (&v)[kLoads]) {
    const uint32_t ks = key16(sm.s_bits[r]);
    uint32_t rank = 0;
#pragma unroll
    for (int q = 0; q < kLoads; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int col = col_of(c0, q, e);
            const uint32_t w = v[q][e >> 1];
            const uint32_t h = (e & 1) ? (w >> 16) : (w & 0xFFFFu);
            rank += (col < s_tok && (h & 0x7FFFu) < 0x7F80u && key16(h) == ks) ? 1u : 0u;
        }
    rank = block_sum<uint32_t>(rank, reinterpret_cast<uint32_t*>(sm.redi));
    if (threadIdx.x == 0) sm.rank_s[r] = rank;
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
    // largest key: highest non-empty bin or special
    uint32_t mk = 0;
#pragma unroll 1
    for (int b = threadIdx.x; b < kBins; b += blockDim.x)
        if (sm.u.hist[r][b] != 0) mk = max(mk, bin_key(b));
    if ((int)threadIdx.x < nsp) mk = max(mk, sm.sp_key[r][threadIdx.x]);
    mk = block_max<uint32_t>(mk, reinterpret_cast<uint32_t*>(sm.redi));
    const float m = mk ? key16_value(mk) : -__builtin_inff();
    // per-group masses (relative to this slice's largest logit), one wave per group
#pragma unroll 1
    for (int g = wave; g < kGroups; g += kWaves) {
        const int bin = g * kGroup + lane;
        const uint32_t c = sm.u.hist[r][bin];
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
            P->maxkey = mk;
            P->flags = (sm.flags[r] & 1u) | ((int)sm.n_sp[r] > kSpecial ? 2u : 0u);
            P->n_neginf = sm.neginf[r];
            P->n_finite = nfin;
            P->n_special = (uint32_t)nsp;
            P->S = S;
            P->rank_s = sm.rank_s[r];
            P->n_top = sm.n_top[r];
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
        fine32[i] = (sm.u.hist[r][2 * i] & 0xFFFFu) | (sm.u.hist[r][2 * i + 1] << 16);
    __syncthreads();  // segm is reused by the next row
}

// Counts this thread's columns of row r into sm.u.hist[r].  Values in the exact bins take
// the straight path; the rest (zero, specials, -inf, +inf, NaN) are marked in a bit mask and
// handled in a second, normally empty, loop.  TAIL: the slice ends inside the row.
template <bool TAIL>
__device__ __forceinline__ void count_row(CountSmem& sm, int r, int c0, int V, const u32x4 (&v)[kLoads]) {
    uint32_t rare = 0;
#pragma unroll
    for (int q = 0; q < kLoads; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t w = v[q][e >> 1];
            const uint32_t h = (e & 1) ? (w >> 16) : (w & 0xFFFFu);
            const uint32_t off = (h & 0x7FFFu) - (uint32_t)(kExpLo << 7);
            const bool in = off < (uint32_t)kNegBins && (!TAIL || col_of(c0, q, e) < V);
            if (in) atomicAdd(&sm.u.hist[r][(h & 0x8000u) ? (kNegBins - 1 - (int)off) : (kPosBase + (int)off)], 1u);
            else if (!TAIL || col_of(c0, q, e) < V) rare |= 1u << (q * 8 + e);
        }
    uint32_t bad = 0, ninf = 0;
    while (rare) {
        const int i = __builtin_ctz(rare);
        rare &= rare - 1;
        const int q = i >> 3, e = i & 7;
        const uint32_t w = v[q][e >> 1];
        const uint32_t h = (e & 1) ? (w >> 16) : (w & 0xFFFFu);
        int bin;
        const int kind = classify(h, &bin);
        if (kind == kKindBin) {
            atomicAdd(&sm.u.hist[r][bin], 1u);
        } else if (kind == kKindSpecial) {
            const uint32_t slot = atomicAdd(&sm.n_sp[r], 1u);
            if (slot < (uint32_t)kSpecial) {
                sm.sp_key[r][slot] = key16(h);
                sm.sp_id[r][slot] = col_of(c0, q, e);
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
    for (int i = threadIdx.x; i < 2 * kBins; i += blockDim.x) (&sm.u.hist[0][0])[i] = 0u;
    if (threadIdx.x < 2) {
        sm.n_sp[threadIdx.x] = 0;
        sm.flags[threadIdx.x] = 0;
        sm.neginf[threadIdx.x] = 0;
        sm.s_bits[threadIdx.x] = 0;
    }
    // the draft token's bits, needed for its rank by the slice that holds it
    if (threadIdx.x == kWave && two && tok_ok && s_tok / kSliceCols == slice) {
        sm.s_bits[0] = trow[s_tok];
        sm.s_bits[1] = drow[s_tok];
    }
    __syncthreads();
    const int ncols = min(kSliceCols, a.V - c0);
    if (ncols == kSliceCols) {
        count_row<false>(sm, 0, c0, a.V, vq);
        if (two) count_row<false>(sm, 1, c0, a.V, vp);
    } else {
        count_row<true>(sm, 0, c0, a.V, vq);
        if (two) count_row<true>(sm, 1, c0, a.V, vp);
    }
    if (threadIdx.x < 2) {
        sm.n_top[threadIdx.x] = 0;
        sm.rank_s[threadIdx.x] = 0;
    }
    __syncthreads();
    seg_counts(sm, 0);
    if (two) seg_counts(sm, 1);
    __syncthreads();
    // passes over the columns (registers) first, so the columns are dead for the summaries
    const bool holds_s = two && tok_ok && s_tok / kSliceCols == slice;
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

    if (threadIdx.x < 2) sm.s_bits[threadIdx.x] = 0;
    __syncthreads();
    if (threadIdx.x == kWave && two && tok_ok) {  // a lane outside wave 0, which loads the headers
        sm.s_bits[0] = trow[s_tok];
        sm.s_bits[1] = drow[s_tok];
    }

    uint32_t status = 0;
    int accept = 0;
    bool need_resid = false;
    bool fb_unit = false;
    if (!param_ok) {
        status = kStBadParam;
    } else {
        combine_row(f, sm, unit, 0, prm, false);
        if (two) combine_row(f, sm, unit, 1, prm, true);
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
                    const double ps = prob_of_s(f, sm, unit, 1, s_tok, true);
                    const double qs = prob_of_s(f, sm, unit, 0, s_tok, false);
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

// ------------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------------
FastPlan fast_plan(int B, int K, int V) {
    FastPlan p;
    p.nS = (V + kSliceCols - 1) / kSliceCols;
    p.units = B * (K + 1);
    const int reqs_per_xcd = (B + kXcd - 1) / kXcd;
    p.grid = kXcd * reqs_per_xcd * (K + 1) * p.nS;
    p.ws_bytes = layout(B, p.units, p.nS).total;
    return p;
}

bool fast_path_applies(const VerifyArgs& a) {
    if (a.dtype != SPEC_BF16 || (a.flags & SPEC_SAMPLE_DRAFT)) return false;
    if (a.V % 8 != 0 || a.V < 2048) return false;
    if ((reinterpret_cast<uintptr_t>(a.draft) & 15) || (reinterpret_cast<uintptr_t>(a.target) & 15)) return false;
    const int nS = (a.V + kSliceCols - 1) / kSliceCols;
    return nS * kTop <= kMergeCap;  // every slice's candidate list fits the merge buffer
}

int fast_verify(const VerifyArgs& a, void* ws, size_t ws_bytes, hipStream_t stream) {
    const FastPlan p = fast_plan(a.B, a.K, a.V);
    if (ws_bytes < p.ws_bytes) return SPEC_EWORKSPACE;
    FastArgs f;
    f.a = a;
    f.nS = p.nS;
    f.units = p.units;
    f.ws = static_cast<char*>(ws);
    f.L = layout(a.B, p.units, p.nS);
    hipLaunchKernelGGL(fast_count_kernel, dim3((unsigned)p.grid), dim3(kThreads), 0, stream, f);
    hipLaunchKernelGGL(fast_resolve_kernel, dim3((unsigned)p.grid), dim3(kThreads), 0, stream, f);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

}  // namespace fast
}  // namespace sv
