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
    size_t ctr, flag, req, parts, units, idcut, chunks, total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

__host__ __device__ inline Layout layout(int B, int units, int nS) {
    Layout L;
    size_t o = 0;
    L.ctr = o;    o += align256((size_t)units * 128);           // unit arrival counters (one line each)
    L.flag = o;   o += align256((size_t)units * 128);           // unit release flags
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
// L2-local synchronisation between the slices of a unit (all on one XCD)
// ------------------------------------------------------------------------------------------
constexpr unsigned kSpinLimit = 1u << 20;

__device__ __forceinline__ unsigned l2_fetch_add(unsigned* p, unsigned v) {
    unsigned old;
    asm volatile("s_waitcnt vmcnt(0)\n\tglobal_atomic_add %0, %1, %2, off sc0\n\ts_waitcnt vmcnt(0)"
                 : "=v"(old) : "v"(p), "v"(v) : "memory");
    return old;
}
__device__ __forceinline__ void l2_store_add(unsigned* p, unsigned v) {
    asm volatile("s_waitcnt vmcnt(0)\n\tglobal_atomic_add %0, %1, off\n\ts_waitcnt vmcnt(0)" :: "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ unsigned l2_read(unsigned* p) { return l2_fetch_add(p, 0u); }

// Every slice of the unit arrives; the last one raises the unit's flag; the others poll it.
// Returns false when the wait gave up (the unit's results are then flagged).  Data published
// before the barrier is read after it with non-temporal loads (ldnt), which bypass the CU's
// vector L1 and are served by the shared L2; a plain load could return a stale L1 line.
// Every wave waits until its own global stores have reached L2; __syncthreads() alone orders
// only LDS traffic, so this must precede the workgroup barrier in front of an arrival.
__device__ __forceinline__ void drain_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ bool unit_barrier(unsigned* ctr, unsigned* flag, int nS) {
    __shared__ int ok;
    drain_stores();
    __syncthreads();
    if (threadIdx.x == 0) {
        ok = 1;
        const unsigned old = l2_fetch_add(ctr, 1u);
        if (old + 1 == (unsigned)nS) {
            l2_store_add(flag, 1u);
        } else {
            unsigned spins = 0;
            while (l2_read(flag) == 0u) {
                __builtin_amdgcn_s_sleep(2);
                if (++spins > kSpinLimit) {
                    ok = 0;
                    break;
                }
            }
        }
    }
    __syncthreads();
    return ok != 0;
}


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
            uint32_t slice_cnt[32];
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
    uint32_t maxbin[2];
    int32_t scan[kWaves + 1];
    double redd[kWaves];
    int32_t redi[kWaves];
    RowView rv[2];
    uint32_t key_s[2];
    float z_s[2];
    uint32_t s_bits[2];   // bf16 bits of token s in each row
    int last;
    int found;
    uint32_t cnt_tmp;
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
// Thread 0: walks this slice's row r from the largest key down over the exact bins (hist[r])
// and the specials, until `L` elements are counted; returns the key of the L-th element and how
// many elements at that key are needed (0 when the row holds fewer than L finite elements).
__device__ __forceinline__ void local_threshold(Smem& sm, int r, int L, uint32_t* tau_out, int* need_out) {
    int cum = 0;
    for (int sg = 0; sg < kSegs; ++sg) {
        const int g = group_of_seg(sg);
        if (g >= 0) {
            for (int bb = kGroup - 1; bb >= 0; --bb) {
                const int bin = g * kGroup + bb;
                const int c = (int)sm.u.hist[r][bin];
                if (c == 0) continue;
                if (cum + c >= L) {
                    *tau_out = bin_key(bin);
                    *need_out = L - cum;
                    return;
                }
                cum += c;
            }
        } else {
            const int n = min((int)sm.n_sp[r], kSpecial);
            uint32_t prev = 0xFFFFFFFFu;  // walk this segment's distinct keys downwards
            while (true) {
                uint32_t best = 0;
                int c = 0;
                for (int i = 0; i < n; ++i) {
                    const uint32_t k = sm.sp_key[r][i];
                    if (special_seg(k) != sg || k >= prev) continue;
                    if (c == 0 || k > best) {
                        best = k;
                        c = 1;
                    } else if (k == best) {
                        ++c;
                    }
                }
                if (c == 0) break;
                if (cum + c >= L) {
                    *tau_out = best;
                    *need_out = L - cum;
                    return;
                }
                cum += c;
                prev = best;
            }
        }
    }
    *tau_out = 0;
    *need_out = 0;
}

// The first L elements (token order: key desc, id asc) of row r in this slice, sorted, into
// sm.top_key / sm.top_id; sm.n_top gets their number.  v holds the slice's columns of row r.
__device__ __forceinline__ void local_top(Smem& sm, int r, int L, int c0, int V, const u32x4 (&v)[kLoads]) {
    __shared__ uint32_t s_tau;
    __shared__ int s_need;
    if (threadIdx.x == 0) {
        local_threshold(sm, r, L, &s_tau, &s_need);
        sm.n_top = 0;
    }
    __syncthreads();
    const uint32_t tau = s_tau;
    const int need = s_need;
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
                const int slot = (int)atomicAdd(&sm.n_top, 1u);
                if (slot < kTop) {
                    sm.top_key[slot] = k;
                    sm.top_id[slot] = col;
                }
            } else if (k == tau && need > 0) {
                tiemask |= 1u << (q * 8 + e);
            }
        }
    __syncthreads();
    int base = min((int)sm.n_top, kTop);
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
                sm.top_key[slot] = tau;
                sm.top_id[slot] = col_of(c0, q, e);
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
        mk = sm.top_key[threadIdx.x];
        mi = sm.top_id[threadIdx.x];
        for (int i = 0; i < n; ++i) {
            const uint32_t k2 = sm.top_key[i];
            const int i2 = sm.top_id[i];
            rank += (k2 > mk || (k2 == mk && i2 < mi)) ? 1 : 0;
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < n) {
        sm.top_key[rank] = mk;
        sm.top_id[rank] = mi;
    }
    if (threadIdx.x == 0) sm.n_top = (uint32_t)n;
    __syncthreads();
}

// ------------------------------------------------------------------------------------------
// Phase C: combining the slices' summaries of one row (every slice computes the same view)
// ------------------------------------------------------------------------------------------
// Merged candidates of the unit's slices for row r, sorted (key desc, id asc); returns their
// number (<= kMergeCap).  Source: each slice's top list.
__device__ __forceinline__ int merge_tops(const FastArgs& f, Smem& sm, int unit, int r, int want) {
    // gather
    int n = 0;
    for (int t = 0; t < f.nS; ++t) {
        const RowPart* P = part_of(f, unit, t, r);
        const int nt = (int)ldnt(&P->n_top);
        for (int i = threadIdx.x; i < nt; i += blockDim.x) {
            if (n + i < kMergeCap) {
                sm.u.m.key[n + i] = ldnt(&P->top_key[i]);
                sm.u.m.id[n + i] = ldnt(&P->top_id[i]);
            }
        }
        n += nt;
    }
    n = min(n, kMergeCap);
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

// Fine counts of group g of row r summed over the slices into sm.u.m.fine[64].
__device__ __forceinline__ void merge_fine(const FastArgs& f, Smem& sm, int unit, int r, int g) {
    if (threadIdx.x < kGroup) {
        uint32_t c = 0;
        for (int t = 0; t < f.nS; ++t) c += ldnt_u16(&part_of(f, unit, t, r)->fine[g * kGroup + threadIdx.x]);
        sm.u.m.fine[threadIdx.x] = c;
    }
    __syncthreads();
}

// Slice owning the take-th element at bin `bin` of row r (in token order), and how many of
// that bin's elements it holds before it; fills c.owner and c.owner_take.
__device__ __forceinline__ void tie_owner(const FastArgs& f, int unit, int r, int bin, Cut& c) {
    int acc = 0;
    c.owner = f.nS - 1;
    c.owner_take = 0;
    for (int t = 0; t < f.nS; ++t) {
        const int n = (int)ldnt_u16(&part_of(f, unit, t, r)->fine[bin]);
        if (acc + n >= c.take) {
            c.owner = t;
            c.owner_take = c.take - acc;
            return;
        }
        acc += n;
    }
}

// Finds the cut where the running weight over the row, walked from the largest key down,
// first reaches `need`.  Weights are counts (MASS false) or masses cnt * e (MASS true);
// elements are restricted to the `lim` cut when given (nucleus inside a top-k set).
// Thread 0 computes; the result is broadcast through sm.rv[r].  Returns the weight above the
// cut plus that of the taken elements (the kept mass for MASS).
template <bool MASS>
__device__ __forceinline__ double find_cut(const FastArgs& f, Smem& sm, int unit, int r, double need, const Cut* lim, Cut* out,
                           int* n_in_out) {
    RowView& rv = sm.rv[r];
    __shared__ int s_seg;
    __shared__ double s_above;
    __shared__ int s_cnt_above;
    // 1. crossing segment (segments below the limit's segment weigh nothing; the limit's own
    //    segment is resolved exactly below)
    if (threadIdx.x == 0) {
        double acc = 0.0;
        int cnt = 0;
        int pick = kSegs - 1;
        const int lim_seg = lim ? (key_is_binned(lim->key) ? seg_of_group(key_bin(lim->key) / kGroup) : special_seg(lim->key)) : kSegs;
        // (callers pass no limit for a cut that keeps everything)
        double acc_before = 0.0;
        int cnt_before = 0;
        bool crossed = false;
        for (int sg = 0; sg < kSegs; ++sg) {
            if (sg >= lim_seg) {
                pick = sg;
                acc_before = acc;
                cnt_before = cnt;
                crossed = true;
                break;
            }
            const double w = MASS ? rv.seg_mass[sg] : (double)rv.seg_count[sg];
            if (rv.seg_count[sg] == 0) continue;
            if (acc + w >= need) {
                pick = sg;
                acc_before = acc;
                cnt_before = cnt;
                crossed = true;
                break;
            }
            // rounding may leave the target beyond the last segment: remember this one
            pick = sg;
            acc_before = acc;
            cnt_before = cnt;
            acc += w;
            cnt += (int)rv.seg_count[sg];
        }
        (void)crossed;
        s_seg = pick;
        s_above = acc_before;
        s_cnt_above = cnt_before;
    }
    __syncthreads();
    const int sg = s_seg;
    const int g = group_of_seg(sg);
    double above = s_above;
    int cnt_above = s_cnt_above;
    __shared__ double s_res;
    __shared__ int s_nin;
    if (g >= 0) {
        merge_fine(f, sm, unit, r, g);
        if (threadIdx.x == 0) {
            Cut c;
            c.explicit_id = -1;
            c.key = 0;
            c.take = 0;
            bool done = false;
            double kept_w = above;
            int last_bin = -1, last_n = 0;
            double last_e = 0.0;
            for (int bb = kGroup - 1; bb >= 0 && !done; --bb) {
                const int bin = g * kGroup + bb;
                int n = (int)sm.u.m.fine[bb];
                if (n == 0) continue;
                const uint32_t key = bin_key(bin);
                if (lim) {
                    if (key < lim->key) break;
                    if (key == lim->key) n = min(n, lim->take);
                }
                const double e = MASS ? mass_of(key16_value(key), rv.m, rv.T) : 1.0;
                const double w = (double)n * e;
                if (above + w >= need || (lim && key == lim->key)) {
                    int take = n;
                    if (MASS) {
                        if (e > 0.0) {
                            const double q = ceil((need - above) / e);
                            take = q < 1.0 ? 1 : (q > (double)n ? n : (int)q);
                        }
                    } else {
                        take = (int)(need - above);
                        take = take < 1 ? 1 : (take > n ? n : take);
                    }
                    if (above + w < need) take = n;  // the limit ends the walk first
                    c.key = key;
                    c.take = take;
                    c.count_above = cnt_above;
                    kept_w = above + (double)take * e;
                    done = true;
                } else {
                    above += w;
                    cnt_above += n;
                    last_bin = bin;
                    last_n = n;
                    last_e = e;
                }
            }
            if (!done) {  // rounding left the target just beyond the group: cut at its lowest bin
                if (last_bin >= 0) {
                    above -= (double)last_n * last_e;
                    cnt_above -= last_n;
                    c.key = bin_key(last_bin);
                    c.take = last_n;
                } else {
                    c.key = 0;
                    c.take = 0;
                }
                c.count_above = cnt_above;
                kept_w = above + (double)last_n * last_e;
            }
            *out = c;
            s_res = kept_w;
            s_nin = cnt_above + c.take;
        }
        __syncthreads();
        if (out->key != 0 && out->explicit_id < 0) {
            if (threadIdx.x == 0) tie_owner(f, unit, r, key_bin(out->key), *out);
            __syncthreads();
        }
    } else {
        const int n = merge_specials(f, sm, unit, r, sg);
        if (threadIdx.x == 0) {
            Cut c;
            c.key = 0;
            c.take = 0;
            c.explicit_id = -1;
            c.owner = 0;
            c.owner_take = 0;
            double kept_w = above;
            int i = 0;
            for (; i < n; ++i) {
                const uint32_t key = sm.u.m.key[i];
                if (lim && (key < lim->key || (key == lim->key && lim->explicit_id >= 0 && sm.u.m.id[i] > lim->explicit_id))) break;
                const double w = MASS ? mass_of(key16_value(key), rv.m, rv.T) : 1.0;
                above += w;
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
            c.count_above = cnt_above;
            kept_w = above;
            *out = c;
            s_res = kept_w;
            s_nin = cnt_above + i;
        }
        __syncthreads();
    }
    const double res = s_res;
    if (n_in_out) *n_in_out = s_nin;
    __syncthreads();
    return res;
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

// Global rank (0-based, token order) of token s among the elements of row r with key == key_s.
__device__ __forceinline__ int global_rank_s(const FastArgs& f, int unit, int r, uint32_t key_s, int s) {
    const int owner = s / kSliceCols;
    int acc = 0;
    if (key_is_binned(key_s)) {
        const int bin = key_bin(key_s);
        for (int t = 0; t < owner && t < f.nS; ++t) acc += (int)ldnt_u16(&part_of(f, unit, t, r)->fine[bin]);
    } else {
        for (int t = 0; t < owner && t < f.nS; ++t) {
            const RowPart* P = part_of(f, unit, t, r);
            const int ns = min((int)ldnt(&P->n_special), kSpecial);
            for (int i = 0; i < ns; ++i) acc += (ldnt(&P->sp_key[i]) == key_s) ? 1 : 0;
        }
    }
    return acc + (int)ldnt(&part_of(f, unit, owner, r)->rank_s);
}

__device__ __forceinline__ bool cut_keeps_s(const FastArgs& f, int unit, int r, const Cut& c, uint32_t key_s, int s) {
    if (key_s > c.key) return true;
    if (key_s < c.key) return false;
    if (c.explicit_id >= 0) return s <= c.explicit_id;
    return global_rank_s(f, unit, r, key_s, s) < c.take;
}

// ------------------------------------------------------------------------------------------
// Combine one row (all threads)
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void combine_row(const FastArgs& f, Smem& sm, int unit, int r, const spec_params& prm, bool draft) {
    RowView& rv = sm.rv[r];
    const VerifyArgs& a = f.a;
    const double T = (double)prm.temperature;
    if (threadIdx.x == 0) {
        float m = -__builtin_inff();
        uint32_t fl = 0, nfin = 0;
        int has_sp = 0;
        for (int t = 0; t < f.nS; ++t) {
            const RowPart* P = part_of(f, unit, t, r);
            const float mt = ldnt(&P->m);
            fl |= ldnt(&P->flags);
            nfin += ldnt(&P->n_finite);
            has_sp |= ldnt(&P->n_special) > 0 ? 1 : 0;
            m = mt > m ? mt : m;
        }
        rv.m = m;
        rv.T = T;
        rv.bad = ((fl & 1u) || nfin == 0) ? 1 : 0;
        rv.overflow = (fl & 2u) ? 1 : 0;
        rv.n_finite = nfin;
        rv.greedy = prm.temperature == 0.0f ? 1 : 0;
        rv.has_special = has_sp;
        rv.argmax = -1;
        double S = 0.0;
        for (int t = 0; t < f.nS && t < 32; ++t) {
            const RowPart* P = part_of(f, unit, t, r);
            const float mt = ldnt(&P->m);
            rv.sc[t] = (T > 0.0 && mt > -__builtin_inff()) ? exp(((double)mt - (double)m) / T) : 0.0;
            S += rv.sc[t] * ldnt(&P->S);
        }
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
        if (threadIdx.x == 0) rv.overflow = 1;
        __syncthreads();
        return;
    }
    // merged segment weights
    for (int sg = threadIdx.x; sg < kSegs; sg += blockDim.x) {
        double ms = 0.0;
        uint32_t cs = 0;
        for (int t = 0; t < f.nS && t < 32; ++t) {
            const RowPart* P = part_of(f, unit, t, r);
            ms += rv.sc[t] * ldnt(&P->seg_mass[sg]);
            cs += ldnt(&P->seg_count[sg]);
        }
        rv.seg_mass[sg] = ms;
        rv.seg_count[sg] = cs;
    }
    __syncthreads();
    // top-k
    if (!rv.has_k) {
        if (threadIdx.x == 0) {
            rv.S_kept = rv.S_all;
            rv.n_kept = (int)rv.n_finite;
        }
        __syncthreads();
    } else if (small_k) {
        if (threadIdx.x == 0) {
            double s = 0.0;
            for (int i = 0; i < prm.top_k; ++i) s += mass_of(key16_value(sm.u.m.okey[i]), rv.m, T);
            rv.S_kept = s;
            rv.n_kept = prm.top_k;
            rv.ck = Cut{sm.u.m.okey[prm.top_k - 1], 0, sm.u.m.oid[prm.top_k - 1], 0, 0, sm.u.m.oid[prm.top_k - 1], 0};
        }
        __syncthreads();
    } else {
        Cut c;
        int nin = 0;
        find_cut<false>(f, sm, unit, r, (double)prm.top_k, nullptr, &sm.rv[r].ck, &nin);
        // kept mass: segments above the cut plus the taken part of the cut's bin / specials
        __syncthreads();
        if (threadIdx.x == 0) {
            c = rv.ck;
            double s = 0.0;
            const int cut_seg = key_is_binned(c.key) ? seg_of_group(key_bin(c.key) / kGroup) : special_seg(c.key);
            for (int sg = 0; sg < cut_seg; ++sg) s += rv.seg_mass[sg];
            rv.S_kept = s;  // completed below with the cut segment's kept part
            rv.n_kept = nin;
        }
        __syncthreads();
        // the cut segment's kept mass
        {
            const Cut c2 = rv.ck;
            if (key_is_binned(c2.key)) {
                const int g = key_bin(c2.key) / kGroup;
                merge_fine(f, sm, unit, r, g);
                if (threadIdx.x == 0) {
                    double s = 0.0;
                    for (int bb = kGroup - 1; bb >= 0; --bb) {
                        const int bin = g * kGroup + bb;
                        const uint32_t key = bin_key(bin);
                        const int n = (int)sm.u.m.fine[bb];
                        if (n == 0 || key < c2.key) continue;
                        const int take = key == c2.key ? c2.take : n;
                        s += (double)take * mass_of(key16_value(key), rv.m, T);
                    }
                    rv.S_kept += s;
                }
            } else {
                const int n = merge_specials(f, sm, unit, r, special_seg(c2.key));
                if (threadIdx.x == 0) {
                    double s = 0.0;
                    for (int i = 0; i < n; ++i) {
                        const uint32_t key = sm.u.m.key[i];
                        if (key < c2.key || (key == c2.key && sm.u.m.id[i] > c2.explicit_id)) break;
                        s += mass_of(key16_value(key), rv.m, T);
                    }
                    rv.S_kept += s;
                }
            }
            __syncthreads();
        }
    }
    // nucleus
    if (!rv.has_p) {
        if (threadIdx.x == 0) {
            rv.S = rv.S_kept;
            rv.n_nuc = rv.n_kept;
        }
        __syncthreads();
    } else if (small_k) {
        if (threadIdx.x == 0) {
            const double need = (double)prm.top_p * rv.S_kept;
            double cum = 0.0;
            int i = 0;
            for (; i < prm.top_k; ++i) {
                cum += mass_of(key16_value(sm.u.m.okey[i]), rv.m, T);
                if (cum >= need) break;
            }
            if (i >= prm.top_k) i = prm.top_k - 1;
            rv.cp = Cut{sm.u.m.okey[i], 0, sm.u.m.oid[i], 0, 0, sm.u.m.oid[i], 0};
            rv.S = cum;
            rv.n_nuc = i + 1;
        }
        __syncthreads();
    } else {
        int nin = 0;
        const Cut lim = rv.ck;
        const bool use_lim = rv.has_k && lim.key != 0;
        const double kept = find_cut<true>(f, sm, unit, r, (double)prm.top_p * rv.S_kept, use_lim ? &lim : nullptr,
                                           &sm.rv[r].cp, &nin);
        if (threadIdx.x == 0) {
            rv.S = kept;
            rv.n_nuc = nin;
        }
        __syncthreads();
    }
    // downweighted set: the first F elements of the processed order that carry mass
    if (want_set) {
        if (threadIdx.x == 0) {
            int n = min(min(a.F, rv.n_nuc), nm);
            while (n > 0 && !(mass_of(key16_value(sm.u.m.okey[n - 1]), rv.m, T) > 0.0)) --n;
            rv.nset = n;
            if (n > 0) {
                rv.kF = sm.u.m.okey[n - 1];
                rv.idF = sm.u.m.oid[n - 1];
                double ps = 0.0;
                for (int i = 0; i < n; ++i) ps += mass_of(key16_value(sm.u.m.okey[i]), rv.m, T) / rv.S;
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
        __syncthreads();
    }
}

// Processed probability of token s in row r (after the combine).
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

// Phase A for row r: counts are in sm.u.hist[r]; publishes the slice summary.
__device__ __forceinline__ void publish_row(const FastArgs& f, Smem& sm, int unit, int slice, int r, const spec_params& prm, bool draft,
                            int c0, const u32x4 (&v)[kLoads], int s_tok) {
    const VerifyArgs& a = f.a;
    RowPart* P = part_of(f, unit, slice, r);
    const double T = (double)prm.temperature;
    const int nsp = min((int)sm.n_sp[r], kSpecial);
    // largest key: highest non-empty bin or special
    uint32_t mk = 0;
    for (int b = threadIdx.x; b < kBins; b += blockDim.x)
        if (sm.u.hist[r][b] != 0) mk = max(mk, bin_key(b));
    for (int i = threadIdx.x; i < nsp; i += blockDim.x) mk = max(mk, sm.sp_key[r][i]);
    mk = block_max<uint32_t>(mk, reinterpret_cast<uint32_t*>(sm.redi));
    const float m = mk ? key16_value(mk) : -__builtin_inff();
    // per-group counts and masses (relative to this slice's largest logit)
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    for (int g = wave; g < kGroups; g += kWaves) {
        const int bin = g * kGroup + lane;
        const uint32_t c = sm.u.hist[r][bin];
        double ms = 0.0;
        if (c != 0 && T > 0.0) ms = (double)c * mass_of(key16_value(bin_key(bin)), m, T);
        ms = wave_sum(ms);
        const uint32_t cs = wave_sum(c);
        if (lane == 0) {
            const int sg = seg_of_group(g);
            sm.segm[sg] = ms;
            sm.segc[sg] = cs;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int sps[4] = {kSegHugePos, kSegTinyPos, kSegTinyNeg, kSegHugeNeg};
        for (int x = 0; x < 4; ++x) {
            sm.segm[sps[x]] = 0.0;
            sm.segc[sps[x]] = 0;
        }
        for (int i = 0; i < nsp; ++i) {
            const uint32_t k = sm.sp_key[r][i];
            const int sg = special_seg(k);
            if (T > 0.0) sm.segm[sg] += mass_of(key16_value(k), m, T);
            sm.segc[sg] += 1;
        }
        double S = 0.0;
        uint32_t nfin = 0;
        for (int sg = 0; sg < kSegs; ++sg) {
            S += sm.segm[sg];
            nfin += sm.segc[sg];
        }
        P->m = m;
        P->maxkey = mk;
        P->flags = (sm.flags[r] & 1u) | ((int)sm.n_sp[r] > kSpecial ? 2u : 0u);
        P->n_neginf = sm.neginf[r];
        P->n_finite = nfin;
        P->n_special = (uint32_t)nsp;
        P->S = S;
    }
    for (int sg = threadIdx.x; sg < kSegs; sg += blockDim.x) {
        P->seg_mass[sg] = sm.segm[sg];
        P->seg_count[sg] = sm.segc[sg];
    }
    for (int i = threadIdx.x; i < nsp; i += blockDim.x) {
        P->sp_key[i] = sm.sp_key[r][i];
        P->sp_id[i] = sm.sp_id[r][i];
    }
    // fine counts, two per dword (a slice holds < 65536 columns)
    uint32_t* fine32 = reinterpret_cast<uint32_t*>(P->fine);
    for (int i = threadIdx.x; i < kBins / 2; i += blockDim.x)
        fine32[i] = (sm.u.hist[r][2 * i] & 0xFFFFu) | (sm.u.hist[r][2 * i + 1] << 16);
    // rank of the draft token among equal keys in the slice that holds it
    uint32_t rank = 0;
    if (s_tok >= 0 && s_tok / kSliceCols == slice) {
        const uint32_t ks = key16(sm.s_bits[r]);
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
    }
    if (threadIdx.x == 0) P->rank_s = rank;
    // leading candidates
    const int want = list_len(a, prm, draft);
    if (want > 0) {
        local_top(sm, r, want, c0, a.V, v);
        for (int i = threadIdx.x; i < (int)sm.n_top; i += blockDim.x) {
            P->top_key[i] = sm.top_key[i];
            P->top_id[i] = sm.top_id[i];
        }
        if (threadIdx.x == 0) P->n_top = sm.n_top;
    } else if (threadIdx.x == 0) {
        P->n_top = 0;
    }
    __syncthreads();
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

// The general algorithm for one unit (out of line: a rare path).
__device__ __noinline__ void fallback_unit(const VerifyArgs& a, int b, int j, Smem& sm) {
    unit_verify(a, b, j, &sm.urec, sm.u.generic, sm.gst[0], sm.gst[1]);
}

// ------------------------------------------------------------------------------------------
// Finaliser: the last workgroup of a request picks k and t*
// ------------------------------------------------------------------------------------------
__device__ __noinline__ void finalize_request(const FastArgs& f, Smem& sm, int b) {
    const VerifyArgs& a = f.a;
    const int K = a.K;
    UnitFast* U = reinterpret_cast<UnitFast*>(f.ws + f.L.units);
    const int32_t* IC = reinterpret_cast<const int32_t*>(f.ws + f.L.idcut);
    __shared__ int s_k, s_t, s_mode, s_c;
    __shared__ uint32_t s_status;
    __shared__ double s_W, s_target, s_base;
    if (threadIdx.x == 0) {
        uint32_t any = 0, deg = 0;
        for (int j = 0; j <= K; ++j) {
            const uint32_t st = ldnt(&U[b * (K + 1) + j].status);
            any |= st;
            if (j < K) deg |= st & kStDegenerate;
        }
        int k = 0, mode = 0;  // mode 0: done, 1: chunk search, 2: empty residual
        uint32_t status;
        int t = -1;
        double W = 0.0;
        if (any & SPEC_ST_SYNC_TIMEOUT) {
            status = SPEC_ST_SYNC_TIMEOUT;
        } else if (any & kStBadParam) {
            status = kStBadParam;
        } else if (any & kStBadLogit) {
            status = kStBadLogit;
        } else if (any & kStBadToken) {
            status = deg | kStBadToken;
        } else {
            status = deg;
            k = K;
            for (int j = 0; j < K; ++j) {
                const UnitFast* u = &U[b * (K + 1) + j];
                status |= ldnt(&u->status) & kStOutside;
                if (!ldnt(&u->accept)) {
                    k = j;
                    break;
                }
            }
            const UnitFast* uk = &U[b * (K + 1) + k];
            if (ldnt(&uk->fallback)) {
                t = ldnt(&uk->tcand);
                W = (double)ldnt(&uk->W);
                status |= ldnt(&uk->status) & kStEmptyResidual;
            } else if (ldnt(&uk->rq.greedy)) {
                t = ldnt(&uk->rq.argmax);
            } else {
                const double* ch = reinterpret_cast<const double*>(f.ws + f.L.chunks) +
                                   (size_t)(b * (K + 1) + k) * f.nS * kChunks;
                const int n = f.nS * kChunks;
                for (int c = 0; c < n; ++c) W += ldnt(&ch[c]);
                const double v = uniform_at(a.seed, a.round, (uint64_t)b, (uint64_t)k, 1);
                const double target = v * W;
                if (W > 0.0) {
                    double cum = 0.0, base = 0.0;
                    int pick = -1;
                    for (int c = 0; c < n; ++c) {
                        const double x = ldnt(&ch[c]);
                        if (x > 0.0 && cum <= target) {
                            pick = c;
                            base = cum;
                        }
                        cum += x;
                    }
                    s_c = pick;
                    s_base = base;
                    s_target = target;
                    mode = 1;
                } else {
                    status |= kStEmptyResidual;
                    s_target = v;
                    mode = 2;
                }
            }
            if (k == K) W = 0.0;
        }
        s_k = k;
        s_t = t;
        s_W = W;
        s_status = status;
        s_mode = mode;
    }
    __syncthreads();
    const int k = s_k;
    const int mode = s_mode;
    if (mode != 0) {
        const int unit = b * (K + 1) + k;
        const UnitFast* uk = &U[unit];
        RowFinal rq, rp;
        // copy the row statistics (published by slice 0 of that unit)
        {
            const uint32_t* src = reinterpret_cast<const uint32_t*>(&uk->rq);
            uint32_t* dq = reinterpret_cast<uint32_t*>(&rq);
            uint32_t* dp = reinterpret_cast<uint32_t*>(&rp);
            for (int i = 0; i < (int)(sizeof(RowFinal) / 4); ++i) {
                dq[i] = ldnt(&src[i]);
                dp[i] = ldnt(&src[i + sizeof(RowFinal) / 4]);
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
            const int c = s_c;
            const int slice = c / kChunks, within = c % kChunks;
            lo = slice * kSliceCols + (within / kWaves) * (kThreads * 8) + (within % kWaves) * kChunkCols;
            hi = min(lo + kChunkCols, a.V);
            base = s_base;
        } else {
            lo = 0;
            hi = a.V;
            base = 0.0;
        }
        const double target = mode == 1 ? s_target : 0.0;
        // mode 2 needs the total of q first
        double total_q = 0.0;
        if (mode == 2) {
            double acc = 0.0;
            for (int col = threadIdx.x; col < a.V; col += blockDim.x)
                acc += final_prob(rq, idk_q, idp_q, trow[col], col, false);
            total_q = block_sum<double>(acc, sm.redd);
        }
        const double tgt = mode == 1 ? target : s_target * total_q;
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
        if (threadIdx.x == 0) s_t = best != 0x7FFFFFFF ? best : last;
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        a.out_k[b] = k;
        a.out_t[b] = s_t;
        if (a.out_W) a.out_W[b] = (float)s_W;
        if (a.out_status) a.out_status[b] = s_status;
        // leave the request's counters zeroed for the next call
        *reinterpret_cast<unsigned*>(f.ws + f.L.req + (size_t)b * 128) = 0u;
        for (int j = 0; j <= K; ++j) {
            const int unit = b * (K + 1) + j;
            *reinterpret_cast<unsigned*>(f.ws + f.L.ctr + (size_t)unit * 128) = 0u;
            *reinterpret_cast<unsigned*>(f.ws + f.L.flag + (size_t)unit * 128) = 0u;
        }
    }
}

// ------------------------------------------------------------------------------------------
// The kernel
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void fast_verify_kernel(FastArgs f) {
    __shared__ Smem sm;
    const VerifyArgs& a = f.a;
    // placement: request b runs on XCD b % 8; its (K+1) units x nS slices follow in order
    const int x = blockIdx.x % kXcd;
    const int l = blockIdx.x / kXcd;
    const int per_req = (a.K + 1) * f.nS;
    const int b = (l / per_req) * kXcd + x;
    if (b >= a.B) return;
    const int j = (l / f.nS) % (a.K + 1);
    const int slice = l % f.nS;
    const int unit = b * (a.K + 1) + j;
    const int c0 = slice * kSliceCols;
    const bool two = j < a.K;
    const spec_params prm = a.params[b];
    const bool param_ok = prm.temperature >= 0.0f && !isinf(prm.temperature) && prm.top_p > 0.0f;
    const size_t stride = (size_t)a.V;
    const uint16_t* trow = static_cast<const uint16_t*>(a.target) + ((size_t)b * (a.K + 1) + j) * stride;
    const uint16_t* drow = two ? static_cast<const uint16_t*>(a.draft) + ((size_t)b * a.draft_rows + j) * stride : nullptr;
    const int s_tok = two ? a.tokens[(size_t)b * a.K + j] : -1;
    const bool tok_ok = !two || (s_tok >= 0 && s_tok < a.V);
    UnitFast* U = reinterpret_cast<UnitFast*>(f.ws + f.L.units) + unit;
    int32_t* IC = reinterpret_cast<int32_t*>(f.ws + f.L.idcut) + unit * 4;

    // ---- phase A: load, count, publish ----
    u32x4 vq[kLoads], vp[kLoads];
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
        const int col = col_of(c0, q, 0);
        vq[q] = col < a.V ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(trow + col)) : u32x4{0, 0, 0, 0};
        vp[q] = (two && col < a.V) ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(drow + col))
                                   : u32x4{0, 0, 0, 0};
    }
    for (int i = threadIdx.x; i < 2 * kBins; i += blockDim.x) (&sm.u.hist[0][0])[i] = 0u;
    if (threadIdx.x < 2) {
        sm.n_sp[threadIdx.x] = 0;
        sm.flags[threadIdx.x] = 0;
        sm.neginf[threadIdx.x] = 0;
        sm.s_bits[threadIdx.x] = 0;
    }
    if (threadIdx.x == 0 && two && tok_ok) {
        sm.s_bits[0] = trow[s_tok];
        sm.s_bits[1] = drow[s_tok];
    }
    __syncthreads();
    if (param_ok) {
        for (int r = 0; r < (two ? 2 : 1); ++r) {
            uint32_t bad = 0, ninf = 0;
#pragma unroll
            for (int q = 0; q < kLoads; ++q)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int col = col_of(c0, q, e);
                    const uint32_t w = r == 0 ? vq[q][e >> 1] : vp[q][e >> 1];
                    const uint32_t h = (e & 1) ? (w >> 16) : (w & 0xFFFFu);
                    if (col >= a.V) continue;
                    const uint32_t off = (h & 0x7FFFu) - (uint32_t)(kExpLo << 7);
                    if (off < (uint32_t)kNegBins) {
                        const int bin = (h & 0x8000u) ? (kNegBins - 1 - (int)off) : (kPosBase + (int)off);
                        atomicAdd(&sm.u.hist[r][bin], 1u);
                    } else {
                        int bin;
                        const int kind = classify(h, &bin);
                        if (kind == kKindBin) {
                            atomicAdd(&sm.u.hist[r][bin], 1u);
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
                }
            if (bad) atomicOr(&sm.flags[r], 1u);
            if (ninf) atomicAdd(&sm.neginf[r], ninf);
        }
        __syncthreads();
        publish_row(f, sm, unit, slice, 0, prm, false, c0, vq, two && tok_ok ? s_tok : -1);
        if (two) publish_row(f, sm, unit, slice, 1, prm, true, c0, vp, tok_ok ? s_tok : -1);
    }

    // ---- unit barrier ----
    unsigned* ctr = reinterpret_cast<unsigned*>(f.ws + f.L.ctr + (size_t)unit * 128);
    unsigned* flag = reinterpret_cast<unsigned*>(f.ws + f.L.flag + (size_t)unit * 128);
    const bool synced = unit_barrier(ctr, flag, f.nS);

    // ---- phase C: combine, accept, residual ----
    uint32_t status = 0;
    int accept = 0;
    bool need_resid = false;
    bool fb_unit = false;
    if (!synced) {
        status = SPEC_ST_SYNC_TIMEOUT;
    } else if (!param_ok) {
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
                    const Cut* cs[2] = {&rv.ck, &rv.cp};
                    const int has[2] = {rv.has_k, rv.has_p};
                    for (int c = 0; c < 2; ++c) {
                        if (!has[c] || cs[c]->key == 0) IC[r * 2 + c] = a.V - 1;
                        else if (cs[c]->explicit_id >= 0) IC[r * 2 + c] = cs[c]->explicit_id;
                    }
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
        sm.last = (old + 1 == (unsigned)per_req) ? 1 : 0;
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
    return nS <= 32;
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
    hipLaunchKernelGGL(fast_verify_kernel, dim3((unsigned)p.grid), dim3(kThreads), 0, stream, f);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

}  // namespace fast
}  // namespace sv
