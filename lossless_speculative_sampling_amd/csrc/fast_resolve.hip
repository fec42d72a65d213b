// Resolve kernel of the bf16 verification path.  The count kernel has decided every request:
// its first rejected position k (or K) and whether a residual is still to be drawn.  Here
// the slices of unit k sum the residual (q_k - p'_k)+ (or the target q_K at the bonus
// position) over 512-column chunks, and the last of them draws t* by inverse CDF in token
// order (DeepMind speculative-sampling page, sections 1 and 3; SSD reading notes, section
// 2.2).  Requests whose units the counts could not settle run the general algorithm.
#include "fast_common.h"
#include "rowproc.h"

namespace sv {
namespace fast {

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
    UnitCut cut[2][2];
    uint32_t flags[2];             // this slice's RowPart flags of each row
    int eff[2][2];                 // this slice's id cut at each cut key (V-1 all, -1 none)
    int32_t scan[kWaves + 1];
    double redd[kWaves];
    int32_t redi[kWaves];
    int found;
    int last;
    int fc;
    double ftarget, fbase;
};

// The n-th (1-based) element of this slice, in token order, whose key equals `key`.
__device__ __forceinline__ int local_nth_at_key(ResSmem& sm, const u32x4 (&v)[kLoads], int c0, int V, uint32_t key, int n) {
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

// Processed probability of one element from the row's final statistics and id cuts
// (operation order ((e / S) * f) / Z, the same as the per-bin tables).
__device__ __forceinline__ double final_prob(const RowFinal& rf, int idk, int idp, uint32_t h, int col, bool draft) {
    const uint32_t mag = h & 0x7FFFu;
    if (mag >= 0x7F80u) return 0.0;  // -inf (rows with NaN or +inf never get here)
    if (rf.greedy) return col == rf.argmax ? 1.0 : 0.0;
    const uint32_t key = key16(h);
    if (!in_cut_id(rf.kk, idk, key, col) || !in_cut_id(rf.kp, idp, key, col)) return 0.0;
    const double e = mass_of(__uint_as_float(h << 16), rf.m, rf.invT);
    const double p = e / rf.S;
    if (!draft) return p;
    const double fct = (rf.nS > 0 && e > 0.0 && in_cut_id(rf.kF, rf.idF, key, col)) ? rf.C : 1.0;
    return (p * fct) / rf.Z;
}

// Whether this slice's elements at a cut key are kept: all (before the owner), none (after),
// or decided per element (the owner itself).
__device__ __forceinline__ bool slice_keeps(const UnitCut& c, int slice) { return slice <= c.owner; }

// Table entries that stand for "decide this element exactly": large enough that any 512-
// column partial sum containing one exceeds kMarkSeen, which no true sum of probabilities can.
constexpr double kMarkQ = 1e300;    // in the target table: (q - p)+ and q become huge
constexpr double kMarkP = -1e300;   // in the draft table: (q - p)+ becomes huge
constexpr double kMarkSeen = 1e299;

// Per-bin values of row r for this slice: q = e / S, p' = ((e / S) * f) / Z, with every cut
// key resolved as this slice sees it.  Where this slice decides elements at a key one by one
// (it holds the last kept element at a cut key, or the draft row's downweighted-set
// boundary), and in the padding words when the slice holds values outside the exact bins,
// the entry is a marker.  Bins above the row maximum hold no element and bins below the cuts
// are 0, so only bins between them need an exp.
__device__ __forceinline__ void build_table(ResSmem& sm, int r, int slice, bool draft) {
    const RowFinal& rf = sm.rf[r];
    const UnitCut& ck = sm.cut[r][0];
    const UnitCut& cp = sm.cut[r][1];
    const uint32_t kmax = key16(__float_as_uint(rf.m) >> 16);
    const uint32_t klow = max(ck.key, cp.key);
    const int ownerF = rf.nS > 0 ? rf.idF / kSliceCols : -1;
    const double mark = r == 0 ? kMarkQ : kMarkP;
    const bool rare = (sm.flags[r] & 4u) != 0;
    const uint32_t own_k = (ck.key != 0u && ck.owner == slice) ? ck.key : 0xFFFFFFFFu;
    const uint32_t own_p = (cp.key != 0u && cp.owner == slice) ? cp.key : 0xFFFFFFFFu;
    const uint32_t own_F = (draft && ownerF == slice) ? rf.kF : 0xFFFFFFFFu;
    double* t = &sm.u.tab[r][0];
    for (int i = threadIdx.x; i < kHistRow; i += blockDim.x) {
        const int bin = i - kHistLead;
        double v = 0.0;
        if (bin >= 0 && bin < kBins) {
            const uint32_t key = bin_key(bin);
            if (key == own_k || key == own_p || key == own_F) {
                v = mark;
            } else if (key >= klow && key <= kmax && (key > ck.key || slice_keeps(ck, slice)) &&
                       (key > cp.key || slice_keeps(cp, slice))) {
                const double e = mass_of(key16_value(key), rf.m, rf.invT);
                v = e / rf.S;
                if (draft) {
                    const bool in_set = rf.nS > 0 && e > 0.0 && (key > rf.kF || (key == rf.kF && slice <= ownerF));
                    v = (v * (in_set ? rf.C : 1.0)) / rf.Z;
                }
            }
        } else if (rare) {
            v = mark;
        }
        t[i] = v;
    }
}

// Byte offsets of the two fp64 table entries of the bf16 values packed in w.
__device__ __forceinline__ uint32_t tab_offsets2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, hist_offsets2(w)) << (u16x2)(uint16_t)1);
}
__device__ __forceinline__ double tab_at(const char* base, uint32_t off) {
    return *reinterpret_cast<const double*>(base + off);
}

// Residual of unit k over this slice's columns, per 512-column chunk: table lookups for every
// element; a thread's 8 columns of one chunk that met a marker are recomputed exactly.
__device__ __forceinline__ void residual_slice(const FastArgs& f, ResSmem& sm, int b, int slice, int c0, bool two,
                                               const u32x4 (&vq)[kLoads], const u32x4 (&vp)[kLoads]) {
    const VerifyArgs& a = f.a;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const char* tq = reinterpret_cast<const char*>(&sm.u.tab[0][0]);
    const char* tp = reinterpret_cast<const char*>(&sm.u.tab[1][0]);
    double* out = reinterpret_cast<double*>(f.ws + f.L.chunks) + ((size_t)b * f.nS + slice) * kChunks;
#pragma unroll
    for (int q = 0; q < kLoads; ++q) {
        double s = 0.0;
        if (col_of(c0, q, 0) < a.V) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t oq = tab_offsets2(vq[q][d]);
                const double q0 = tab_at(tq, oq & 0xFFFFu), q1 = tab_at(tq, oq >> 16);
                if (two) {
                    const uint32_t op = tab_offsets2(vp[q][d]);
                    const double p0 = tab_at(tp, op & 0xFFFFu), p1 = tab_at(tp, op >> 16);
                    s += max(q0 - p0, 0.0);
                    s += max(q1 - p1, 0.0);
                } else {
                    s += q0;
                    s += q1;
                }
            }
            if (s > kMarkSeen) {  // rare: decide these columns exactly
                s = 0.0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int col = col_of(c0, q, e);
                    const uint32_t wq = vq[q][e >> 1];
                    const uint32_t hq = (e & 1) ? (wq >> 16) : (wq & 0xFFFFu);
                    const double qe = final_prob(sm.rf[0], sm.eff[0][0], sm.eff[0][1], hq, col, false);
                    if (two) {
                        const uint32_t wp = vp[q][e >> 1];
                        const uint32_t hp = (e & 1) ? (wp >> 16) : (wp & 0xFFFFu);
                        s += max(qe - final_prob(sm.rf[1], sm.eff[1][0], sm.eff[1][1], hp, col, true), 0.0);
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

// The last slice of unit k: the chunk whose cumulative residual passes v * W, then the token
// inside it by an exact scan (or, with no residual mass, inverse CDF of q_k).
__device__ __forceinline__ void finalize_residual(const FastArgs& f, ResSmem& sm, int b, int k, uint32_t status) {
    const VerifyArgs& a = f.a;
    const int K = a.K;
    const int n = f.nS * kChunks;
    const double* ch = reinterpret_cast<const double*>(f.ws + f.L.chunks) + (size_t)b * f.nS * kChunks;
    const int32_t* IC = reinterpret_cast<const int32_t*>(f.ws + f.L.idcut) + b * 4;
    const int c = threadIdx.x;
    const double x = c < n ? ldnt(&ch[c]) : 0.0;
    const int idk_q = ldnt(&IC[0]), idp_q = ldnt(&IC[1]), idk_p = ldnt(&IC[2]), idp_p = ldnt(&IC[3]);
    double W;
    const double before = block_exclusive_scan<double>(x, sm.redd, &W);
    const double v = uniform_at(a.seed, a.round, (uint64_t)b, (uint64_t)k, 1);
    int mode;
    if (W > 0.0) {
        // the last chunk with mass whose preceding mass is <= v * W
        const double target = v * W;
        const int pick = block_max<int>((x > 0.0 && before <= target) ? c : -1, sm.redi);
        if (pick == c) sm.fbase = before;
        if (threadIdx.x == 0) {
            sm.fc = pick;
            sm.ftarget = target;
        }
        mode = 1;
    } else {
        if (threadIdx.x == 0) sm.ftarget = v;
        status |= kStEmptyResidual;
        mode = 2;
    }
    __syncthreads();
    const RowFinal& rq = sm.rf[0];
    const RowFinal& rp = sm.rf[1];
    const size_t stride = (size_t)a.V;
    const uint16_t* trow = static_cast<const uint16_t*>(a.target) + ((size_t)b * (K + 1) + k) * stride;
    const uint16_t* drow = k < K ? static_cast<const uint16_t*>(a.draft) + ((size_t)b * a.draft_rows + k) * stride : nullptr;
    // columns to scan: the picked chunk (mode 1) or the whole target row (mode 2)
    int lo, hi;
    double base;
    if (mode == 1) {
        const int cc = sm.fc;
        const int slice = cc / kChunks, within = cc % kChunks;
        lo = slice * kSliceCols + (within / kWaves) * (kThreads * 8) + (within % kWaves) * kChunkCols;
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
        for (int col = threadIdx.x; col < a.V; col += blockDim.x) acc += final_prob(rq, idk_q, idp_q, trow[col], col, false);
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
        const double bef = block_exclusive_scan<double>(w, sm.redd, &tot);
        const double cum = base + bef + w;
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
    if (threadIdx.x == 0) {
        a.out_k[b] = k;
        a.out_t[b] = best != 0x7FFFFFFF ? best : last;
        if (a.out_W) a.out_W[b] = k == K ? 0.0f : (float)W;
        if (a.out_status) a.out_status[b] = status;
    }
}

// The general algorithm for one unit (out of line: a rare path).  The arguments come by
// value so that no pointer to the kernel's own arguments escapes (which would move them to
// scratch memory for the whole kernel).
__device__ __noinline__ void fallback_unit(VerifyArgs a, int b, int j, ResSmem& sm) {
    unit_verify(a, b, j, &sm.urec, sm.u.generic, sm.gst[0], sm.gst[1]);
}

// Request arrival in the XCD's L2; true for the last of `expected` workgroups (which resets
// the counter for the next call).
__device__ __forceinline__ bool arrive_last(const FastArgs& f, ResSmem& sm, int b, int expected) {
    drain_stores();
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned* rc = reinterpret_cast<unsigned*>(f.ws + f.L.res_ctr + (size_t)b * 128);
        const unsigned old = l2_fetch_add(rc, 1u);
        sm.last = (old + 1 == (unsigned)expected) ? 1 : 0;
        if (sm.last) *rc = 0u;
    }
    __syncthreads();
    return sm.last != 0;
}

// The general algorithm for every unit of request b, and the request's outcome from them.
__device__ __forceinline__ void general_request(const FastArgs& f, ResSmem& sm, int b, int j) {
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
    if (a.out_status) a.out_status[b] = st;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void fast_resolve_kernel(FastArgs f) {
    __shared__ ResSmem sm;
    const VerifyArgs& a = f.a;
    const Place P = place_of(f);
    if (P.b >= a.B) return;
    const int b = P.b, j = P.j, slice = P.slice, unit = P.unit;
    // outcome-cache rows the count kernel's candidate lists could not settle
    if (f.cache && slice == 0 && reinterpret_cast<const int32_t*>(f.ws + f.L.cache_gen)[unit]) {
        CacheArgs c{a.draft, a.dtype, a.B, a.K, a.V, a.tokens, f.budget, f.fan, f.out_cache};
        cache_row(c, b, j, sm.u.cache.rs, sm.gst[0], sm.u.cache.cs);
        __syncthreads();
    }
    const ReqFast* R = reinterpret_cast<const ReqFast*>(f.ws + f.L.reqs) + b;
    const int mode = R->mode;
    if (mode == 0) return;  // decided by the count kernel
    if (mode == 2) {
        if (slice == 0) general_request(f, sm, b, j);
        return;
    }
    // mode 1: the residual of unit k
    const int k = R->k;
    if (j != k) return;
    const uint32_t status = R->status;
    const bool two = k < a.K;
    const int c0 = slice * kSliceCols;
    const size_t stride = (size_t)a.V;
    const uint16_t* trow = static_cast<const uint16_t*>(a.target) + ((size_t)b * (a.K + 1) + k) * stride;
    const uint16_t* drow = two ? static_cast<const uint16_t*>(a.draft) + ((size_t)b * a.draft_rows + k) * stride : nullptr;
    u32x4 vq[kLoads], vp[kLoads];
    load_slice(trow, c0, a.V, vq);
    if (two) {
        load_slice(drow, c0, a.V, vp);
    } else {
#pragma unroll
        for (int q = 0; q < kLoads; ++q) vp[q] = u32x4{0, 0, 0, 0};
    }
    // the unit's record (row statistics and cuts) and this slice's flags
    {
        static_assert(offsetof(UnitFast, rp) == offsetof(UnitFast, rq) + sizeof(RowFinal), "rq, rp adjacent");
        const UnitFast* U = reinterpret_cast<const UnitFast*>(f.ws + f.L.units) + unit;
        constexpr int kRf = (int)(sizeof(RowFinal) / 4), kCut = (int)(sizeof(UnitCut) / 4);
        const uint32_t* src = reinterpret_cast<const uint32_t*>(&U->rq);
        const uint32_t* srcc = reinterpret_cast<const uint32_t*>(&U->cut[0][0]);
        const int nrf = two ? 2 * kRf : kRf, ncut = two ? 4 * kCut : 2 * kCut;
        if ((int)threadIdx.x < nrf) reinterpret_cast<uint32_t*>(&sm.rf[0])[threadIdx.x] = ldnt(src + threadIdx.x);
        if ((int)threadIdx.x < ncut) reinterpret_cast<uint32_t*>(&sm.cut[0][0])[threadIdx.x] = ldnt(srcc + threadIdx.x);
        if (!two && threadIdx.x >= kWave && threadIdx.x < kWave + 2) sm.cut[1][threadIdx.x - kWave] = UnitCut{0u, -1, 0, 0};
        if (threadIdx.x < 2) sm.flags[threadIdx.x] = (threadIdx.x == 0 || two) ? ldnt(&part_of(f, unit, slice, threadIdx.x)->flags) : 0u;
    }
    __syncthreads();
    // this slice's id cut at each cut key; the owner of a histogram cut finds its id
    int32_t* IC = reinterpret_cast<int32_t*>(f.ws + f.L.idcut) + b * 4;
    for (int r = 0; r < 2; ++r) {
        for (int c = 0; c < 2; ++c) {
            const UnitCut uc = sm.cut[r][c];
            int e = a.V - 1;
            if (uc.key != 0u) {
                if (uc.explicit_id >= 0) e = uc.explicit_id;
                else if (slice < uc.owner) e = a.V - 1;
                else if (slice > uc.owner) e = -1;
                else e = local_nth_at_key(sm, r == 0 ? vq : vp, c0, a.V, uc.key, uc.owner_take);
            }
            if (threadIdx.x == 0) {
                sm.eff[r][c] = e;
                // the id cut the finaliser uses: explicit or none from slice 0, a histogram
                // cut's from its owner
                const bool writer = (uc.key == 0u || uc.explicit_id >= 0) ? slice == 0 : slice == uc.owner;
                if (writer) IC[r * 2 + c] = e;
            }
        }
    }
    build_table(sm, 0, slice, false);
    if (two) build_table(sm, 1, slice, true);
    __syncthreads();
    residual_slice(f, sm, b, slice, c0, two, vq, vp);
    if (!arrive_last(f, sm, b, f.nS)) return;
    finalize_residual(f, sm, b, k, status);
}

void launch_resolve(const FastArgs& f, int grid, hipStream_t stream) {
    hipLaunchKernelGGL(fast_resolve_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, f);
}

}  // namespace fast
}  // namespace sv
