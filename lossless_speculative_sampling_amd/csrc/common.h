// Device-side building blocks of the gfx950 verification kernels: order keys, the Philox
// stream, element loads and workgroup reductions for 64-wide wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/specverify.h"

namespace sv {

constexpr int kWave = 64;

// Per-request status bits (values fixed by the C ABI).
constexpr uint32_t kStEmptyResidual = SPEC_ST_EMPTY_RESIDUAL;
constexpr uint32_t kStOutside = SPEC_ST_OUTSIDE_DRAFT_SUPPORT;
constexpr uint32_t kStBadLogit = SPEC_ST_BAD_LOGIT;
constexpr uint32_t kStBadToken = SPEC_ST_BAD_TOKEN;
constexpr uint32_t kStDegenerate = SPEC_ST_DEGENERATE_DOWNWEIGHT;
constexpr uint32_t kStBadParam = SPEC_ST_BAD_PARAM;
constexpr uint32_t kStPlacement = SPEC_ST_PLACEMENT;

// ------------------------------------------------------------------------------------------
// Token order: a 32-bit key that grows with the logit.  -0 is folded onto +0 so that equal
// logits tie (and fall back to the lower token id); NaN gets key 0, below -inf.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key_bits(uint32_t u) {
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;  // NaN
    if (u == 0x80000000u) u = 0u;                      // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint32_t order_key(float x) { return order_key_bits(__float_as_uint(x)); }
__device__ __forceinline__ float key_to_float(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}
constexpr uint32_t kKeyPosInf = 0xFF800000u;  // order_key(+inf)

// Element i of a logit row, widened to fp32 (bf16 -> fp32 is exact).
__device__ __forceinline__ float load_logit(const void* row, int dtype, int i) {
    if (dtype == SPEC_BF16) {
        uint32_t h = static_cast<const uint16_t*>(row)[i];
        return __uint_as_float(h << 16);
    }
    return static_cast<const float*>(row)[i];
}

// ------------------------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw: "Parallel Random Numbers: As Easy as 1, 2, 3",
// SC'11).  Two 64x64 -> 128-bit products per round, Weyl key schedule between rounds.
// ------------------------------------------------------------------------------------------
struct Block4 {
    uint64_t w[4];
};

__device__ __forceinline__ Block4 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3, uint64_t key0,
                                                uint64_t key1) {
    const uint64_t mulA = 0xD2E7470EE14C6C93ull, mulB = 0xCA5A826395121157ull;
    const uint64_t weylA = 0x9E3779B97F4A7C15ull, weylB = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t pa_hi = __umul64hi(mulA, c0), pa_lo = mulA * c0;
        const uint64_t pb_hi = __umul64hi(mulB, c2), pb_lo = mulB * c2;
        const uint64_t n0 = pb_hi ^ c1 ^ key0;
        const uint64_t n2 = pa_hi ^ c3 ^ key1;
        c0 = n0;
        c1 = pb_lo;
        c2 = n2;
        c3 = pa_lo;
        key0 += weylA;
        key1 += weylB;
    }
    Block4 b;
    b.w[0] = c0;
    b.w[1] = c1;
    b.w[2] = c2;
    b.w[3] = c3;
    return b;
}

// Uniform in (0, 1) from one 64-bit word: the top 52 bits plus half an ulp (exact in fp64).
__device__ __forceinline__ double word_to_uniform(uint64_t w) {
    return ((double)(w >> 12) + 0.5) * 0x1.0p-52;
}

// The uniforms of request b, position j: word 0 acceptance, 1 residual/bonus, 2 draft sampling.
__device__ __forceinline__ double uniform_at(uint64_t seed, uint64_t round, uint64_t b, uint64_t j, int word) {
    Block4 x = philox4x64_10(round, b, j, 0, seed, 0);
    return word_to_uniform(x.w[word]);
}

// A draw from the uniform law on [0, V) by inverse CDF, floor(u V), for the uniform u of word
// w: u = (2 (w >> 12) + 1) / 2^53 exactly, so the floor is taken on the exact 128-bit product.
__device__ __forceinline__ int uniform_token_of(uint64_t w, int V) {
    const uint64_t m = 2 * (w >> 12) + 1;
    const uint64_t lo = m * (uint64_t)V, hi = __umul64hi(m, (uint64_t)V);
    return (int)((hi << 11) | (lo >> 53));
}
// The backup speculator's draft token for request b, position j (word 2, the draft lane).
__device__ __forceinline__ int uniform_draft_token(uint64_t seed, uint64_t round, uint64_t b, uint64_t j, int V) {
    Block4 x = philox4x64_10(round, b, j, 0, seed, 0);
    return uniform_token_of(x.w[2], V);
}

// ------------------------------------------------------------------------------------------
// Cross-lane moves.  Reductions and scans use DPP (operand permutations inside VALU
// instructions) and v_readlane, never ds_bpermute: those go through the LDS unit, where they
// queue behind other workgroups' histogram atomics.
// ------------------------------------------------------------------------------------------
enum : int {
    kDppQuadSwap1 = 0xB1,      // quad_perm [1,0,3,2]: lane ^ 1
    kDppQuadSwap2 = 0x4E,      // quad_perm [2,3,0,1]: lane ^ 2
    kDppRowShr1 = 0x111,
    kDppRowShr2 = 0x112,
    kDppRowShr4 = 0x114,
    kDppRowShr8 = 0x118,
    kDppWaveShr1 = 0x138,      // lane i <- lane i - 1 across the wave
    kDppRowMirror = 0x140,     // within 16 lanes: i <- 15 - i
    kDppRowHalfMirror = 0x141, // within 8 lanes: i <- 7 - i
    kDppRowBcast15 = 0x142,    // lane 15 of each row -> the next row
    kDppRowBcast31 = 0x143,    // lane 31 -> rows 2 and 3
};

// v from the lane that DPP control CTRL names; 0 where the source lane does not exist or the
// row is masked off (ROW_MASK).
template <int CTRL, int ROW_MASK = 0xF, typename T>
__device__ __forceinline__ T dpp(T v) {
    static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
    if constexpr (sizeof(T) == 4) {
        int u;
        __builtin_memcpy(&u, &v, 4);
        u = __builtin_amdgcn_update_dpp(0, u, CTRL, ROW_MASK, 0xF, true);
        T r;
        __builtin_memcpy(&r, &u, 4);
        return r;
    } else {
        int u[2];
        __builtin_memcpy(u, &v, 8);
        u[0] = __builtin_amdgcn_update_dpp(0, u[0], CTRL, ROW_MASK, 0xF, true);
        u[1] = __builtin_amdgcn_update_dpp(0, u[1], CTRL, ROW_MASK, 0xF, true);
        T r;
        __builtin_memcpy(&r, u, 8);
        return r;
    }
}

// v of lane `lane` (a wave-uniform index) in every lane.
template <typename T>
__device__ __forceinline__ T wave_bcast(T v, int lane) {
    static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
    if constexpr (sizeof(T) == 4) {
        int u;
        __builtin_memcpy(&u, &v, 4);
        u = __builtin_amdgcn_readlane(u, lane);
        T r;
        __builtin_memcpy(&r, &u, 4);
        return r;
    } else {
        int u[2];
        __builtin_memcpy(u, &v, 8);
        u[0] = __builtin_amdgcn_readlane(u[0], lane);
        u[1] = __builtin_amdgcn_readlane(u[1], lane);
        T r;
        __builtin_memcpy(&r, u, 8);
        return r;
    }
}

// Butterfly over each row of 16 lanes, then the four row results; fixed order, so every
// wave of every workgroup combining the same values gets the same bits.
template <typename T, typename Op>
__device__ __forceinline__ T wave_allreduce(T v, Op op) {
    v = op(v, dpp<kDppQuadSwap1>(v));
    v = op(v, dpp<kDppQuadSwap2>(v));
    v = op(v, dpp<kDppRowHalfMirror>(v));
    v = op(v, dpp<kDppRowMirror>(v));
    const T r0 = wave_bcast(v, 0), r1 = wave_bcast(v, 16), r2 = wave_bcast(v, 32), r3 = wave_bcast(v, 48);
    return op(op(r0, r1), op(r2, r3));
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
    return wave_allreduce(v, [](T a, T b) { return a + b; });
}
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
    return wave_allreduce(v, [](T a, T b) { return b > a ? b : a; });
}
template <typename T>
__device__ __forceinline__ T wave_min(T v) {
    return wave_allreduce(v, [](T a, T b) { return b < a ? b : a; });
}
template <typename T>
__device__ __forceinline__ T wave_or(T v) {
    return wave_allreduce(v, [](T a, T b) { return a | b; });
}

// Sum over each aligned group of 8 lanes, in every lane of the group.
template <typename T>
__device__ __forceinline__ T group8_sum(T v) {
    v += dpp<kDppQuadSwap1>(v);
    v += dpp<kDppQuadSwap2>(v);
    v += dpp<kDppRowHalfMirror>(v);
    return v;
}

template <typename T, int OP>  // OP 0 sum, 1 max, 2 min
__device__ __forceinline__ T wave_reduce(T v) {
    if (OP == 0) return wave_sum(v);
    if (OP == 1) return wave_max(v);
    return wave_min(v);
}

// Inclusive prefix sum over the lanes of a wave in lane order; *excl gets the exclusive one.
template <typename T>
__device__ __forceinline__ T wave_scan(T v, T* excl) {
    v += dpp<kDppRowShr1>(v);
    v += dpp<kDppRowShr2>(v);
    v += dpp<kDppRowShr4>(v);
    v += dpp<kDppRowShr8>(v);
    v += dpp<kDppRowBcast15, 0xA>(v);
    v += dpp<kDppRowBcast31, 0xC>(v);
    *excl = dpp<kDppWaveShr1>(v);
    return v;
}

// Lowest / highest set lane of a ballot (-1 when empty).
__device__ __forceinline__ int first_lane(uint64_t m) { return m ? __builtin_ctzll(m) : -1; }
__device__ __forceinline__ int last_lane(uint64_t m) { return m ? 63 - __builtin_clzll(m) : -1; }

// Workgroup reduction; every thread gets the result.  Deterministic (fixed tree).
template <typename T, int OP>
__device__ __forceinline__ T block_reduce(T v, T* red) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwaves = blockDim.x / kWave;
    v = wave_reduce<T, OP>(v);
    __syncthreads();  // red may still be read by a previous reduction
    if (lane == 0) red[wave] = v;
    __syncthreads();
    T r = red[0];
    for (int w = 1; w < nwaves; ++w) {
        T x = red[w];
        if (OP == 0) r += x;
        else if (OP == 1) r = x > r ? x : r;
        else r = x < r ? x : r;
    }
    return r;
}

template <typename T>
__device__ __forceinline__ T block_sum(T v, T* red) { return block_reduce<T, 0>(v, red); }
template <typename T>
__device__ __forceinline__ T block_max(T v, T* red) { return block_reduce<T, 1>(v, red); }
template <typename T>
__device__ __forceinline__ T block_min(T v, T* red) { return block_reduce<T, 2>(v, red); }

// Exclusive prefix sum over the workgroup in thread order; *total gets the sum.
template <typename T>
__device__ __forceinline__ T block_exclusive_scan(T v, T* red, T* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwaves = blockDim.x / kWave;
    T exc;
    const T inc = wave_scan(v, &exc);
    __syncthreads();
    if (lane == kWave - 1) red[wave] = inc;
    __syncthreads();
    T before = T(0), all = T(0);
    for (int w = 0; w < nwaves; ++w) {
        T x = red[w];
        if (w < wave) before += x;
        all += x;
    }
    *total = all;
    return before + exc;
}

constexpr int kXcd = 8;  // XCDs on MI355X

// ------------------------------------------------------------------------------------------
// Arrival counters in an XCD's L2 (every workgroup that meets at one counter runs on one XCD:
// the dispatcher hands workgroup x to XCD x % kXcd)
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ unsigned l2_fetch_add(unsigned* p, unsigned v) {
    unsigned old;
    asm volatile("s_waitcnt vmcnt(0)\n\tglobal_atomic_add %0, %1, %2, off sc0\n\ts_waitcnt vmcnt(0)"
                 : "=v"(old) : "v"(p), "v"(v) : "memory");
    return old;
}

__device__ __forceinline__ uint64_t l2_fetch_add64(uint64_t* p, uint64_t v) {
    uint64_t old;
    asm volatile("s_waitcnt vmcnt(0)\n\tglobal_atomic_add_x2 %0, %1, %2, off sc0\n\ts_waitcnt vmcnt(0)"
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

}  // namespace sv
