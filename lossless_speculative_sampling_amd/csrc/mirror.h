// Mirror-SD signposts and draft-tree reuse (Mirror Speculative Decoding reading notes, sections
// 3.1-3.3): launch arguments and sizing shared by the C ABI and the kernels.
//
// Signposts: for each request, the kappa most likely tokens of the early-exit distribution
// (softmax of one logit row) with their log-probabilities.  A row is cut into slices of
// kSliceSpan columns, one 4-wave workgroup per slice and 32 contiguous columns per lane.  Each
// wave publishes its own sorted top-kappa list with its maximum and its sum of exponentials;
// the last workgroup of the row to arrive merges the lists.  All workgroups of a row run on
// one XCD (workgroup x -> XCD x % kXcd), so they meet at an arrival counter in that XCD's L2.
#pragma once

#include "common.h"

namespace sv {
namespace mirror {

constexpr int kThreads = 256;                   // signpost workgroup (4 waves)
constexpr int kWaves = kThreads / kWave;
constexpr int kPer = 32;                        // contiguous columns per lane
constexpr int kWaveSpan = kWave * kPer;         // 2048 columns per wave
constexpr int kSliceSpan = kWaves * kWaveSpan;  // 8192 columns per workgroup
constexpr int kMaxKappa = SPEC_MAX_KAPPA;
constexpr int kMaxV = 1 << 19;                  // up to 256 lists per row (the merge holds them in LDS)
constexpr int kTreeThreads = 256;
constexpr int kTreeLdsNodes = 4096;             // trees up to this size are walked in LDS
constexpr int kMaxGamma = 1024;

// One wave's list: header, then `kappa` entries (order key << 32 | ~column, descending).
struct ListHead {
    float m;        // the wave's largest logit (-inf if it holds none)
    int32_t count;  // valid entries (min(kappa, columns))
    double S;       // sum of exp(z - m) over the wave's columns (NaN flags a NaN / +inf logit)
};

struct SpPlan {
    int nS, L;              // slices per row, lists per row
    size_t rec_stride;      // bytes per list record
    size_t ctr_bytes, ws_bytes;
    size_t wave_lds;        // per-wave LDS of the list phase
    size_t lds_bytes;       // dynamic LDS of a workgroup (list phase, then the merge)
};

__host__ __device__ inline size_t align_to(size_t x, size_t a) { return (x + a - 1) / a * a; }

// LDS of one wave's list phase: up to 2 kappa staged lanes (32 floats each) and their lane
// ids, then the elements above the threshold (at most 32 (kappa - 1)) and the first kappa ties.
__host__ __device__ inline size_t wave_stage_bytes(int kappa) {
    return align_to((size_t)2 * kappa * kPer * 4 + (size_t)2 * kappa * 4, 8);
}
__host__ __device__ inline size_t wave_lds_bytes(int kappa) {
    return wave_stage_bytes(kappa) + (size_t)kPer * kappa * 8 + (size_t)kappa * 8;
}
// LDS of the merge: maxima, counts, top-head lists, sums, kappa^2 candidates, heads, entries.
__host__ __device__ inline size_t merge_lds_bytes(int L, int kappa) {
    return align_to((size_t)L * 8 + (size_t)kappa * 4, 8) + (size_t)L * 8 + (size_t)kappa * kappa * 8 +
           (size_t)L * 8 + (size_t)L * kappa * 8;
}

__host__ __device__ inline SpPlan signpost_plan(int B, int V, int kappa) {
    SpPlan p;
    p.nS = (V + kSliceSpan - 1) / kSliceSpan;
    p.L = p.nS * kWaves;
    p.rec_stride = sizeof(ListHead) + (size_t)kappa * sizeof(uint64_t);
    p.ctr_bytes = align_to((size_t)B * 128, 256);
    p.ws_bytes = p.ctr_bytes + align_to((size_t)B * p.L * p.rec_stride, 256);
    p.wave_lds = wave_lds_bytes(kappa);
    const size_t lists = kWaves * p.wave_lds;
    const size_t merge = merge_lds_bytes(p.L, kappa);
    p.lds_bytes = lists > merge ? lists : merge;
    return p;
}

struct SignpostArgs {
    const void* logits;
    int dtype, B, V, kappa;
    SpPlan plan;
    int32_t* out_ids;
    float* out_logp;
    uint16_t* out_logp_bf16;
    uint32_t* out_status;
    char* ws;
};

struct TreeArgs {
    const int32_t* tokens;
    const int32_t* parents;
    int B, N, gamma;
    const int32_t* path;
    const int32_t* k;
    const int32_t* tstar;
    int32_t* out_node;
    uint8_t* out_hit;
    int32_t* out_batch;
};

// Launchers (hipGetLastError reports launch failures to the caller).
void launch_signposts(const SignpostArgs& a, int vec, hipStream_t stream);
void launch_tree_lookup(const TreeArgs& a, hipStream_t stream);

}  // namespace mirror
}  // namespace sv
