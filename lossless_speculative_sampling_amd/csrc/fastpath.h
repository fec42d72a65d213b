// Register-resident bf16 verification path (one kernel per call).
//
// A (request b, position j) unit covers draft row j and target row j (target row K alone for
// j = K).  Each unit is split into slices of kSliceCols token columns; the slices of a unit
// run on one XCD (workgroup b -> XCD b % 8), hold their columns in registers, count every
// distinct bf16 logit in LDS, publish compact summaries, meet once at a unit barrier through
// that XCD's L2, resolve the exact processed distributions redundantly, and, when the draft
// token is rejected (or at the bonus position), sum the residual (q - p)+ over 512-column
// chunks.  The last slice of a request to finish picks k and t*.
#pragma once

#include "generic.h"

namespace sv {
namespace fast {

constexpr int kThreads = 512;                  // workgroup size (8 waves)
constexpr int kColsPerThread = 32;             // per row
constexpr int kLoads = kColsPerThread / 8;     // 16-byte loads per row per thread
constexpr int kSliceCols = kThreads * kColsPerThread;  // 16384
constexpr int kChunkCols = 512;                // one wave x one 16-byte load per lane
constexpr int kChunks = kSliceCols / kChunkCols;       // 32 per slice

// Exact bins: one per bf16 value with |z| in [2^-6, 2^5), plus zero.  Negative values occupy
// bins [0, kNegBins) in ascending value order, zero bin kZeroBin, positive values
// [kPosBase, kPosBase + kNegBins).  Bins are grouped by 64 (aligned), zero in its own group.
constexpr int kExpLo = 121;                    // bf16 exponent field of 2^-6
constexpr int kExpHi = 132;                    // first exponent outside (2^5)
constexpr int kNegBins = (kExpHi - kExpLo) * 128;      // 1408
constexpr int kGroup = 64;
constexpr int kZeroBin = kNegBins;                     // 1408
constexpr int kPosBase = kNegBins + kGroup;            // 1472
constexpr int kBins = kPosBase + kNegBins;             // 2880 (padded)
constexpr int kGroups = kBins / kGroup;                // 45
constexpr int kNegGroups = kNegBins / kGroup;          // 22
constexpr int kZeroGroup = kNegGroups;                 // 22
// Segments in descending value order: huge positive specials, positive groups (high to low),
// tiny positive specials, the zero group, tiny negative specials, negative groups (high to
// low), huge negative specials.
constexpr int kSegs = kGroups + 4;                     // 49
constexpr int kSegHugePos = 0;
constexpr int kSegTinyPos = 1 + kNegGroups;            // 23
constexpr int kSegZero = kSegTinyPos + 1;              // 24
constexpr int kSegTinyNeg = kSegZero + 1;              // 25
constexpr int kSegHugeNeg = kSegs - 1;                 // 48

constexpr int kTop = 64;        // per slice-row candidate list (top by token order)
constexpr int kSpecial = 64;    // per slice-row finite values outside the exact bins

struct FastPlan {
    int nS;          // slices per row
    int units;       // B * (K + 1)
    int grid;        // workgroups of the count kernel
    int grid_resolve;// workgroups of the resolve kernel
    int halves;      // resolve workgroups per slice of the residual (2: each sums half the chunks)
    int slice_prio;  // the count grid is resident at once (one round of workgroups)
    int grid_diverge;// workgroups of the divergence kernel (fuzzy acceptance)
    size_t ws_bytes; // fast workspace bytes
};

FastPlan fast_plan(int B, int K, int V);
// bf16 rows, V % 8 == 0 and V >= 2048, 16-byte aligned rows, at most 16 slices per row and
// K + 1 <= 64 positions per request (longer drafts take the general path).
bool fast_path_applies(const VerifyArgs& a);
// Fuzzy acceptance (a.tau set) on this path: not the assisted variant, at most 63 positions.
bool fast_fuzzy_applies(const VerifyArgs& a);
int fast_verify(const VerifyArgs& a, void* ws, size_t ws_bytes, hipStream_t stream);
// The same pass also builds the Saguaro outcome cache (cache != nullptr); fast_cache_applies
// says whether every depth's list fits the per-slice candidate lists.
bool fast_cache_applies(const VerifyArgs& a, const CacheArgs& c);
int fast_verify_cache(const VerifyArgs& a, const CacheArgs& c, void* ws, size_t ws_bytes, hipStream_t stream);
// The same with the cache lookup of the outcomes (saguaro_cache_lookup mode 0) fused into the
// resolve kernel; fast_lookup_fuses says whether it applies (otherwise the caller launches the
// lookup after the call).
struct LookupOut {
    int32_t* slot;
    uint8_t* hit;
    int32_t* batch;
};
bool fast_lookup_fuses(const VerifyArgs& a);
// Optional HIP events that bound the count kernel's execution (the launch's start and stop
// events, for timing that kernel on its own); null: none.
struct CountEvents {
    hipEvent_t before, after;
};
int fast_verify_cache_lookup(const VerifyArgs& a, const CacheArgs& c, const LookupOut& l, void* ws, size_t ws_bytes,
                             hipStream_t stream, const CountEvents* ev = nullptr);

}  // namespace fast
}  // namespace sv
