// Launch arguments shared by the C-ABI layer and the kernels.
#pragma once

#include "common.h"

namespace sv {

constexpr int kMaxK = 64;             // largest draft length the cache entry points accept
constexpr int kRowThreadsHost = 1024;  // workgroup size of the row-processing kernels

// Per-(request, position) verification record in the workspace.
struct UnitRec {
    int32_t accept;  // draft token accepted at this position (1 for the bonus position)
    int32_t tcand;   // correction (or bonus) token if this is the first rejection
    float W;         // residual mass at this position when rejected
    uint32_t status; // status bits raised by this position
    int32_t token;   // the draft token evaluated here
};

struct VerifyArgs {
    const void* draft;
    const void* target;
    int draft_rows, dtype, B, K, V;
    const spec_params* params;
    int F;
    float C;
    int32_t* tokens;
    uint64_t seed, round;
    uint32_t flags;
    int32_t* out_k;
    int32_t* out_t;
    float* out_W;
    uint32_t* out_status;
    UnitRec* units;
    // fuzzy acceptance (PyramidSD): per-request thresholds on the Jensen-Shannon divergence of
    // q_j and p'_j (null: the lossless rule), the divergences out [B][K] (nullable)
    const float* tau;
    float* out_div;
};

struct DownweightArgs {
    const void* draft;
    int draft_rows, dtype, B, K, V;
    const spec_params* params;
    int F;
    float C;
    int32_t* out_ids;
    float* out_Z;
    float* out_probs;
    uint32_t* out_status;
};

struct Fanout {
    int32_t f[kMaxK + 1];
    int32_t off[kMaxK + 2];
};

struct CacheArgs {
    const void* draft;
    int dtype, B, K, V;
    const int32_t* tokens;
    int budget;
    Fanout fanout;
    int32_t* out_cache;
};

struct LookupArgs {
    int mode;
    const int32_t* cache;
    int K, B, budget, kappa, gamma;
    Fanout fanout;
    const int32_t* k;
    const int32_t* tstar;
    int32_t* out_slot;
    uint8_t* out_hit;
    int32_t* out_batch;
};

__global__ void generic_unit_kernel(VerifyArgs a);
__global__ void finalize_kernel(VerifyArgs a);
__global__ void downweight_kernel(DownweightArgs a);
__global__ void cache_build_kernel(CacheArgs a);
__global__ void cache_lookup_kernel(LookupArgs a);

struct BackupArgs {
    int B;
    const uint8_t* hit;
    const int32_t* batch;
    int b_star;
    int32_t* out_use_backup;
    int32_t* out_switch;
};
__global__ void backup_plan_kernel(BackupArgs a);

}  // namespace sv
