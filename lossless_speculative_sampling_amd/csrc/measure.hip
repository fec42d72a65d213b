// Streaming-read ceiling: a plain read of a device buffer of the size one verification call
// reads, as the measured bandwidth the call's own rate is set against (next to the HBM spec
// peak).  Every 16-byte word is loaded once, non-temporally (the data is not reused), four
// loads in flight per thread; one word is stored only if the xor of everything read equals a
// value the caller never supplies, so nothing is written in practice.
#include "common.h"

namespace sv {

typedef uint32_t u32x4m __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadInFlight = 4;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4m* __restrict__ p, size_t n16,
                                                                   uint32_t* __restrict__ sink) {
    uint32_t acc = 0u;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (kReadInFlight - 1) * stride < n16; i += kReadInFlight * stride) {
        u32x4m v[kReadInFlight];
#pragma unroll
        for (int l = 0; l < kReadInFlight; ++l) v[l] = __builtin_nontemporal_load(p + i + l * stride);
#pragma unroll
        for (int l = 0; l < kReadInFlight; ++l) acc ^= v[l][0] ^ v[l][1] ^ v[l][2] ^ v[l][3];
    }
    for (; i < n16; i += stride) {
        const u32x4m v = __builtin_nontemporal_load(p + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace sv

extern "C" int spec_read_ceiling(const void* data, size_t bytes, uint32_t* sink, hipStream_t stream) {
    if (!data || !sink || bytes == 0 || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(data) & 15)) return SPEC_EINVAL;
    const size_t n16 = bytes / 16;
    // eight workgroups per compute unit, fewer for small buffers
    const size_t per_wg = (size_t)sv::kReadThreads * sv::kReadInFlight;
    const size_t want = (n16 + per_wg - 1) / per_wg;
    const unsigned grid = (unsigned)(want < 2048 ? (want > 0 ? want : 1) : 2048);
    hipLaunchKernelGGL(sv::stream_read_kernel, dim3(grid), dim3(sv::kReadThreads), 0, stream,
                       static_cast<const sv::u32x4m*>(data), n16, sink);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}
