// roof.hip -- measured roofs for the benchmark (libw4a16_roof.so; not part of libw4a16 and not
// declared in include/w4a16.h).
//
// The pages quote every kernel time beside what the same GPU does with no arithmetic at all:
// vidyal.ai "Low-Precision Kernels", "How the measurements were taken" (a plain read kernel's
// bandwidth as the measured roof) and thuongvuho.com "Why My 4-Bit CUDA Kernel Wasn't Faster",
// "I finally got results" (a device-to-device copy).  These are the MI355X counterparts:
//  * roof_read: a streaming read of `nbytes` with 16-byte non-temporal loads, each wave load one
//    contiguous KiB, UNROLL loads in flight per lane before any use; the bytes are folded into a
//    value that is stored only if it equals a constant no realistic data produces, so the loads
//    cannot be removed and nothing is written;
//  * roof_empty: a launch that does nothing, the fixed cost of one kernel in a graph.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
constexpr int kUnroll = 4;
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void roof_read_kernel(const u32x4_t* __restrict__ src, uint32_t n16,
                                                             uint32_t* __restrict__ sink) {
    const uint32_t tid = blockIdx.x * kThreads + threadIdx.x;
    const uint32_t stride = gridDim.x * kThreads;
    uint32_t acc = 0;
    for (uint32_t i0 = tid; i0 < n16; i0 += stride * kUnroll) {
        u32x4_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t i = min(i0 + (uint32_t)u * stride, n16 - 1);  // a clamped duplicate is harmless
            v[u] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

__global__ void roof_empty_kernel() {}

}  // namespace

extern "C" {

// Blocks for one pass over the buffer (each lane reads kUnroll chunks), or `blocks` if > 0.
// nbytes: a multiple of 16 below 2^36; src 16-byte aligned; sink: 256 uint32 of device memory.
int roof_read(const void* src, size_t nbytes, uint32_t* sink, int blocks, hipStream_t stream) {
    if (src == nullptr || sink == nullptr || nbytes == 0 || nbytes % 16 != 0 || nbytes / 16 >= ((size_t)1 << 32))
        return 1;
    const uint32_t n16 = (uint32_t)(nbytes / 16);
    if (blocks <= 0) blocks = (int)((n16 + kThreads * kUnroll - 1) / (kThreads * kUnroll));
    hipLaunchKernelGGL(roof_read_kernel, dim3(blocks), dim3(kThreads), 0, stream, static_cast<const u32x4_t*>(src), n16,
                       sink);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

int roof_empty(hipStream_t stream) {
    hipLaunchKernelGGL(roof_empty_kernel, dim3(1), dim3(64), 0, stream);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
