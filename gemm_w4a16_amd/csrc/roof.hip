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
//  * roof_empty: a launch that does nothing, the fixed cost of one kernel in a graph;
//  * roof_shared_read: every block reads all of one shared [M][K] bf16 matrix, as the mid-M
//    kernels read their activations (from L2 after the first block), with one of four shapes per
//    wave load: 0 -- 1 KB of one row; 1 -- 16 rows x 64 B (the A fragments of
//    v_mfma_f32_16x16x32_bf16); 2 -- 32 rows x 32 B (those of v_mfma_f32_32x32x16_bf16); 3 -- 4 rows
//    x 256 B.  It measures what a CU's loads of shared data sustain in each shape.
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

constexpr int kSharedThreads = 1024;  // 16 waves, UNROLL loads in flight per lane

// Wave load i (1 KB) of the pattern: the byte offset of this lane's 16 bytes.  rowb = K * 2.
template <int kPat>
__device__ __forceinline__ uint32_t shared_offset(uint32_t i, uint32_t lane, uint32_t rowb) {
    if constexpr (kPat == 0) {
        return i * 1024u + lane * 16u;
    } else if constexpr (kPat == 1) {
        const uint32_t per = rowb / 64u, rs = i / per, c = i % per;  // 16-row sets, 64-byte columns
        return (rs * 16u + (lane & 15u)) * rowb + c * 64u + (lane >> 4) * 16u;
    } else if constexpr (kPat == 2) {
        const uint32_t per = rowb / 32u, rs = i / per, c = i % per;
        return (rs * 32u + (lane & 31u)) * rowb + c * 32u + (lane >> 5) * 16u;
    } else {
        const uint32_t per = rowb / 256u, rs = i / per, c = i % per;
        return (rs * 4u + (lane >> 4)) * rowb + c * 256u + (lane & 15u) * 16u;
    }
}

template <int kPat>
__global__ __launch_bounds__(kSharedThreads) void roof_shared_read_kernel(const char* __restrict__ x, uint32_t rowb,
                                                                           uint32_t ninst, uint32_t* __restrict__ sink) {
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    uint32_t acc = 0;
    for (uint32_t i0 = wave; i0 < ninst; i0 += (kSharedThreads / 64) * kUnroll) {
        u32x4_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t i = min(i0 + (uint32_t)u * (kSharedThreads / 64), ninst - 1);
            v[u] = *reinterpret_cast<const u32x4_t*>(x + shared_offset<kPat>(i, lane, rowb));
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

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

// blocks blocks each read all of x [M][K] bf16 (16-byte aligned) in pattern 0..3; sink: 1024
// uint32 of device memory.  M a multiple of 32 and K of 512, M * K * 2 < 2^32.
int roof_shared_read(const void* x, int M, int K, int pattern, int blocks, uint32_t* sink, hipStream_t stream) {
    if (x == nullptr || sink == nullptr || M <= 0 || K <= 0 || M % 32 != 0 || K % 512 != 0 || blocks <= 0 ||
        (uint64_t)M * (uint64_t)K * 2u >= ((uint64_t)1 << 32))
        return 1;
    const uint32_t rowb = (uint32_t)K * 2u, ninst = (uint32_t)M * rowb / 1024u;
    const char* xc = static_cast<const char*>(x);
    switch (pattern) {
        case 0: hipLaunchKernelGGL(roof_shared_read_kernel<0>, dim3(blocks), dim3(kSharedThreads), 0, stream, xc, rowb, ninst, sink); break;
        case 1: hipLaunchKernelGGL(roof_shared_read_kernel<1>, dim3(blocks), dim3(kSharedThreads), 0, stream, xc, rowb, ninst, sink); break;
        case 2: hipLaunchKernelGGL(roof_shared_read_kernel<2>, dim3(blocks), dim3(kSharedThreads), 0, stream, xc, rowb, ninst, sink); break;
        case 3: hipLaunchKernelGGL(roof_shared_read_kernel<3>, dim3(blocks), dim3(kSharedThreads), 0, stream, xc, rowb, ninst, sink); break;
        default: return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

int roof_empty(hipStream_t stream) {
    hipLaunchKernelGGL(roof_empty_kernel, dim3(1), dim3(64), 0, stream);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
