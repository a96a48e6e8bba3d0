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
//    x 256 B.  It measures what a CU's loads of shared data sustain in each shape.  Patterns 4
//    and 5 read as pattern 0 but with direct-to-LDS copies (global_load_lds_dwordx4, into a
//    per-wave LDS ring), 4 or 8 of them in flight per wave, as the mid-M kernels stage operands;
//    6 and 7 copy 2 rows x 512 B per wave load, 7 with the 16-byte chunks of each row read in the
//    order chunk ^ (row % 16) (an XOR swizzle of the LDS image, as the 64-row kernel's x copies);
//  * roof_copy_pipeline: the operand copies of a 64-row factored kernel alone, no arithmetic: one
//    block of 8 waves per 64 columns of the G128 weights, one group of 128 k per LDS stage, seven
//    stages, the copies six groups ahead and one barrier per group; per group and block 16 KB of
//    a shared 64-row x (4 rows x 256 B per copy, from L2) and the 4 KB of packed rows and 256 B of
//    parameters (from HBM).  Modes: 0 -- x only; 1 -- words and parameters only; 2 -- both, every
//    wave copying some of each; 3 -- both, waves 0..3 copying the weights and 4..7 x, so that no
//    wave's counter waits on the other stream.  It measures whether a CU overlaps its reads of L2
//    (x) with its reads of HBM (the weights).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lds_dma.h"

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

// Wave load i of the copy patterns: 0 -- 1 KB of one row; 1 -- 2 rows x 512 B; 2 -- the same,
// chunk c of row r read from chunk c ^ (r % 16).  rowb = K * 2.
template <int kShape>
__device__ __forceinline__ uint32_t copy_offset(uint32_t i, uint32_t lane, uint32_t rowb) {
    if constexpr (kShape == 0) {
        return i * 1024u + lane * 16u;
    } else {
        const uint32_t per = rowb / 512u, rp = i / per, seg = i % per;  // row pairs, 512-byte segments
        const uint32_t r = rp * 2u + (lane >> 5), c = lane & 31u;
        return r * rowb + seg * 512u + (kShape == 2 ? (c ^ (r & 15u)) : c) * 16u;
    }
}

// The copy patterns as direct-to-LDS copies: wave w copies its wave loads into LDS slots
// (w * kU + u) KiB, kU in flight, then waits for them all before the next kU.
template <int kU, int kShape>
__global__ __launch_bounds__(kSharedThreads) void roof_shared_dma_kernel(const char* __restrict__ x, uint32_t rowb,
                                                                          uint32_t ninst) {
    __shared__ __attribute__((aligned(16))) char ring[(kSharedThreads / 64) * kU * 1024];
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t base = w4a16::lds_addr(ring) + wave * kU * 1024u;
    for (uint32_t i0 = wave; i0 < ninst; i0 += (kSharedThreads / 64) * kU) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const uint32_t i = min(i0 + (uint32_t)u * (kSharedThreads / 64), ninst - 1);
            w4a16::dma16(copy_offset<kShape>(i, lane, rowb), x, base + (uint32_t)u * 1024u);
        }
        w4a16::wait_vm<0>();
    }
}

// A direct-to-LDS copy of the weights with cache-policy bits: 0 none, 1 nt, 2 sc0 sc1, 3 sc1.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int kPol, int kImm>
__device__ __forceinline__ void dma16_pol(uint32_t voff, const void* sbase, uint32_t lds) {
    if constexpr (kPol == 0) {
        w4a16::dma16<kImm>(voff, sbase, lds);
    } else if constexpr (kPol == 1) {
        asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(lds), "n"(kImm)
                     : "memory", "m0", "scc");
    } else if constexpr (kPol == 2) {
        asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1 sc0 sc1" ::"v"(voff), "s"(sbase), "s"(lds),
                     "n"(kImm)
                     : "memory", "m0", "scc");
    } else {
        asm volatile("s_add_u32 m0, %2, %3\n\tglobal_load_lds_dwordx4 %0, %1 sc1" ::"v"(voff), "s"(sbase), "s"(lds), "n"(kImm)
                     : "memory", "m0", "scc");
    }
}
#pragma clang diagnostic pop

// roof_copy_pipeline's geometry: 64 rows, 64 columns per block, one group per stage.
constexpr int kCpRows = 64, kCpX = kCpRows * 256, kCpW = 4096, kCpS = kCpX + kCpW + 512;
constexpr int kCpStages = (160 * 1024) / kCpS;  // 7

template <int kMode, int kPol = 0>
__global__ __launch_bounds__(512) void roof_copy_pipeline_kernel(const uint16_t* __restrict__ x,
                                                                 const uint32_t* __restrict__ codes,
                                                                 const uint16_t* __restrict__ scales,
                                                                 const uint16_t* __restrict__ mins, int N, int K) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kCpStages * kCpS];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * 64, G = K / 128;
    const uint32_t sm = w4a16::lds_addr(smem);
    // copy j of a wave copying x: rows 4 c .. 4 c + 3 with c = (number of the copy in the stage),
    // lane l row 4 c + l / 16, 16-byte chunk (l % 16) ^ (row % 16) of the row's group
    constexpr bool kSplit = kMode == 3;
    constexpr int kXPerWave = kSplit ? 4 : 2;  // x copies of a wave that copies x
    uint32_t xoff[kXPerWave];
    const int xw = __builtin_amdgcn_readfirstlane(kSplit ? max(wave - 4, 0) : wave);
#pragma unroll
    for (int j = 0; j < kXPerWave; ++j) {
        const int r = 4 * (kXPerWave * xw + j) + lane / 16, p = lane % 16;
        xoff[j] = (uint32_t)((r * K + 8 * (p ^ (r & 15))) * 2);
    }
    // packed rows: split mode, wave w < 4 copies rows 4 w .. 4 w + 3 (1 KB); else lanes 0..31 of
    // wave w copy rows 2 w, 2 w + 1; lane l the 4 columns at 4 (l % 16), clamped to the last 4
    const int wrow = kSplit ? 4 * wave + lane / 16 : 2 * wave + (lane & 31) / 16;
    const uint32_t woff = (uint32_t)(((size_t)wrow * N + min(n0 + 4 * (lane & 15), N - 4)) * 4);
    const uint32_t poff = (uint32_t)(min(n0 / 2 + min(lane, 31), N / 2 - 1) * 4);
    const char* const parr = (wave & 1) ? reinterpret_cast<const char*>(mins) : reinterpret_cast<const char*>(scales);
    constexpr bool kX = kMode != 1, kW = kMode != 0;
    const bool copies_x = kX && (!kSplit || wave >= 4), copies_w = kW && (!kSplit || wave < 4);
    const bool copies_p = kW && wave < 2;
    auto issue = [&](int g, int st) {
        g = min(g, G - 1);
        const uint32_t base = sm + (uint32_t)(st * kCpS);
        if (copies_x) {
            const char* xs = reinterpret_cast<const char*>(x + (size_t)g * 128);
            const uint32_t b = base + 1024u * kXPerWave * (uint32_t)xw;
            w4a16::dma16<0>(xoff[0], xs, b);
            w4a16::dma16<1024>(xoff[1], xs, b);
            if constexpr (kXPerWave == 4) {
                w4a16::dma16<2048>(xoff[2], xs, b);
                w4a16::dma16<3072>(xoff[3], xs, b);
            }
        }
        if (copies_w) {
            if (kSplit) dma16_pol<kPol, kCpX>(woff, codes + (size_t)16 * g * N, base + 1024u * wave);
            else if (lane < 32) dma16_pol<kPol, kCpX>(woff, codes + (size_t)16 * g * N, base + 512u * wave);
        }
        if (copies_p) w4a16::dma4<kCpX + kCpW>(poff, parr + (size_t)g * N * 2, base + 256u * wave);
    };
    for (int g = 0; g < kCpStages; ++g) issue(g, g);
    // each wave waits for its copies of group g (issued kCpStages groups before it runs): the
    // copies it issues per group, times the kCpStages - 2 groups that may stay in flight
    const int per = (copies_x ? kXPerWave : 0) + (copies_w ? 1 : 0) + (copies_p ? 1 : 0);
    int st = 0;
    for (int g = 0; g < G; ++g) {
        switch (per) {
            case 0: w4a16::wait_vm<0>(); break;
            case 1: w4a16::wait_vm<(kCpStages - 2) * 1>(); break;
            case 2: w4a16::wait_vm<(kCpStages - 2) * 2>(); break;
            case 3: w4a16::wait_vm<(kCpStages - 2) * 3>(); break;
            default: w4a16::wait_vm<(kCpStages - 2) * 4>(); break;
        }
        __syncthreads();
        issue(g + kCpStages, st);
        st = st + 1 == kCpStages ? 0 : st + 1;
    }
    w4a16::wait_vm<0>();
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

// blocks blocks each read all of x [M][K] bf16 (16-byte aligned) in pattern 0..7; sink: 1024
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
        case 4: hipLaunchKernelGGL((roof_shared_dma_kernel<4, 0>), dim3(blocks), dim3(kSharedThreads), 0, stream, xc, rowb, ninst); break;
        case 5: hipLaunchKernelGGL((roof_shared_dma_kernel<8, 0>), dim3(blocks), dim3(kSharedThreads), 0, stream, xc, rowb, ninst); break;
        case 6: hipLaunchKernelGGL((roof_shared_dma_kernel<4, 1>), dim3(blocks), dim3(kSharedThreads), 0, stream, xc, rowb, ninst); break;
        case 7: hipLaunchKernelGGL((roof_shared_dma_kernel<4, 2>), dim3(blocks), dim3(kSharedThreads), 0, stream, xc, rowb, ninst); break;
        default: return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

// x: [64][K] bf16; codes, scales, mins: a G128 matrix [K/8][N], [K/128][N] x2.  N % 4 == 0,
// K % 128 == 0, 64 * K * 2 < 2^32 and (K / 8) * N * 4 < 2^32.
int roof_copy_pipeline(const void* x, const void* codes, const void* scales, const void* mins, int N, int K, int mode,
                       hipStream_t stream) {
    if (x == nullptr || codes == nullptr || scales == nullptr || mins == nullptr || N <= 0 || K <= 0 || N % 4 != 0 ||
        K % 128 != 0 || (uint64_t)kCpRows * K * 2 >= ((uint64_t)1 << 32) || (uint64_t)(K / 8) * N * 4 >= ((uint64_t)1 << 32))
        return 1;
    const dim3 grid((unsigned)((N + 63) / 64)), block(512);
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    const uint32_t* c = static_cast<const uint32_t*>(codes);
    const uint16_t* sc = static_cast<const uint16_t*>(scales);
    const uint16_t* mn = static_cast<const uint16_t*>(mins);
    switch (mode) {
        case 0: hipLaunchKernelGGL(roof_copy_pipeline_kernel<0>, grid, block, 0, stream, xs, c, sc, mn, N, K); break;
        case 1: hipLaunchKernelGGL(roof_copy_pipeline_kernel<1>, grid, block, 0, stream, xs, c, sc, mn, N, K); break;
        case 2: hipLaunchKernelGGL(roof_copy_pipeline_kernel<2>, grid, block, 0, stream, xs, c, sc, mn, N, K); break;
        case 3: hipLaunchKernelGGL(roof_copy_pipeline_kernel<3>, grid, block, 0, stream, xs, c, sc, mn, N, K); break;
        case 4: hipLaunchKernelGGL((roof_copy_pipeline_kernel<2, 1>), grid, block, 0, stream, xs, c, sc, mn, N, K); break;
        case 5: hipLaunchKernelGGL((roof_copy_pipeline_kernel<2, 2>), grid, block, 0, stream, xs, c, sc, mn, N, K); break;
        case 6: hipLaunchKernelGGL((roof_copy_pipeline_kernel<2, 3>), grid, block, 0, stream, xs, c, sc, mn, N, K); break;
        case 7: hipLaunchKernelGGL((roof_copy_pipeline_kernel<1, 1>), grid, block, 0, stream, xs, c, sc, mn, N, K); break;
        case 8: hipLaunchKernelGGL((roof_copy_pipeline_kernel<1, 2>), grid, block, 0, stream, xs, c, sc, mn, N, K); break;
        default: return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

int roof_empty(hipStream_t stream) {
    hipLaunchKernelGGL(roof_empty_kernel, dim3(1), dim3(64), 0, stream);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
