// gemm.hip -- large-M W4A16 GEMM on bf16 MFMA (the compute-bound path).
//
// vidyal.ai "Low-Precision Kernels", Step 2 builds the B tile of a tiled matmul from packed
// integers (shift/mask, then q * scale + min in fp32 rounded to bf16) and feeds it to the
// tensor-core dot with fp32 accumulation; BF16 weights never reach memory.  Here that becomes:
//
//  * block tile 128 (M) x 128 (N) x 64 (K), 256 threads = 4 waves in a 2 x 2 grid, each wave a
//    64 x 64 sub-tile of 4 x 4 v_mfma_f32_16x16x32_bf16 accumulators;
//  * global -> registers for tile k+1 while the MFMAs of tile k run (one LDS buffer);
//  * the packed B tile (8 packed rows x 128 columns = 4 KB) is dequantized by the threads that
//    load it -- each 32-bit word becomes the 8 bf16 weights k = 8r..8r+7 of one column, written
//    to LDS as one 16-byte row segment of an [n][k] tile, which is exactly an MFMA B fragment;
//  * w_hat = bf16_rne(fmaf(q, s, min)), the same value as the reference dequant;
//  * a K split (when the tile grid alone cannot fill 256 CUs) writes fp32 partials to the
//    caller's workspace and a second kernel adds them in split order, so the result does not
//    depend on scheduling.
#include "device_common.h"
#include "launch.h"

namespace w4a16 {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDT = BK + 8;  // LDS row pitch in bf16: 144 B, conflict-free 16-byte fragment reads
constexpr int kThreads = 256;
constexpr int kCUs = 256;

struct TileRegs {
    uint4 a[4];    // A: 4 x 16 B (8 bf16 each)
    uint4 b;       // B: 4 packed words = 4 adjacent columns of one packed row
    uint2 s, m;    // 4 bf16 scales / minimums of those columns
};

template <bool kVecN>
__device__ __forceinline__ void load_tile(TileRegs& r, const uint16_t* __restrict__ x, const uint32_t* __restrict__ codes,
                                          const uint16_t* __restrict__ scales, const uint16_t* __restrict__ mins,
                                          int M, int N, int K, int m0, int n0, int k0) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = t + kThreads * i;  // 0..1023: (row, 16-byte chunk) of the 128 x 64 A tile
        const int row = idx >> 3, chunk = idx & 7;
        const int gm = m0 + row;
        r.a[i] = gm < M ? *reinterpret_cast<const uint4*>(x + (size_t)gm * K + k0 + chunk * 8) : make_uint4(0, 0, 0, 0);
    }
    const int prow = t >> 5, c4 = (t & 31) * 4;  // packed row 0..7 of the tile, first of 4 columns
    const size_t rowoff = (size_t)(k0 / 8 + prow) * N;
    const size_t goff = (size_t)(k0 / 128) * N;
    const int gn = n0 + c4;
    if (kVecN && gn + 3 < N) {
        r.b = *reinterpret_cast<const uint4*>(codes + rowoff + gn);
        r.s = *reinterpret_cast<const uint2*>(scales + goff + gn);
        r.m = *reinterpret_cast<const uint2*>(mins + goff + gn);
    } else {
        uint32_t w[4], s[4], m[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = gn + i < N ? gn + i : N - 1;
            w[i] = codes[rowoff + c];
            s[i] = scales[goff + c];
            m[i] = mins[goff + c];
        }
        r.b = make_uint4(w[0], w[1], w[2], w[3]);
        r.s = make_uint2(s[0] | (s[1] << 16), s[2] | (s[3] << 16));
        r.m = make_uint2(m[0] | (m[1] << 16), m[2] | (m[3] << 16));
    }
}

__device__ __forceinline__ void store_tile(const TileRegs& r, uint16_t* As, uint16_t* Bs) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = t + kThreads * i;
        const int row = idx >> 3, chunk = idx & 7;
        *reinterpret_cast<uint4*>(As + row * LDT + chunk * 8) = r.a[i];
    }
    const int prow = t >> 5, c4 = (t & 31) * 4;
    const uint32_t words[4] = {r.b.x, r.b.y, r.b.z, r.b.w};
    const uint32_t sv[4] = {r.s.x & 0xFFFFu, r.s.x >> 16, r.s.y & 0xFFFFu, r.s.y >> 16};
    const uint32_t mv[4] = {r.m.x & 0xFFFFu, r.m.x >> 16, r.m.y & 0xFFFFu, r.m.y >> 16};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float s = bf16_bits_to_f32(sv[i]), m = bf16_bits_to_f32(mv[i]);
        const uint32_t w = words[i];
        const uint32_t ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;  // q0 q2 q4 q6 / q1 q3 q5 q7
        float v[8];
        v[0] = __builtin_fmaf((float)(ev & 0xFF), s, m);
        v[2] = __builtin_fmaf((float)((ev >> 8) & 0xFF), s, m);
        v[4] = __builtin_fmaf((float)((ev >> 16) & 0xFF), s, m);
        v[6] = __builtin_fmaf((float)(ev >> 24), s, m);
        v[1] = __builtin_fmaf((float)(od & 0xFF), s, m);
        v[3] = __builtin_fmaf((float)((od >> 8) & 0xFF), s, m);
        v[5] = __builtin_fmaf((float)((od >> 16) & 0xFF), s, m);
        v[7] = __builtin_fmaf((float)(od >> 24), s, m);
        const uint4 packed = make_uint4(pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3]), pack2_bf16(v[4], v[5]),
                                        pack2_bf16(v[6], v[7]));
        *reinterpret_cast<uint4*>(Bs + (c4 + i) * LDT + prow * 8) = packed;
    }
}

template <bool kVecN>
__global__ __launch_bounds__(kThreads) void gemm_g128_kernel(const uint16_t* __restrict__ x,
                                                             const uint32_t* __restrict__ codes,
                                                             const uint16_t* __restrict__ scales,
                                                             const uint16_t* __restrict__ mins,
                                                             uint16_t* __restrict__ y, float* __restrict__ ws,
                                                             int M, int N, int K, int k_per_split) {
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDT];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDT];
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int kbeg = blockIdx.z * k_per_split;
    const int kend = min(K, kbeg + k_per_split);
    const int lane = lane_id(), wave = wave_id();
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 15, lk = (lane >> 4) * 8;

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    TileRegs regs;
    load_tile<kVecN>(regs, x, codes, scales, mins, M, N, K, m0, n0, kbeg);
    for (int k0 = kbeg; k0 < kend; k0 += BK) {
        __syncthreads();  // the previous tile's fragments have been read
        store_tile(regs, As, Bs);
        __syncthreads();
        if (k0 + BK < kend) load_tile<kVecN>(regs, x, codes, scales, mins, M, N, K, m0, n0, k0 + BK);
#pragma unroll
        for (int ks = 0; ks < BK; ks += 32) {
            bf16x8_t af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = __builtin_bit_cast(bf16x8_t,
                                           *reinterpret_cast<const uint4*>(As + (wm * 64 + i * 16 + lr) * LDT + ks + lk));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bfr[j] = __builtin_bit_cast(bf16x8_t,
                                            *reinterpret_cast<const uint4*>(Bs + (wn * 64 + j * 16 + lr) * LDT + ks + lk));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }
    // D fragment: lane holds rows 4*(lane/16) + e, column lane % 16 of each 16 x 16 tile.
    const bool split = gridDim.z > 1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn * 64 + j * 16 + lr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + e;
                if (row < M && col < N) {
                    if (split)
                        ws[((size_t)blockIdx.z * M + row) * N + col] = acc[i][j][e];
                    else
                        y[(size_t)row * N + col] = f32_to_bf16_bits(acc[i][j][e]);
                }
            }
        }
}

// y = bf16(sum over splits, in split order) of the fp32 partials.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, uint16_t* __restrict__ y,
                                                            int64_t MN, int splits) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= MN) return;
    float s = ws[i];
    for (int z = 1; z < splits; ++z) s += ws[(size_t)z * MN + i];
    y[i] = f32_to_bf16_bits(s);
}

struct Plan {
    int tiles_m, tiles_n, splits, k_per_split;
};

Plan plan_gemm(int64_t M, int64_t N, int64_t K) {
    Plan p;
    p.tiles_m = (int)((M + BM - 1) / BM);
    p.tiles_n = (int)((N + BN - 1) / BN);
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    const int groups = (int)(K / 128);
    int splits = 1;
    if (tiles < kCUs) splits = (int)std::min<int64_t>(groups, (kCUs + tiles - 1) / tiles);
    // k per split in whole groups; recompute the split count so no split is empty
    const int groups_per_split = (groups + splits - 1) / splits;
    p.k_per_split = groups_per_split * 128;
    p.splits = (groups + groups_per_split - 1) / groups_per_split;
    return p;
}

}  // namespace

size_t gemm_g128_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const Plan p = plan_gemm(M, N, K);
    return p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemm_g128(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                            const uint16_t* mins, int64_t N, int64_t K, uint16_t* y, float* workspace,
                            hipStream_t stream) {
    const Plan p = plan_gemm(M, N, K);
    const dim3 grid((unsigned)p.tiles_n, (unsigned)p.tiles_m, (unsigned)p.splits);
    if (N % 4 == 0)
        hipLaunchKernelGGL(gemm_g128_kernel<true>, grid, dim3(kThreads), 0, stream, x, codes, scales, mins, y,
                           workspace, (int)M, (int)N, (int)K, p.k_per_split);
    else
        hipLaunchKernelGGL(gemm_g128_kernel<false>, grid, dim3(kThreads), 0, stream, x, codes, scales, mins, y,
                           workspace, (int)M, (int)N, (int)K, p.k_per_split);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    const int64_t MN = M * N;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, stream, workspace, y,
                       MN, p.splits);
    return hipGetLastError();
}

}  // namespace w4a16
