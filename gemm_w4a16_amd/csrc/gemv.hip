// gemv.hip -- small-M W4A16 kernels: the memory-bound path.
//
// Both kernels use the factored per-group form of vidyal.ai "Low-Precision Kernels" ("How the
// measurements were taken": for one row, s * sum(x*q) + min * sum(x) per group in FP32, no
// matrix cores) and the register dequant of anrans "Quantization and GEMV" ("W4A16:
// dequantizing in registers"), reorganised for CDNA4:
//
//  * Nibbles become bf16/fp16 numbers with one AND-OR each pair: (w >> 4j) & 0x000F000F with
//    exponent bits 0x4300 (bf16) or 0x6400 (fp16) OR-ed in is the pair (B + q_j, B + q_{j+4})
//    with B = 128 or 1024 (the magic-number trick both pages describe).  v_dot2c_f32_{bf16,f16}
//    then multiplies two weights per instruction with fp32 accumulation.  The activations are
//    paired the same way, (x_j, x_{j+4}), so no nibble has to move.
//  * The offset B is removed once per group: s*sum(x*(B+q)) + (min - B*s)*sum(x).
//
// G128 kernel: the packed matrix is [K/8][N] (N contiguous), so a wave reads one packed row of
// 64 consecutive columns per load (256 B, coalesced); the eight k of that row are the same for
// every lane, so x comes through the scalar cache into SGPRs.  A 512-thread block owns 64
// columns; its 8 waves split K by groups and add their partial sums through LDS in a fixed
// order.  All of a wave's loads (up to 4 groups = 64 words per lane) are issued before any math.
//
// Q4 kernel: codes are [N][K/32][16] bytes (a row's blocks contiguous), so 16 lanes read 512 B
// of one row per pair of 16-byte loads and a wave covers 4 rows per step.  Each lane always
// handles the same 64 k of the row, so its activations are loaded once, kept in VGPRs already
// paired, and their per-block sums folded into a constant.  The 16 lanes of a row finish with a
// DPP row reduction; the 16 waves of a 1024-thread block own 16 K-slices and add in LDS.
#include "device_common.h"
#include "launch.h"

namespace w4a16 {

namespace {

constexpr uint32_t kNibblePairMask = 0x000F000Fu;
constexpr uint32_t kBf16Magic = 0x43004300u;  // bf16 128.0 in both halves
constexpr uint32_t kF16Magic = 0x64006400u;   // fp16 1024.0 in both halves
constexpr uint32_t kBf16OnePair = 0x3F803F80u;
constexpr uint32_t kF16OnePair = 0x3C003C00u;

// (lo half of a, lo half of b) and (hi half of a, hi half of b) as one dword each.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// ---------------------------------------------------------------------------------------------
// G128: 512 threads, 64 columns per block, groups strided over the 8 waves.
// ---------------------------------------------------------------------------------------------
constexpr int kG128Waves = 8;
constexpr int kG128GroupsPerPass = 4;  // per wave: 4 x 16 packed rows in flight

template <int MR>
__global__ __launch_bounds__(512) void gemv_g128_kernel(const uint16_t* __restrict__ x,
                                                        const uint32_t* __restrict__ codes,
                                                        const uint16_t* __restrict__ scales,
                                                        const uint16_t* __restrict__ mins,
                                                        uint16_t* __restrict__ y, int M, int N, int K) {
    __shared__ float part[kG128Waves][MR][64];
    const int lane = lane_id(), wave = wave_id();
    const int n = blockIdx.x * 64 + lane;
    const int nc = n < N ? n : N - 1;  // dead lanes read a valid column and never store
    const int G = K >> 7;
    float yacc[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) yacc[m] = 0.0f;

    for (int g0 = wave; g0 < G; g0 += kG128Waves * kG128GroupsPerPass) {
        // 1) per-group activation sums first: one dword of x per lane per (group, row), summed
        //    across the wave with DPP (their loads are the oldest, so they are waited for first).
        float sx[kG128GroupsPerPass][MR];
        uint32_t xp[kG128GroupsPerPass][MR];
#pragma unroll
        for (int j = 0; j < kG128GroupsPerPass; ++j) {
            const int g = g0 + kG128Waves * j;
#pragma unroll
            for (int m = 0; m < MR; ++m)
                xp[j][m] = (g < G && m < M)
                               ? reinterpret_cast<const uint32_t*>(x + (size_t)m * K + (size_t)g * 128)[lane]
                               : 0u;
        }
        // 2) all packed words and group parameters of this pass.
        uint32_t w[kG128GroupsPerPass][16];
        uint32_t sb[kG128GroupsPerPass], mb[kG128GroupsPerPass];
#pragma unroll
        for (int j = 0; j < kG128GroupsPerPass; ++j) {
            const int g = g0 + kG128Waves * j;
            if (g < G) {
                const uint32_t* col = codes + (size_t)g * 16 * N + nc;
#pragma unroll
                for (int i = 0; i < 16; ++i) w[j][i] = col[(size_t)i * N];
                sb[j] = scales[(size_t)g * N + nc];
                mb[j] = mins[(size_t)g * N + nc];
            }
        }
#pragma unroll
        for (int j = 0; j < kG128GroupsPerPass; ++j)
#pragma unroll
            for (int m = 0; m < MR; ++m) sx[j][m] = wave_sum(dot2_bf16(xp[j][m], kBf16OnePair, 0.0f));
        // 3) dot products, one group at a time as its words arrive.
#pragma unroll
        for (int j = 0; j < kG128GroupsPerPass; ++j) {
            const int g = g0 + kG128Waves * j;
            if (g >= G) break;
            const float s = bf16_bits_to_f32(sb[j]);
            const float c = __builtin_fmaf(-128.0f, s, bf16_bits_to_f32(mb[j]));  // min - 128 s
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                if (m >= M) break;
                const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)m * K + (size_t)g * 128);
                float acc = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const uint4 xv = xr[i];  // x[8i .. 8i+7], the same for every lane
                    const uint32_t x04 = pack_lo(xv.x, xv.z), x15 = pack_hi(xv.x, xv.z);
                    const uint32_t x26 = pack_lo(xv.y, xv.w), x37 = pack_hi(xv.y, xv.w);
                    const uint32_t wd = w[j][i];
                    acc = dot2_bf16((wd & kNibblePairMask) | kBf16Magic, x04, acc);
                    acc = dot2_bf16(((wd >> 4) & kNibblePairMask) | kBf16Magic, x15, acc);
                    acc = dot2_bf16(((wd >> 8) & kNibblePairMask) | kBf16Magic, x26, acc);
                    acc = dot2_bf16(((wd >> 12) & kNibblePairMask) | kBf16Magic, x37, acc);
                }
                yacc[m] = __builtin_fmaf(s, acc, yacc[m]);
                yacc[m] = __builtin_fmaf(c, sx[j][m], yacc[m]);
            }
        }
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) part[wave][m][lane] = yacc[m];
    __syncthreads();
    const int t = threadIdx.x;
    if (t < MR * 64) {
        const int m = t >> 6, l = t & 63;
        const int col = blockIdx.x * 64 + l;
        if (m < M && col < N) {
            float sum = 0.0f;
#pragma unroll
            for (int v = 0; v < kG128Waves; ++v) sum += part[v][m][l];
            y[(size_t)m * N + col] = f32_to_bf16_bits(sum);
        }
    }
}

// ---------------------------------------------------------------------------------------------
// Q4 block-32: 1024 threads = 16 waves = 16 K-slices of 1024 k; 64 rows per block.
// ---------------------------------------------------------------------------------------------
constexpr int kQ4Waves = 16;
constexpr int kQ4Rows = 64;   // rows per block = 16 steps x 4 rows
constexpr int kQ4Unroll = 4;  // row steps whose loads are in flight together

template <bool kF16>
__global__ __launch_bounds__(1024) void gemv_q4b32_kernel(const uint16_t* __restrict__ x,
                                                          const uint32_t* __restrict__ codes,
                                                          const uint16_t* __restrict__ scales,
                                                          uint16_t* __restrict__ y, int N, int K) {
    __shared__ float part[kQ4Waves][kQ4Rows];
    const int lane = lane_id(), wave = wave_id();
    const int sub = lane & 15;   // position along k inside the slice
    const int rsub = lane >> 4;  // which of the 4 rows of a step
    const int B = K >> 5;        // blocks per row
    const int n0 = blockIdx.x * kQ4Rows;
    const uint32_t magic = kF16 ? kF16Magic : kBf16Magic;
    const float offset = kF16 ? 1032.0f : 136.0f;  // B + 8: (q - 8) = (B + q) - (B + 8)

    // Per-row partial of this wave; each K-slice a wave owns adds into its own LDS slot.
    for (int t = threadIdx.x & 63; t < kQ4Rows; t += 64) part[wave][t] = 0.0f;

    for (int slice = wave; slice * 32 < B; slice += kQ4Waves) {
        const int b0 = slice * 32 + sub * 2;  // this lane's two blocks
        const bool has0 = b0 < B, has1 = b0 + 1 < B;
        // activations of the two blocks, paired (x_j, x_{j+4}) per 8 k, and their sums
        uint32_t xq[2][16];
        float cst[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bool has = h ? has1 : has0;
            const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)(b0 + h) * 32);
            float sum = 0.0f;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint4 xv = has ? xr[d] : make_uint4(0, 0, 0, 0);
                xq[h][4 * d + 0] = pack_lo(xv.x, xv.z);
                xq[h][4 * d + 1] = pack_hi(xv.x, xv.z);
                xq[h][4 * d + 2] = pack_lo(xv.y, xv.w);
                xq[h][4 * d + 3] = pack_hi(xv.y, xv.w);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sum = kF16 ? dot2_f16(xq[h][4 * d + e], kF16OnePair, sum)
                               : dot2_bf16(xq[h][4 * d + e], kBf16OnePair, sum);
            }
            cst[h] = -offset * sum;
        }
#pragma unroll 1
        for (int t0 = 0; t0 < kQ4Rows / 4; t0 += kQ4Unroll) {
            uint4 cw[kQ4Unroll][2];
            uint32_t sc[kQ4Unroll][2];
#pragma unroll
            for (int u = 0; u < kQ4Unroll; ++u) {
                int n = n0 + 4 * (t0 + u) + rsub;
                n = n < N ? n : N - 1;
                const uint4* cr = reinterpret_cast<const uint4*>(codes) + (size_t)n * B;  // 16 B per block
                cw[u][0] = has0 ? cr[b0] : make_uint4(0, 0, 0, 0);
                cw[u][1] = has1 ? cr[b0 + 1] : make_uint4(0, 0, 0, 0);
                sc[u][0] = has0 ? scales[(size_t)n * B + b0] : 0u;
                sc[u][1] = has1 ? scales[(size_t)n * B + b0 + 1] : 0u;
            }
#pragma unroll
            for (int u = 0; u < kQ4Unroll; ++u) {
                float part_row = 0.0f;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t wd[4] = {cw[u][h].x, cw[u][h].y, cw[u][h].z, cw[u][h].w};
                    float acc = cst[h];
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t p = ((wd[d] >> (4 * e)) & kNibblePairMask) | magic;
                            acc = kF16 ? dot2_f16(p, xq[h][4 * d + e], acc) : dot2_bf16(p, xq[h][4 * d + e], acc);
                        }
                    }
                    part_row = __builtin_fmaf(f16_bits_to_f32(sc[u][h]), acc, part_row);
                }
                // the 16 lanes of a row -> one value, added to this wave's slot for the row
                const float v = row16_sum(part_row);
                if (sub == 15) part[wave][4 * (t0 + u) + rsub] += v;
            }
        }
    }
    // the 16 K-slices of each row, added through LDS in a fixed order
    __syncthreads();
    const int t = threadIdx.x;
    if (t < kQ4Rows && n0 + t < N) {
        float sum = 0.0f;
#pragma unroll
        for (int v = 0; v < kQ4Waves; ++v) sum += part[v][t];
        y[n0 + t] = kF16 ? f32_to_f16_bits(sum) : f32_to_bf16_bits(sum);
    }
}

}  // namespace

hipError_t launch_gemv_g128(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                            const uint16_t* mins, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
    const dim3 grid((unsigned)((N + 63) / 64)), block(512);
    const int m = (int)M, n = (int)N, k = (int)K;
    if (M == 1)
        hipLaunchKernelGGL(gemv_g128_kernel<1>, grid, block, 0, stream, x, codes, scales, mins, y, m, n, k);
    else if (M == 2)
        hipLaunchKernelGGL(gemv_g128_kernel<2>, grid, block, 0, stream, x, codes, scales, mins, y, m, n, k);
    else
        hipLaunchKernelGGL(gemv_g128_kernel<4>, grid, block, 0, stream, x, codes, scales, mins, y, m, n, k);
    return hipGetLastError();
}

hipError_t launch_gemv_q4b32(const uint16_t* x, int64_t M, bool act_f16, const uint8_t* codes,
                             const uint16_t* scales, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
    const dim3 grid((unsigned)((N + kQ4Rows - 1) / kQ4Rows)), block(1024);
    for (int64_t m = 0; m < M; ++m) {  // one pass per activation row
        const uint16_t* xm = x + m * K;
        uint16_t* ym = y + m * N;
        if (act_f16)
            hipLaunchKernelGGL(gemv_q4b32_kernel<true>, grid, block, 0, stream, xm,
                               reinterpret_cast<const uint32_t*>(codes), scales, ym, (int)N, (int)K);
        else
            hipLaunchKernelGGL(gemv_q4b32_kernel<false>, grid, block, 0, stream, xm,
                               reinterpret_cast<const uint32_t*>(codes), scales, ym, (int)N, (int)K);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace w4a16
