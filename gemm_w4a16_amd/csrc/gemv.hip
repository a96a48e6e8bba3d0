// gemv.hip -- the Q4 block-32 GEMV (thuongvuho.com "Why My 4-Bit CUDA Kernel Wasn't Faster":
// 16 code bytes + one fp16 scale per 32 weights, fp16 activations).
//
// It uses the per-block factored form (scale applied once per block after an unscaled dot, as
// that page and anrans "Quantization and GEMV", exercise 1, do) and the register dequant of
// anrans "W4A16: dequantizing in registers", reorganised for CDNA4:
//
//  * Nibbles become bf16/fp16 numbers with one AND-OR each pair: (w >> 4j) & 0x000F000F with
//    exponent bits 0x4300 (bf16) or 0x6400 (fp16) OR-ed in is the pair (B + q_j, B + q_{j+4})
//    with B = 128 or 1024 (the magic-number trick both pages describe).  v_dot2c_f32_{bf16,f16}
//    then multiplies two weights per instruction with fp32 accumulation.  The activations are
//    paired the same way, (x_j, x_{j+4}), so no nibble has to move.
//  * The offset B and the bias 8 are removed once per block: s * (sum(x*(B+q)) - (B+8)*sum(x)).
//
// Layout: codes are [N][K/32][16] bytes (a row's blocks contiguous), so 16 lanes read 512 B
// of one row per pair of 16-byte loads (256 contiguous bytes each) and a wave covers 4 rows per
// step.  Each lane always handles the same two blocks (64 k) of the row, so its activations
// are loaded once, kept in VGPRs already
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
// Q4 block-32: 1024 threads = 16 waves = 16 K-slices of 1024 k; 64 rows per block.
// ---------------------------------------------------------------------------------------------
constexpr int kQ4Waves = 16;
constexpr int kQ4Rows = 64;               // rows per block
constexpr int kQ4Steps = kQ4Rows / 4;      // a wave step covers 4 rows
constexpr int kQ4Pair = 4;                 // row steps whose loads are in flight together

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
        // this lane's two blocks, 16 apart: each load instruction of a row's 16 lanes then reads
        // 256 contiguous bytes (whole cache lines) rather than every other 16 bytes of 512
        const int b0 = slice * 32 + sub, b1 = b0 + 16;
        const bool has0 = b0 < B, has1 = b1 < B;
        // A block past the row's end is read at a clamped index and its contribution dropped by a
        // select after the load: no load sits under a branch (a branch would make every load
        // wait for all earlier ones).
        const int bb0 = min(b0, B - 1), bb1 = min(b1, B - 1);
        // activations of the two blocks, paired (x_j, x_{j+4}) per 8 k, and their sums
        uint32_t xq[2][16];
        float cst[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bool has = h ? has1 : has0;
            const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(x + (size_t)(h ? bb1 : bb0) * 32);
            float sum = 0.0f;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const u32x4_t xl = xr[d];
                const uint4 xv = has ? make_uint4(xl[0], xl[1], xl[2], xl[3]) : make_uint4(0, 0, 0, 0);
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
        // Row steps of 4 rows, kQ4Pair at a time: all their loads are issued, then the rows are
        // computed in order as their data arrives.
        struct Rows {
            u32x4_t c[kQ4Pair][2];
            uint32_t s[kQ4Pair][2];
        };
        auto load = [&](int t0, Rows& R) {
#pragma unroll
            for (int u = 0; u < kQ4Pair; ++u) {
                int n = n0 + 4 * (t0 + u) + rsub;
                n = n < N ? n : N - 1;
                const u32x4_t* cr = reinterpret_cast<const u32x4_t*>(codes) + (size_t)n * B;  // 16 B per block
                R.c[u][0] = cr[bb0];
                R.c[u][1] = cr[bb1];
                const uint32_t s0 = scales[(size_t)n * B + bb0], s1 = scales[(size_t)n * B + bb1];
                R.s[u][0] = has0 ? s0 : 0u;  // fp16 +0: the block contributes nothing
                R.s[u][1] = has1 ? s1 : 0u;
            }
        };
        auto compute = [&](int t0, const Rows& R) {
#pragma unroll
            for (int u = 0; u < kQ4Pair; ++u) {
                float part_row = 0.0f;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    float acc = cst[h];
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t p = ((R.c[u][h][d] >> (4 * e)) & kNibblePairMask) | magic;
                            acc = kF16 ? dot2_f16(p, xq[h][4 * d + e], acc) : dot2_bf16(p, xq[h][4 * d + e], acc);
                        }
                    }
                    part_row = __builtin_fmaf(f16_bits_to_f32(R.s[u][h]), acc, part_row);
                }
                // the 16 lanes of a row -> one value, added to this wave's slot for the row
                const float v = row16_sum(part_row);
                if (sub == 15) part[wave][4 * (t0 + u) + rsub] += v;
            }
        };
#pragma unroll 1
        for (int t0 = 0; t0 < kQ4Steps; t0 += kQ4Pair) {
            Rows r;
            load(t0, r);
            compute(t0, r);
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
