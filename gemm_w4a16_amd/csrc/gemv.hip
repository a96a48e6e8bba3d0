// gemv.hip -- the row-major 4-bit GEMVs: the Q4 block-32 format (thuongvuho.com "Why My 4-Bit
// CUDA Kernel Wasn't Faster": 16 code bytes + one fp16 scale per 32 weights, fp16 activations) and
// the integer-zero-point format (anrans.github.io "Quantization and GEMV": words [N][K/8], an fp16
// scale and zero point per group of 128, decode (q - z) s).  Their code bytes are laid out alike,
// 16 bytes per 32 k along each row, so one kernel serves both: the zero-point form takes z * sum(x)
// off each block's dot product per row, where Q4's constant bias 8 is folded into the per-block
// constants.
//
// It uses the per-block factored form (scale applied once per block after an unscaled dot, as
// that page and anrans "Quantization and GEMV", exercise 1, do) and the register dequant of
// anrans "W4A16: dequantizing in registers", reorganised for CDNA4:
//
//  * Nibbles become fp16 numbers with one AND-OR per pair (the magic-number trick both pages
//    describe): with the exponent of 1024 OR-ed in, mask 0x000F000F turns the nibbles of k = 0
//    and 4 into 1024 + q, and mask 0x00F000F0 turns those of k = 1 and 5 into 1024 + 16q, both
//    exact in fp16; the word shifted right by 8 gives k = 2, 6 and 3, 7 the same way.  That is
//    five instructions per 8 codes.  v_dot2c_f32_f16 multiplies two weights per instruction
//    with fp32 accumulation into two sums (the 1x and the 16x nibbles), against activations
//    paired the same way, (x_j, x_{j+4}).  The offsets and the bias 8 are removed once per block:
//    sum (q - 8) x = [sum (1024 + q) x - 1032 sum x] + [sum (1024 + 16q) x - 1152 sum x] / 16.
//    (bf16 activations, accepted as an extension, use 128 + q from the low nibble of each half
//    after a shift: seven instructions per 8 codes.)
//
// Layout: codes are [N][K/32][16] bytes (a row's blocks contiguous), so 16 lanes read 512 B
// of one row per pair of 16-byte loads (256 contiguous bytes each) and a wave covers 4 rows per
// step.  Each lane always handles the same two blocks (64 k) of the row, so its activations
// are loaded once, kept in VGPRs already paired, and their per-block sums folded into
// constants.  Each wave keeps the loads of the next steps in flight while it computes one (a
// rolling window, issued before the activations are even waited for).  The 16 lanes of a row
// finish with a DPP row reduction; the 16 waves of a 1024-thread block own 16 K-slices and add
// in LDS.
#include "device_common.h"
#include "launch.h"

namespace w4a16 {

namespace {

constexpr uint32_t kNibblePairMask = 0x000F000Fu;
constexpr uint32_t kNibblePairMaskHi = 0x00F000F0u;
constexpr uint32_t kBf16Magic = 0x43004300u;  // bf16 128.0 in both halves
constexpr uint32_t kF16Magic = 0x64006400u;   // fp16 1024.0 in both halves
constexpr uint32_t kBf16OnePair = 0x3F803F80u;
constexpr uint32_t kF16OnePair = 0x3C003C00u;

// (lo half of a, lo half of b) and (hi half of a, hi half of b) as one dword each.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// ---------------------------------------------------------------------------------------------
// Row-major 4-bit GEMV: 1024 threads = 16 waves; 64 rows per block.  The 16 waves are kS K-slices
// of 32 blocks (1024 k) times 16/kS row groups: with K = 16384 all 16 waves split K and each walks
// the block's 16 row steps; with K = 4096 four waves split K and each walks 4 of the 16 steps.
// ---------------------------------------------------------------------------------------------
constexpr int kGvWaves = 16;
constexpr int kGvRows = 64;                // rows per block
constexpr int kGvSteps = kGvRows / 4;      // a wave step covers 4 rows
constexpr int kGvAhead = 2;                // row steps whose loads are in flight ahead of the math

// One row step's data for one lane: its two 16-byte code blocks, their scales and (zero-point
// format) their zero points.
struct GvStep {
    u32x4_t c[2];
    uint32_t s[2];
    uint32_t z[2];
};

// Formats of the row-major kernel.  Q4 and ZP share their code bytes (16 bytes per 32 k along
// each row); W8 has 16 bytes per 16 k (signed bytes) and one scale per row.
enum RowFmt { kRowQ4 = 0, kRowZP = 1, kRowW8 = 2 };

// Code blocks per lane and row step: two (a K-slice of 32 blocks), or one (16 blocks) where a lane
// carries two rows of 4-bit activations, whose paired fp16 values for two blocks would not fit in
// the 128 VGPRs of a 1024-thread block beside the load window.
__host__ __device__ constexpr int rowmajor_blocks_per_lane(int fmt, int mr) { return mr >= 4 || (mr == 2 && fmt != kRowW8) ? 1 : 2; }

// kF16: fp16 (else bf16) activations.  kFmt: kRowQ4 (a scale per block, decode (q - 8) s),
// kRowZP (a scale and an fp16 zero point per group of 4 blocks, decode (q - z) s) or kRowW8 (int8
// codes, one fp32 scale per row applied to the row's sum; fp16 activations only).  kMR: activation
// rows (1, 2 or 4; rows of x and y K and N elements apart) against one pass over the weights, of
// which the first `rows` are real (a row past them repeats the last one and is not stored); each
// unpacked word then feeds kMR dot products.
template <bool kF16, int kFmt, int kS, int kMR>
__global__ __launch_bounds__(1024) void gemv_rowmajor_kernel(const uint16_t* __restrict__ x,
                                                             const uint32_t* __restrict__ codes,
                                                             const uint16_t* __restrict__ scales,
                                                             const uint16_t* __restrict__ zeros,
                                                             uint16_t* __restrict__ y, int N, int K, int rows) {
    constexpr bool kZP = kFmt == kRowZP, kW8 = kFmt == kRowW8;
    static_assert(!kW8 || kF16, "int8 codes need fp16 activations (1024 + u with u < 256)");
    constexpr int kBlockK = kW8 ? 16 : 32;    // k per 16-byte block of codes
    constexpr int kXq = kBlockK / 2;          // paired activation dwords per block
    constexpr int kR = kGvWaves / kS;         // row groups
    constexpr int kMySteps = kGvSteps / kR;   // row steps per wave: rg, rg + kR, ...
    constexpr int kNB = rowmajor_blocks_per_lane(kFmt, kMR);
    constexpr int kSW = 16 * kNB;             // blocks per K-slice
    // with one block per lane a step's loads are half as large: twice as many steps in flight, but
    // for two rows only (four rows' activations leave no registers for them)
    constexpr int kAheadW = kNB == 1 && kMR <= 2 ? 2 * kGvAhead : kGvAhead;
    constexpr int kAhead = kAheadW < kMySteps ? kAheadW : kMySteps;
    __shared__ float part[kMR][kGvWaves][kGvRows];
    const int lane = lane_id(), wave = wave_id();
    const int sub = lane & 15;   // position along k inside the slice
    const int rsub = lane >> 4;  // which of the 4 rows of a step
    const int my_slice = wave % kS, rg = wave / kS;
    const int B = K / kBlockK;   // blocks per row
    const int G = K >> 7;        // groups of 128 per row (zero-point format)
    const int n0 = blockIdx.x * kGvRows;
    const bool full = n0 + kGvRows <= N;
    // this block's first row of codes (16 B per block), of scales and of zero points
    const char* cblk = reinterpret_cast<const char*>(codes) + (size_t)n0 * B * 16;
    const char* sblk = reinterpret_cast<const char*>(scales) + (size_t)n0 * (kZP ? G : B) * 2;  // (not W8)
    const char* zblk = kZP ? reinterpret_cast<const char*>(zeros) + (size_t)n0 * G * 2 : nullptr;
    // The masks in SGPRs and the exponent in a VGPR, opaque to the compiler, so that each pair is
    // one v_and_or_b32 (VOP3 takes no literal and one scalar operand on gfx9).
    uint32_t mask_lo, mask_hi, magic_v;
    asm volatile("s_mov_b32 %0, %1" : "=s"(mask_lo) : "i"(kW8 ? 0x00FF00FFu : kNibblePairMask));
    asm volatile("s_mov_b32 %0, %1" : "=s"(mask_hi) : "i"(kNibblePairMaskHi));
    asm volatile("v_mov_b32 %0, %1" : "=v"(magic_v) : "i"(kF16 ? kF16Magic : kBf16Magic));

    // Per-row partial of this wave; each K-slice a wave owns adds into its own LDS slot.
    for (int t = threadIdx.x & 63; t < kGvRows; t += 64)
#pragma unroll
        for (int m = 0; m < kMR; ++m) part[m][wave][t] = 0.0f;

    for (int slice = my_slice; slice * kSW < B; slice += kS) {
        // this lane's blocks, 16 apart: each load instruction of a row's 16 lanes then reads
        // 256 contiguous bytes (whole cache lines) rather than every other 16 bytes of 512
        const int b0 = slice * kSW + sub, b1 = b0 + 16;
        const bool has0 = b0 < B, has1 = kNB == 2 && b1 < B;
        // A block past the row's end is read at a clamped index and its contribution dropped by a
        // zero scale after the load: no load sits under a branch (a branch would make every load
        // wait for all earlier ones).
        const int bb0 = min(b0, B - 1), bb1 = min(b1, B - 1);
        // Loads address a wave-uniform base (this block's first row) plus a 32-bit lane offset;
        // rows past N (last block only) re-read row N - 1, whose result is never stored.
        auto load = [&](int t, GvStep& R) {
            uint32_t r = 4 * t + rsub;
            if (!full) r = min(r, (uint32_t)(N - 1 - n0));
            // byte offsets in 32 bits, so that each load is SGPR base + VGPR offset
            const uint32_t o0 = r * (uint32_t)B + (uint32_t)bb0, o1 = r * (uint32_t)B + (uint32_t)bb1;
            R.c[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(cblk + o0 * 16u));
            if constexpr (kNB == 2) R.c[1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(cblk + o1 * 16u));
            if constexpr (kW8) return;  // the row's scale is applied to its total
            const uint32_t p0 = kZP ? r * (uint32_t)G + (uint32_t)(bb0 >> 2) : o0;
            const uint32_t p1 = kZP ? r * (uint32_t)G + (uint32_t)(bb1 >> 2) : o1;
            const uint32_t s0 = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(sblk + p0 * 2u));
            R.s[0] = has0 ? s0 : 0u;  // fp16 +0: the block contributes nothing
            if constexpr (kNB == 2) {
                const uint32_t s1 = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(sblk + p1 * 2u));
                R.s[1] = has1 ? s1 : 0u;
            }
            if constexpr (kZP) {
                R.z[0] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(zblk + p0 * 2u));
                if constexpr (kNB == 2) R.z[1] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(zblk + p1 * 2u));
            }
        };
        // The activations of the two blocks (L2-resident, read by every block) and the first steps'
        // weight loads.  A wave's loads return in order, so where a wave has few row steps of 4-bit
        // codes the activations go first: behind the weights they held back the first step's math
        // and with it the rolling window (zero-point decode shape 8.49 -> 7.90 us).  The int8 codes
        // keep the weights first (10.63 against 10.85 us), and so do long rows (Q4 16384^2 alike
        // either way, and the activations held across the first loads spilled there).
        constexpr bool kXFirst = !kW8 && kMySteps <= 4;
        GvStep r[kMySteps];
        constexpr int kXd = kBlockK / 8;  // 16-byte activation chunks per block
        u32x4_t xraw[kMR][kNB][kXd];
        auto load_x = [&] {
#pragma unroll
            for (int m = 0; m < kMR; ++m)
#pragma unroll
                for (int h = 0; h < kNB; ++h)
#pragma unroll
                    for (int d = 0; d < kXd; ++d)
                        xraw[m][h][d] = reinterpret_cast<const u32x4_t*>(x + (size_t)min(m, rows - 1) * K +
                                                                         (size_t)(h ? bb1 : bb0) * kBlockK)[d];
        };
        if constexpr (kXFirst) {
            load_x();
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < kAhead; ++i) load(rg + kR * i, r[i]);
        if constexpr (kXFirst) __builtin_amdgcn_sched_barrier(0);
        // The activations paired per 8 k, and the per-block constants that remove the magic offset
        // (and, for Q4, the code bias; see the top of this file).
        uint32_t xq[kMR][kNB][kXq];
        float cst[kMR][kNB][2], sx[kMR][kNB];
#pragma unroll
        for (int hm = 0; hm < kNB * kMR; ++hm) {
            const int h = hm % kNB, m = hm / kNB;
            const bool has = h ? has1 : has0;
            const u32x4_t* xr =
                reinterpret_cast<const u32x4_t*>(x + (size_t)min(m, rows - 1) * K + (size_t)(h ? bb1 : bb0) * kBlockK);
            float sum_a = 0.0f, sum_b = 0.0f;
            if constexpr (kW8) {
                // per 4 k of a code dword: (x0, x2) and (x1, x3), which meet the byte pairs below
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    const u32x4_t xl = kXFirst ? xraw[m][h][d] : xr[d];
                    const uint4 xv = has ? make_uint4(xl[0], xl[1], xl[2], xl[3]) : make_uint4(0, 0, 0, 0);
                    xq[m][h][4 * d + 0] = pack_lo(xv.x, xv.y);
                    xq[m][h][4 * d + 1] = pack_hi(xv.x, xv.y);
                    xq[m][h][4 * d + 2] = pack_lo(xv.z, xv.w);
                    xq[m][h][4 * d + 3] = pack_hi(xv.z, xv.w);
#pragma unroll
                    for (int e = 0; e < 4; ++e) sum_a = dot2_f16(xq[m][h][4 * d + e], kF16OnePair, sum_a);
                }
                sx[m][h] = sum_a;
                cst[m][h][0] = -1152.0f * sum_a;  // sum (1024 + 128 + q) x - 1152 sum x = sum q x
                cst[m][h][1] = 0.0f;
                continue;
            }
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const u32x4_t xl = kXFirst ? xraw[m][h][d] : xr[d];
                const uint4 xv = has ? make_uint4(xl[0], xl[1], xl[2], xl[3]) : make_uint4(0, 0, 0, 0);
                // (x0,x4) (x1,x5) (x2,x6) (x3,x7) of these 8 k
                xq[m][h][4 * d + 0] = pack_lo(xv.x, xv.z);
                xq[m][h][4 * d + 1] = pack_hi(xv.x, xv.z);
                xq[m][h][4 * d + 2] = pack_lo(xv.y, xv.w);
                xq[m][h][4 * d + 3] = pack_hi(xv.y, xv.w);
                if (kF16) {
                    // even-position pairs (x0,x4), (x2,x6) meet 1024 + q; odd ones (x1,x5),
                    // (x3,x7) meet 1024 + 16q
                    sum_a = dot2_f16(xq[m][h][4 * d + 0], kF16OnePair, sum_a);
                    sum_a = dot2_f16(xq[m][h][4 * d + 2], kF16OnePair, sum_a);
                    sum_b = dot2_f16(xq[m][h][4 * d + 1], kF16OnePair, sum_b);
                    sum_b = dot2_f16(xq[m][h][4 * d + 3], kF16OnePair, sum_b);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) sum_a = dot2_bf16(xq[m][h][4 * d + e], kBf16OnePair, sum_a);
                }
            }
            sx[m][h] = sum_a + sum_b;
            if (kF16) {
                // Q4: sum (1024 + q) x - 1032 sum x = sum (q - 8) x and
                //     (sum (1024 + 16q) x - 1152 sum x) / 16 = sum (q - 8) x;
                // zero point: the offsets 1024 only, z sum x is taken off per row
                cst[m][h][0] = (kZP ? -1024.0f : -1032.0f) * sum_a;
                cst[m][h][1] = (kZP ? -1024.0f : -1152.0f) * sum_b;
            } else {
                cst[m][h][0] = (kZP ? -128.0f : -136.0f) * sum_a;  // 128 + q, less 128 (and the bias 8)
                cst[m][h][1] = 0.0f;
            }
        }
        auto compute = [&](int t, const GvStep& R) {
            float part_row[kMR];
#pragma unroll
            for (int m = 0; m < kMR; ++m) part_row[m] = 0.0f;
#pragma unroll
            for (int h = 0; h < kNB; ++h) {
                float dot[kMR];
                if constexpr (kW8) {
                    // Signed bytes with the top bit flipped are u = q + 128 in 0..255; OR-ed into
                    // the fp16 exponent of 1024 they are 1024 + u, exact: bytes 0 and 2 of a
                    // dword with mask 0x00FF00FF, bytes 1 and 3 after a shift by 8.
                    float acc[kMR];
#pragma unroll
                    for (int m = 0; m < kMR; ++m) acc[m] = cst[m][h][0];
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const uint32_t u = R.c[h][d] ^ 0x80808080u;
                        const uint32_t u0 = (u & mask_lo) | magic_v, u1 = ((u >> 8) & mask_lo) | magic_v;
#pragma unroll
                        for (int m = 0; m < kMR; ++m) {
                            acc[m] = dot2_f16(u0, xq[m][h][2 * d + 0], acc[m]);
                            acc[m] = dot2_f16(u1, xq[m][h][2 * d + 1], acc[m]);
                        }
                    }
#pragma unroll
                    for (int m = 0; m < kMR; ++m) part_row[m] += acc[m];
                    continue;
                }
                if (kF16) {
                    // Nibbles j (bits 4j) of a word hold k = j of its 8 k.  With the fp16 exponent
                    // of 1024 OR-ed in, mask 0x000F000F keeps k = 0 and 4 as 1024 + q and mask
                    // 0x00F000F0 keeps k = 1 and 5 as 1024 + 16q, both exact; the word shifted
                    // by 8 gives k = 2, 6 and 3, 7 the same way: five instructions per 8 codes.
                    float acc_a[kMR], acc_b[kMR];
#pragma unroll
                    for (int m = 0; m < kMR; ++m) acc_a[m] = cst[m][h][0], acc_b[m] = cst[m][h][1];
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const uint32_t w = R.c[h][d], w8 = w >> 8;
                        const uint32_t u0 = (w & mask_lo) | magic_v, u1 = (w & mask_hi) | magic_v;
                        const uint32_t u2 = (w8 & mask_lo) | magic_v, u3 = (w8 & mask_hi) | magic_v;
#pragma unroll
                        for (int m = 0; m < kMR; ++m) {
                            acc_a[m] = dot2_f16(u0, xq[m][h][4 * d + 0], acc_a[m]);
                            acc_b[m] = dot2_f16(u1, xq[m][h][4 * d + 1], acc_b[m]);
                            acc_a[m] = dot2_f16(u2, xq[m][h][4 * d + 2], acc_a[m]);
                            acc_b[m] = dot2_f16(u3, xq[m][h][4 * d + 3], acc_b[m]);
                        }
                    }
#pragma unroll
                    for (int m = 0; m < kMR; ++m) dot[m] = __builtin_fmaf(acc_b[m], 0.0625f, acc_a[m]);
                } else {
                    float acc[kMR];
#pragma unroll
                    for (int m = 0; m < kMR; ++m) acc[m] = cst[m][h][0];
#pragma unroll
                    for (int d = 0; d < 4; ++d)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const uint32_t u = ((R.c[h][d] >> (4 * e)) & mask_lo) | magic_v;
#pragma unroll
                            for (int m = 0; m < kMR; ++m) acc[m] = dot2_bf16(u, xq[m][h][4 * d + e], acc[m]);
                        }
#pragma unroll
                    for (int m = 0; m < kMR; ++m) dot[m] = acc[m];
                }
                const float sc = f16_bits_to_f32(R.s[h]);
#pragma unroll
                for (int m = 0; m < kMR; ++m) {
                    if constexpr (kZP) dot[m] = __builtin_fmaf(-f16_bits_to_f32(R.z[h]), sx[m][h], dot[m]);
                    part_row[m] = __builtin_fmaf(sc, dot[m], part_row[m]);
                }
            }
            // the 16 lanes of a row -> one value, added to this wave's slot for the row
#pragma unroll
            for (int m = 0; m < kMR; ++m) {
                const float v = row16_sum(part_row[m]);
                if (sub == 15) part[m][wave][4 * t + rsub] += v;
            }
        };
        // A rolling window: the loads of step i + kAhead are issued before the math of step i.
#pragma unroll
        for (int i = 0; i < kMySteps; ++i) {
            if (i + kAhead < kMySteps) load(rg + kR * (i + kAhead), r[i + kAhead]);
            compute(rg + kR * i, r[i]);
            // keep the window as written: the scheduler would otherwise hoist later steps' loads
            // past the register budget
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // the 16 waves' partials of each row (zero where a wave has no part in it), added through LDS
    // in a fixed order
    __syncthreads();
    const int t = threadIdx.x & 63, m = threadIdx.x >> 6;
    if (m < rows && n0 + t < N) {
        float sum = 0.0f;
#pragma unroll
        for (int v = 0; v < kGvWaves; ++v) sum += part[m][v][t];
        if constexpr (kW8) sum *= reinterpret_cast<const float*>(scales)[n0 + t];
        y[(size_t)m * N + n0 + t] = kF16 ? f32_to_f16_bits(sum) : f32_to_bf16_bits(sum);
    }
}

template <bool kF16, int kFmt, int kMR>
void launch_rowmajor(const uint16_t* x, const uint32_t* codes, const uint16_t* scales, const uint16_t* zeros,
                     int64_t N, int64_t K, uint16_t* y, int rows, hipStream_t stream) {
    const dim3 grid((unsigned)((N + kGvRows - 1) / kGvRows)), block(1024);
    // K-slices of 16 or 32 blocks: as many as K has, rounded up to a power of two, at most 16
    constexpr int kSW = 16 * rowmajor_blocks_per_lane(kFmt, kMR);
    const int64_t slices = (K / (kFmt == kRowW8 ? 16 : 32) + kSW - 1) / kSW;
    const int n = (int)N, k = (int)K;
    if (slices >= 9)
        hipLaunchKernelGGL((gemv_rowmajor_kernel<kF16, kFmt, 16, kMR>), grid, block, 0, stream, x, codes, scales, zeros, y, n, k, rows);
    else if (slices >= 5)
        hipLaunchKernelGGL((gemv_rowmajor_kernel<kF16, kFmt, 8, kMR>), grid, block, 0, stream, x, codes, scales, zeros, y, n, k, rows);
    else if (slices >= 3)
        hipLaunchKernelGGL((gemv_rowmajor_kernel<kF16, kFmt, 4, kMR>), grid, block, 0, stream, x, codes, scales, zeros, y, n, k, rows);
    else if (slices == 2)
        hipLaunchKernelGGL((gemv_rowmajor_kernel<kF16, kFmt, 2, kMR>), grid, block, 0, stream, x, codes, scales, zeros, y, n, k, rows);
    else
        hipLaunchKernelGGL((gemv_rowmajor_kernel<kF16, kFmt, 1, kMR>), grid, block, 0, stream, x, codes, scales, zeros, y, n, k, rows);
}

// M activation rows in passes of kRowGemvRows(format) over the weights (a last pass of three rows
// as a four-row pass, of two or one row as such).
template <bool kF16, int kFmt>
hipError_t launch_rowmajor_rows(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                                const uint16_t* zeros, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
    constexpr int kMax = kFmt == kRowZP ? kRowGemvRowsZP : kRowGemvRows;
    for (int64_t m = 0; m < M; m += kMax) {
        const int rows = (int)(M - m < kMax ? M - m : kMax);
        if (rows >= 3) {
            if constexpr (kMax >= 4)
                launch_rowmajor<kF16, kFmt, 4>(x + m * K, codes, scales, zeros, N, K, y + m * N, rows, stream);
        } else if (rows == 2) {
            launch_rowmajor<kF16, kFmt, 2>(x + m * K, codes, scales, zeros, N, K, y + m * N, rows, stream);
        } else {
            launch_rowmajor<kF16, kFmt, 1>(x + m * K, codes, scales, zeros, N, K, y + m * N, rows, stream);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_gemv_q4b32(const uint16_t* x, int64_t M, bool act_f16, const uint8_t* codes,
                             const uint16_t* scales, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
    const uint32_t* words = reinterpret_cast<const uint32_t*>(codes);
    return act_f16 ? launch_rowmajor_rows<true, kRowQ4>(x, M, words, scales, nullptr, N, K, y, stream)
                   : launch_rowmajor_rows<false, kRowQ4>(x, M, words, scales, nullptr, N, K, y, stream);
}

hipError_t launch_gemv_g128zp(const uint16_t* x, int64_t M, bool act_f16, const uint32_t* codes,
                              const uint16_t* scales, const uint16_t* zeros, int64_t N, int64_t K, uint16_t* y,
                              hipStream_t stream) {
    return act_f16 ? launch_rowmajor_rows<true, kRowZP>(x, M, codes, scales, zeros, N, K, y, stream)
                   : launch_rowmajor_rows<false, kRowZP>(x, M, codes, scales, zeros, N, K, y, stream);
}

hipError_t launch_gemv_w8row(const uint16_t* x, int64_t M, const int8_t* codes, const float* scales, int64_t N,
                             int64_t K, uint16_t* y, hipStream_t stream) {
    return launch_rowmajor_rows<true, kRowW8>(x, M, reinterpret_cast<const uint32_t*>(codes),
                                              reinterpret_cast<const uint16_t*>(scales), nullptr, N, K, y, stream);
}

}  // namespace w4a16
