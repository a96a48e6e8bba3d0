// skinny.hip -- small-M W4A16 path (1 <= M <= 16) on bf16 MFMA, for the [K/8][N] G128 format.
//
// The per-group factored form of vidyal.ai "Low-Precision Kernels" ("How the measurements were
// taken": per group s * sum(x*q) + min * sum(x) in fp32) with the inner sums on the matrix
// cores.  At M = 1 the MFMA does 16x the needed multiplies, but the matrix core is idle in a
// memory-bound kernel anyway, and every dot2 instruction it replaces is VALU time taken from
// unpacking -- the cost that kept the pages' own M = 1 kernel at 68% of its roof.
//
// Data flow per wave (16 waves per block, K split by groups over the waves):
//  * one 16-byte load per lane reads 4 adjacent columns of one packed row; a wave load covers
//    4 packed rows x 64 columns (4 x 256 B, coalesced), i.e. one k-step of 32 for 4 MFMA tiles;
//  * each 32-bit word is exactly one lane's B fragment of v_mfma_f32_16x16x32_bf16 (8 k of one
//    column): (w >> 4j) & 0x000F000F | 0x43004300 gives the bf16 pair (128 + q_j, 128 + q_{j+4}),
//    so the B fragment holds k in the order 0 4 1 5 2 6 3 7 and the activations are stored in
//    LDS in the same order;
//  * a fifth MFMA against a B fragment of ones gives sum(x) per row and group in the same
//    accumulator layout, so the group epilogue is s * acc + (min - 128 s) * sum(x);
//  * the activations a wave needs (its 4 groups x M rows) are staged in its own LDS slice, so only
//    a wave-scope ordering (no block barrier) is needed before the math; lanes whose A row is past
//    M read a zero row.
// The waves' partial sums are added through LDS in a fixed order, so results are bitwise
// reproducible.  All global loads are issued before the first MFMA and never under a branch.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace w4a16 {

namespace {

constexpr int kSkinnyWaves = 16;  // waves per block: one block per CU, four waves per SIMD
constexpr uint32_t kNibblePairMask = 0x000F000Fu;
constexpr uint32_t kBf16Magic = 0x43004300u;  // bf16 128.0 in both halves
constexpr uint32_t kF16Magic = 0x64006400u;   // fp16 1024.0 in both halves

// The register budget is sized for one block per CU.  (32-column blocks are used when N is
// small, so that there are more blocks; two of them per CU would halve the register budget and
// spill, for a grid that rarely exceeds the CU count.)

// `mask` arrives as a kernel argument (0x000F000F) and `magic` (0x43004300) is set by a v_mov of an
// immediate, both opaque to the compiler, so that they sit in
// registers and each pair is one v_and_or_b32 (VOP3 cannot take a literal on gfx9).
__device__ __forceinline__ bf16x8_t unpack_b_fragment(uint32_t w, uint32_t mask, uint32_t magic) {
    const u32x4_t p = {(w & mask) | magic, ((w >> 4) & mask) | magic, ((w >> 8) & mask) | magic,
                       ((w >> 12) & mask) | magic};
    return __builtin_bit_cast(bf16x8_t, p);
}

// v_mfma_f32_16x16x32 on bf16 or, with kF16, on fp16 operands (the same bit patterns in registers)
template <bool kF16>
__device__ __forceinline__ f32x4_t mfma16_t(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    if constexpr (kF16) {
        typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0,
                                                      0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
}

// (x0..x7) as four dwords (x0,x1) (x2,x3) (x4,x5) (x6,x7) -> (x0,x4) (x1,x5) (x2,x6) (x3,x7)
__device__ __forceinline__ uint4 pair_up(uint4 v) {
    return make_uint4((v.x & 0xFFFFu) | (v.z << 16), (v.x >> 16) | (v.z & 0xFFFF0000u),
                      (v.y & 0xFFFFu) | (v.w << 16), (v.y >> 16) | (v.w & 0xFFFF0000u));
}

// TPL words of one packed row: `row` is the (wave-uniform) row start, `off` this lane's byte
// offset from it (its 4-row sub-block and first column), so the address is SGPR base + VGPR
// offset with no per-load 64-bit arithmetic.  Streaming data: non-temporal loads.
template <int TPL, bool kVec>
__device__ __forceinline__ void load_cols(const uint32_t* __restrict__ row, uint32_t off, const uint32_t* __restrict__ clamp_row,
                                          int N, int cbase, uint32_t (&out)[TPL]) {
    if (kVec) {
        const char* p = reinterpret_cast<const char*>(row) + off;
        if (TPL == 4) {
            const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
#pragma unroll
            for (int t = 0; t < TPL; ++t) out[t] = v[t];
        } else {
            typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;
            const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
#pragma unroll
            for (int t = 0; t < TPL; ++t) out[t] = v[t];
        }
    } else {
#pragma unroll
        for (int t = 0; t < TPL; ++t) out[t] = clamp_row[min(cbase + t, N - 1)];
    }
}

// TPL bf16 scales (or minimums) of this lane's columns, kept as raw bits until the group's
// epilogue so that the loads stay in flight with the packed words.
template <int TPL, bool kVec>
__device__ __forceinline__ void load_params(const uint16_t* __restrict__ p, int N, int cbase, uint32_t (&out)[TPL / 2]) {
    if (kVec && TPL == 4) {
        const uint2 v = *reinterpret_cast<const uint2*>(p + cbase);
        out[0] = v.x;
        out[TPL / 2 - 1] = v.y;
    } else if (kVec && TPL == 2) {
        out[0] = *reinterpret_cast<const uint32_t*>(p + cbase);
    } else {
#pragma unroll
        for (int t = 0; t < TPL / 2; ++t)
            out[t] = (uint32_t)p[min(cbase + 2 * t, N - 1)] | ((uint32_t)p[min(cbase + 2 * t + 1, N - 1)] << 16);
    }
}

__device__ __forceinline__ float bf16_half(const uint32_t* v, int t) {
    return bf16_bits_to_f32((t & 1) ? (v[t >> 1] >> 16) : (v[t >> 1] & 0xFFFFu));
}

// The same for fp32 parameters (the prepared copy of the zero-point format): TPL floats.
template <int TPL, bool kVec>
__device__ __forceinline__ void load_params32(const float* __restrict__ p, int N, int cbase, float (&out)[TPL]) {
    if (kVec && TPL == 4) {
        const float4 v = *reinterpret_cast<const float4*>(p + cbase);
        out[0] = v.x;
        out[1 % TPL] = v.y;
        out[2 % TPL] = v.z;
        out[3 % TPL] = v.w;
    } else if (kVec && TPL == 2) {
        const float2 v = *reinterpret_cast<const float2*>(p + cbase);
        out[0] = v.x;
        out[TPL - 1] = v.y;
    } else {
#pragma unroll
        for (int t = 0; t < TPL; ++t) out[t] = p[min(cbase + t, N - 1)];
    }
}

// MR: activation rows staged (M <= MR; 1, 2, 4, 8 or 16).  TPL: adjacent columns per lane (4 or 2),
// i.e. 16 * TPL columns per block.  GPP: groups of 128 k per wave and pass (a pass of the 16 waves
// covers 16 * GPP groups: 2 for K > 2048, where one pass covers K = 4096; 1 up to K = 2048, where
// a second group per wave would only repeat a clamped one)
// groups per pass.  kVec: N % TPL == 0 (vector loads of a lane's columns).  kF16: fp16
// activations and output on the fp16 matrix cores, codes as 1024 + q (else bf16 and 128 + q).
// kP32: scales and minimums are fp32 [K/128][N] (the prepared zero-point copy), else bf16.
template <int MR, int TPL, int GPP, bool kVec, bool kF16 = false, bool kP32 = false, bool kSplit = false>
__global__ __launch_bounds__(64 * kSkinnyWaves)
__attribute__((amdgpu_waves_per_eu(kSkinnyWaves / 4, kSkinnyWaves / 4)))
void skinny_g128_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ codes,
                        const void* __restrict__ scales_v, const void* __restrict__ mins_v,
                        uint16_t* __restrict__ y, int M, int N, int K, uint32_t mask,
                        float* __restrict__ ws, int gps) {
    const uint16_t* __restrict__ scales = static_cast<const uint16_t*>(scales_v);
    const uint16_t* __restrict__ mins = static_cast<const uint16_t*>(mins_v);
    const float* __restrict__ scales32 = static_cast<const float*>(scales_v);
    const float* __restrict__ mins32 = static_cast<const float*>(mins_v);
    constexpr float kOffset = kF16 ? 1024.0f : 128.0f;  // the magic number's value at q = 0
    constexpr int E = MR == 1 ? 1 : 4;  // accumulator rows per lane that can hold a real row
    constexpr int COLS = 16 * TPL;
    constexpr int kWaves = kSkinnyWaves;
    constexpr int kGpp = GPP;  // groups per wave per pass
    // per wave: [group][row 0..MR-1 staged, row MR zeros][8-k chunk] of 16 B
    __shared__ uint4 xs[kWaves][kGpp][MR + 1][16];
    const int lane = lane_id(), wave = wave_id();
    const int lr = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * COLS;
    // kSplit: K split over blockIdx.y, this block's groups gs .. G - 1; else all of K
    const int gs = kSplit ? blockIdx.y * gps : 0;
    const int G = kSplit ? min(K >> 7, gs + gps) : K >> 7;
    // this lane's TPL adjacent columns; a lane past N re-reads in-range columns, never stores
    int cbase = n0 + TPL * lr;
    if (kVec) cbase = min(cbase, N - TPL);
    const int arow = min(lr, MR);  // A-fragment row: rows >= M hold zeros, row MR is all zeros
    auto mfma16 = [](bf16x8_t a, bf16x8_t b, f32x4_t c) { return mfma16_t<kF16>(a, b, c); };

#pragma unroll
    for (int j = 0; j < kGpp; ++j) xs[wave][j][MR][lr] = make_uint4(0, 0, 0, 0);  // the zero row

    float yacc[TPL][E];
#pragma unroll
    for (int t = 0; t < TPL; ++t)
#pragma unroll
        for (int e = 0; e < E; ++e) yacc[t][e] = 0.0f;

    // the magic exponent in a VGPR (the mask stays in an SGPR): one v_and_or_b32 per pair.  An
    // immediate rather than an argument: every argument an unsplit launch reads then fits the 14
    // dwords that are preloaded into SGPRs, so a wave issues its loads without a kernel-argument
    // fetch first.
    uint32_t magic;
    asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "i"(kF16 ? kF16Magic : kBf16Magic));
    constexpr uint32_t kOne = kF16 ? 0x3C003C00u : 0x3F803F80u;  // 1.0 in both halves
    const u32x4_t ones_u = {kOne, kOne, kOne, kOne};
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, ones_u);

    // One pass over CNT groups per wave: wave w takes groups p0 + w + 16 j, j < CNT.
    auto pass = [&](int p0, auto cnt_c) {
        constexpr int CNT = decltype(cnt_c)::value;
        // 1) activation chunks of this wave's groups: chunk q = (j * MR + m) * 16 + c
        constexpr int kChunks = CNT * MR * 16;  // 16-byte chunks of x this wave stages per pass
        constexpr int kNI = (kChunks + 63) / 64;
        uint4 xr[kNI];
#pragma unroll
        for (int i = 0; i < kNI; ++i) {
            const int q = min(lane + 64 * i, kChunks - 1);  // surplus lanes repeat the last chunk
            const int c = q & 15, m = (q >> 4) % MR, j = q / (16 * MR);
            const int g = min(p0 + wave + kWaves * j, G - 1);
            const int mm = min(m, M - 1);
            xr[i] = *reinterpret_cast<const uint4*>(x + (size_t)mm * K + (size_t)g * 128 + c * 8);
        }
        // 2) group parameters and 3) packed words, in the order they are used
        int gj[CNT];
        float live[CNT];
#pragma unroll
        for (int j = 0; j < CNT; ++j) {
            const int g = p0 + wave + kWaves * j;
            live[j] = g < G ? 1.0f : 0.0f;  // a clamped duplicate group contributes nothing
            gj[j] = min(g, G - 1);
        }
        uint32_t sf[CNT][TPL / 2], mf[CNT][TPL / 2];
        float sf32[CNT][TPL], mf32[CNT][TPL];
#pragma unroll
        for (int j = 0; j < CNT; ++j) {
            if constexpr (kP32) {
                load_params32<TPL, kVec>(scales32 + (size_t)gj[j] * N, N, cbase, sf32[j]);
                load_params32<TPL, kVec>(mins32 + (size_t)gj[j] * N, N, cbase, mf32[j]);
            } else {
                load_params<TPL, kVec>(scales + (size_t)gj[j] * N, N, cbase, sf[j]);
                load_params<TPL, kVec>(mins + (size_t)gj[j] * N, N, cbase, mf[j]);
            }
        }
        uint32_t w[CNT][4][TPL];
        const uint32_t lane_off = ((uint32_t)lg * (uint32_t)N + (uint32_t)cbase) * 4u;
#pragma unroll
        for (int j = 0; j < CNT; ++j)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                load_cols<TPL, kVec>(codes + (size_t)(16 * gj[j] + 4 * s) * N, lane_off,
                                     codes + (size_t)(16 * gj[j] + 4 * s + lg) * N, N, cbase, w[j][s]);

        // 4) stage the paired activations (rows >= M as zeros) in this wave's LDS slice
#pragma unroll
        for (int i = 0; i < kNI; ++i) {
            const int q = min(lane + 64 * i, kChunks - 1);
            const int c = q & 15, m = (q >> 4) % MR, j = q / (16 * MR);
            xs[wave][j][m][c] = m < M ? pair_up(xr[i]) : make_uint4(0, 0, 0, 0);
        }
        wave_lds_sync();  // the slice is read below by other lanes of this wave

        // 5) per group: 4 k-steps of (TPL + 1) MFMAs, then the group epilogue
#pragma unroll
        for (int j = 0; j < CNT; ++j) {
            f32x4_t acc[TPL], accs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < TPL; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, xs[wave][j][arow][4 * s + lg]);
#pragma unroll
                for (int t = 0; t < TPL; ++t)
                    acc[t] = mfma16(a, unpack_b_fragment(w[j][s][t], mask, magic), acc[t]);
                accs = mfma16(a, ones, accs);
            }
#pragma unroll
            for (int t = 0; t < TPL; ++t) {
                const float sv = kP32 ? sf32[j][t] : bf16_half(sf[j], t), mv = kP32 ? mf32[j][t] : bf16_half(mf[j], t);
                const float s = sv * live[j];
                const float c = __builtin_fmaf(-kOffset, sv, mv) * live[j];  // min - 128 s (or - 1024 s)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    yacc[t][e] = __builtin_fmaf(s, acc[t][e], yacc[t][e]);
                    yacc[t][e] = __builtin_fmaf(c, accs[e], yacc[t][e]);
                }
            }
        }
        wave_lds_sync();  // this pass's reads of the slice precede the next pass's writes
    };
    // a last pass of 16 groups or fewer: one group per wave, none repeated (not in the instances
    // where the second pass body costs registers: 16 rows with fp32 parameters, scalar columns)
    constexpr bool kShortLast = kGpp > 1 && kVec && !(kP32 && MR == 16);
    for (int p0 = gs; p0 < G; p0 += kWaves * kGpp) {
        if (kShortLast && G - p0 <= kWaves)
            pass(p0, std::integral_constant<int, 1>{});
        else
            pass(p0, std::integral_constant<int, kGpp>{});
    }

    // 6) partial sums through LDS: each wave reuses its own activation slice (it has finished
    //    reading it), rows 0..min(M,16)-1 x COLS columns as fp32; then a fixed-order sum.
    float* part = reinterpret_cast<float*>(&xs[wave][0][0][0]);
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int row = 4 * lg + e;
        if (row < M) {
#pragma unroll
            for (int t = 0; t < TPL; ++t) part[row * COLS + TPL * lr + t] = yacc[t][e];
        }
    }
    __syncthreads();
    const int rows = min(M, 16);
    for (int idx = threadIdx.x; idx < rows * COLS; idx += 64 * kWaves) {
        const int row = idx / COLS, c = idx % COLS;
        const int n = n0 + c;
        if (n < N) {
            float sum = 0.0f;
#pragma unroll
            for (int v = 0; v < kWaves; ++v)
                sum += reinterpret_cast<const float*>(&xs[v][0][0][0])[row * COLS + c];
            if constexpr (kSplit)  // the split's fp32 partial sums, [split][M][N]
                ws[((size_t)blockIdx.y * M + row) * N + n] = sum;
            else
                y[(size_t)row * N + n] = kF16 ? f32_to_f16_bits(sum) : f32_to_bf16_bits(sum);
        }
    }
}

// kSplit: K split over gridDim.y (splits), fp32 partial sums to ws [splits][M][N] (y untouched).
template <int MR, int TPL, int GPP, bool kF16, bool kP32, bool kSplit>
void launch_gpp(const uint16_t* x, int64_t M, const uint32_t* codes, const void* scales, const void* mins,
                int64_t N, int64_t K, uint16_t* y, float* ws, int splits, int gps, hipStream_t stream) {
    constexpr int COLS = 16 * TPL;
    const dim3 grid((unsigned)((N + COLS - 1) / COLS), (unsigned)splits), block(64 * kSkinnyWaves);
    if (N % TPL == 0)
        hipLaunchKernelGGL((skinny_g128_kernel<MR, TPL, GPP, true, kF16, kP32, kSplit>), grid, block, 0, stream, x, codes,
                           scales, mins, y, (int)M, (int)N, (int)K, kNibblePairMask, ws, gps);
    else
        hipLaunchKernelGGL((skinny_g128_kernel<MR, TPL, GPP, false, kF16, kP32, kSplit>), grid, block, 0, stream, x, codes,
                           scales, mins, y, (int)M, (int)N, (int)K, kNibblePairMask, ws, gps);
}

template <int MR, int TPL, bool kF16 = false, bool kP32 = false>
void launch_mr(const uint16_t* x, int64_t M, const uint32_t* codes, const void* scales, const void* mins,
               int64_t N, int64_t K, uint16_t* y, hipStream_t stream, float* ws = nullptr, int splits = 1) {
    const int G = (int)(K >> 7), gps = (G + splits - 1) / splits;  // groups per split
    if (splits > 1) {
        if constexpr (!kF16 && !kP32) {  // the split serves the G128 path only
            if (gps <= kSkinnyWaves)
                launch_gpp<MR, TPL, 1, false, false, true>(x, M, codes, scales, mins, N, K, y, ws, splits, gps, stream);
            else
                launch_gpp<MR, TPL, 2, false, false, true>(x, M, codes, scales, mins, N, K, y, ws, splits, gps, stream);
        }
    } else if (gps <= kSkinnyWaves) {
        launch_gpp<MR, TPL, 1, kF16, kP32, false>(x, M, codes, scales, mins, N, K, y, nullptr, 1, gps, stream);
    } else {
        launch_gpp<MR, TPL, 2, kF16, kP32, false>(x, M, codes, scales, mins, N, K, y, nullptr, 1, gps, stream);
    }
}

}  // namespace

#ifndef W4A16_SKINNY_TPL
#define W4A16_SKINNY_TPL 0  // 0: chosen from N at launch
#endif

namespace {
// M rows, the column split chosen from N (the same for every variant).
template <bool kF16, bool kP32>
void launch_rows(const uint16_t* x, int64_t M, const uint32_t* codes, const void* scales, const void* mins, int64_t N,
                 int64_t K, uint16_t* y, hipStream_t stream) {
    // 64 columns per block (16-byte loads, measured best) unless that leaves most CUs idle
    const int tpl = W4A16_SKINNY_TPL ? W4A16_SKINNY_TPL : ((N + 63) / 64 >= 192 ? 4 : 2);
    if (tpl == 4) {
        if (M == 1) launch_mr<1, 4, kF16, kP32>(x, M, codes, scales, mins, N, K, y, stream);
        else if (M == 2) launch_mr<2, 4, kF16, kP32>(x, M, codes, scales, mins, N, K, y, stream);
        else if (M <= 4) launch_mr<4, 4, kF16, kP32>(x, M, codes, scales, mins, N, K, y, stream);
        else if (M <= 8) launch_mr<8, 4, kF16, kP32>(x, M, codes, scales, mins, N, K, y, stream);
        else launch_mr<16, 4, kF16, kP32>(x, M, codes, scales, mins, N, K, y, stream);
    } else {
        if (M == 1) launch_mr<1, 2, kF16, kP32>(x, M, codes, scales, mins, N, K, y, stream);
        else if (M == 2) launch_mr<2, 2, kF16, kP32>(x, M, codes, scales, mins, N, K, y, stream);
        else if (M <= 4) launch_mr<4, 2, kF16, kP32>(x, M, codes, scales, mins, N, K, y, stream);
        else if (M <= 8) launch_mr<8, 2, kF16, kP32>(x, M, codes, scales, mins, N, K, y, stream);
        else launch_mr<16, 2, kF16, kP32>(x, M, codes, scales, mins, N, K, y, stream);
    }
}
}  // namespace

hipError_t launch_skinny_g128(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                              const uint16_t* mins, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
    launch_rows<false, false>(x, M, codes, scales, mins, N, K, y, stream);
    return hipGetLastError();
}

hipError_t launch_skinny_g128_split(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                                    const uint16_t* mins, int64_t N, int64_t K, uint16_t* y, float* ws, int splits,
                                    hipStream_t stream) {
    // 64-column blocks times `splits` K-slices, then the partials summed in split order
    if (M == 1) launch_mr<1, 4>(x, M, codes, scales, mins, N, K, y, stream, ws, splits);
    else if (M == 2) launch_mr<2, 4>(x, M, codes, scales, mins, N, K, y, stream, ws, splits);
    else if (M <= 4) launch_mr<4, 4>(x, M, codes, scales, mins, N, K, y, stream, ws, splits);
    else if (M <= 8) launch_mr<8, 4>(x, M, codes, scales, mins, N, K, y, stream, ws, splits);
    else launch_mr<16, 4>(x, M, codes, scales, mins, N, K, y, stream, ws, splits);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_splitk_reduce(ws, M * N, splits, y, stream);
}

hipError_t launch_skinny_prepared_zp(const uint16_t* x, int64_t M, bool act_f16, const uint32_t* codes,
                                     const float* scales, const float* mins, int64_t N, int64_t K, uint16_t* y,
                                     hipStream_t stream) {
    if (act_f16)
        launch_rows<true, true>(x, M, codes, scales, mins, N, K, y, stream);
    else
        launch_rows<false, true>(x, M, codes, scales, mins, N, K, y, stream);
    return hipGetLastError();
}

}  // namespace w4a16
