// launch.h -- internal host-side launchers of the libw4a16 kernels (not part of the C ABI).
// Each returns hipSuccess or the HIP error of the launch; arguments are validated by the
// C-ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

// hipGetLastError returns the last error of any runtime call made on this thread -- also of
// calls the caller made before calling into this library and did not check (a "not ready" from
// a query, say).  Each entry point clears it before it launches, so that the hipGetLastError
// after a launch reports that launch alone.
inline void clear_stale_error() { (void)hipGetLastError(); }

hipError_t launch_pack_g128(const float* W, int64_t N, int64_t K, uint32_t* codes, uint16_t* scales,
                            uint16_t* mins, hipStream_t stream);
hipError_t launch_pack_q4b32(const float* W, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales,
                             hipStream_t stream);
// dtype: 0 bf16, 1 fp16, 2 fp32
hipError_t launch_dequant_g128(const uint32_t* codes, const uint16_t* scales, const uint16_t* mins, int64_t N,
                               int64_t K, int dtype, void* out, hipStream_t stream);
hipError_t launch_dequant_q4b32(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K, int dtype,
                                void* out, hipStream_t stream);

// Zero-point format (fp16 scale and zero point per group of 128, words [N][K/8]).
hipError_t launch_pack_g128zp(const float* W, int64_t N, int64_t K, uint32_t* codes, uint16_t* scales,
                              uint16_t* zeros, hipStream_t stream);
hipError_t launch_dequant_g128zp(const uint32_t* codes, const uint16_t* scales, const uint16_t* zeros, int64_t N,
                                 int64_t K, int dtype, void* out, hipStream_t stream);
hipError_t launch_gemv_g128zp(const uint16_t* x, int64_t M, bool act_f16, const uint32_t* codes,
                              const uint16_t* scales, const uint16_t* zeros, int64_t N, int64_t K, uint16_t* y,
                              hipStream_t stream);

// W8 format (int8 [N][K], fp32 scale per row).
hipError_t launch_pack_w8row(const float* W, int64_t N, int64_t K, int8_t* codes, float* scales, hipStream_t stream);
hipError_t launch_dequant_w8row(const int8_t* codes, const float* scales, int64_t N, int64_t K, int dtype, void* out,
                                hipStream_t stream);
hipError_t launch_gemv_w8row(const uint16_t* x, int64_t M, const int8_t* codes, const float* scales, int64_t N,
                             int64_t K, uint16_t* y, hipStream_t stream);

// Small-M G128 path (the skinny MFMA kernel), bf16 activations, M <= kGemvMaxRows.
constexpr int kGemvMaxRows = 16;
hipError_t launch_skinny_g128(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                              const uint16_t* mins, int64_t N, int64_t K, uint16_t* y, hipStream_t stream);
// The same with K split over `splits` blocks per 64 columns, the fp32 partials in ws
// [splits][M][N], then summed in split order into y (two launches).
hipError_t launch_skinny_g128_split(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                                    const uint16_t* mins, int64_t N, int64_t K, uint16_t* y, float* ws, int splits,
                                    hipStream_t stream);
// K splits for the small-M kernel (1: none): where even its 32-column blocks would leave CUs idle
// (fewer than 192 of them) and the codes (at least 16 MiB) pay for the second launch, 64-column
// blocks times enough splits to fill 256 CUs, 2..8, each at least 16 groups of K.  Measured: at
// N = 4096, K = 14336 11.6 / 18.5 us -> 10.1 / 13.0 us for 1 / 16 rows; at N = 2048, K = 16384
// 12.1 / 20.0 -> 8.4 / 10.4 us; at N = 8192 (256 blocks of 32 columns) the split lost.
inline int skinny_splits(int64_t M, int64_t N, int64_t K) {
    const int64_t nb = (N + 63) / 64, G = K / 128;
    if (M < 1 || M > kGemvMaxRows || (N + 31) / 32 >= 192 || N * K / 2 < ((int64_t)16 << 20)) return 1;
    int s = (int)(256 / nb);
    s = s < 2 ? 2 : (s > 8 ? 8 : s);
    while (s > 1 && G / s < 16) --s;
    return s;
}
inline size_t skinny_split_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const int s = skinny_splits(M, N, K);
    return s > 1 ? (size_t)s * (size_t)M * (size_t)N * 4 : 0;
}
// Rows of activations that the row-major GEMV takes against one pass over the weights: four for
// Q4 and W8, two for the zero-point format (whose four-row form spills registers).
constexpr int kRowGemvRows = 4;
constexpr int kRowGemvRowsZP = 2;
// Q4 path, kRowGemvRows activation rows per pass over the weights; act_f16: fp16 (true) or bf16
// (false) activations.  (The zero-point and W8 GEMVs above pass over the weights the same way.)
hipError_t launch_gemv_q4b32(const uint16_t* x, int64_t M, bool act_f16, const uint8_t* codes,
                             const uint16_t* scales, int64_t N, int64_t K, uint16_t* y, hipStream_t stream);

// The zero-point format's prepared copy: words [K/8][N], fp32 s and m = -z s per group [K/128][N];
// and the small-M kernel over it (fp16 or bf16 activations, M <= kGemvMaxRows).
hipError_t launch_prepare_zp(const uint32_t* codes, const uint16_t* scales, const uint16_t* zeros, int64_t N, int64_t K,
                             uint32_t* words, float* s_out, float* m_out, hipStream_t stream);
hipError_t launch_skinny_prepared_zp(const uint16_t* x, int64_t M, bool act_f16, const uint32_t* codes,
                                     const float* scales, const float* mins, int64_t N, int64_t K, uint16_t* y,
                                     hipStream_t stream);
// ... and the 17..32-row kernel over it, and the 64-row one (midr_fits(64, N, K), M <= 64).
hipError_t launch_rows32_prepared_zp(const uint16_t* x, int64_t M, bool act_f16, const uint32_t* codes,
                                     const float* scales, const float* mins, int64_t N, int64_t K, uint16_t* y,
                                     hipStream_t stream);
hipError_t launch_rows64_prepared_zp(const uint16_t* x, int64_t M, bool act_f16, const uint32_t* codes,
                                     const float* scales, const float* mins, int64_t N, int64_t K, uint16_t* y,
                                     hipStream_t stream);
// Shapes the R-row kernels take (R = 64: groups in pairs, R = 32: in fours; 4-column copies);
// others use the general kernels.
inline bool midr_fits(int R, int64_t N, int64_t K) { return N % 4 == 0 && (K / 128) % (R == 64 ? 2 : 4) == 0; }
// K split for the R-row kernels (17..64 rows, G128; splits 1: none): where their 64-column blocks
// number at most 128 (so that two or more splits still fit one wave of 256 blocks; at N = 11008,
// 172 blocks, a second wave made the split 1.5x slower) and the codes are at least 8 MiB, enough
// splits for 256 blocks, 2..8, each a whole number of stages and at least 16 groups of K.
struct MidSplit {
    int splits, gps, rows;  // rows: the R-row kernel (32, or 64 also for 17..32 rows where
                            // K / 128 is not a multiple of 4)
};
inline MidSplit mid_split(int64_t M, int64_t N, int64_t K) {
    const int R = M <= 32 && midr_fits(32, N, K) ? 32 : 64, gsz = R == 64 ? 2 : 4;  // groups per stage
    const int64_t nb = (N + 63) / 64, G = K / 128;
    if (M <= kGemvMaxRows || M > 64 || !midr_fits(R, N, K) || nb > 128 || N * K / 2 < ((int64_t)8 << 20))
        return {1, 0, R};
    int s = (int)(256 / nb);
    s = s < 2 ? 2 : (s > 8 ? 8 : s);
    while (s > 1 && G / s < 16) --s;
    if (s <= 1) return {1, 0, R};
    const int gps = (int)((G + s - 1) / s + gsz - 1) / gsz * gsz;
    return {(int)((G + gps - 1) / gps), gps, R};
}
inline size_t mid_split_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const MidSplit sp = mid_split(M, N, K);
    return sp.splits > 1 ? (size_t)sp.splits * (size_t)M * (size_t)N * 4 : 0;
}
// 17..64 rows with K split as mid_split says: fp32 partials in ws, then summed in split order.
hipError_t launch_mid_g128_split(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                                 const uint16_t* mins, int64_t N, int64_t K, uint16_t* y, float* ws, hipStream_t stream);

// Row-major formats on fp16 MFMA for any number of fp16 activation rows (16 per weight pass).
hipError_t launch_rowmma_q4b32(const uint16_t* x, int64_t M, const uint8_t* codes, const uint16_t* scales, int64_t N,
                               int64_t K, uint16_t* y, hipStream_t stream);
hipError_t launch_rowmma_g128zp(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                                const uint16_t* zeros, int64_t N, int64_t K, uint16_t* y, hipStream_t stream);
hipError_t launch_rowmma_w8row(const uint16_t* x, int64_t M, const int8_t* codes, const float* scales, int64_t N,
                               int64_t K, uint16_t* y, hipStream_t stream);

// Mid-M G128 path (kGemvMaxRows < M <= kMidMaxRows): weights streamed once per 64-row slice,
// dequantized straight into MFMA fragments; no workspace.
constexpr int kMidMaxRows = 64;  // measured: beyond 64 rows the large-M kernel is faster
hipError_t launch_mid_g128(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                           const uint16_t* mins, int64_t N, int64_t K, uint16_t* y, hipStream_t stream);

// Large-M G128 path on bf16 MFMA (the mid path below kMidMaxRows rows).
size_t gemm_g128_workspace_bytes(int64_t M, int64_t N, int64_t K);
// y [MN] = bf16 of the sum over `splits` fp32 partial arrays ws [splits][MN], in split order.
hipError_t launch_splitk_reduce(const float* ws, int64_t MN, int splits, uint16_t* y, hipStream_t stream);
hipError_t launch_gemm_g128(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                            const uint16_t* mins, int64_t N, int64_t K, uint16_t* y, float* workspace,
                            hipStream_t stream);

// W4A8: per-row int8 activations (xq [M][K], ascale [M], xsum [K/128][M]) and the int8-MFMA GEMM
// against the G128 weights (N % 4 == 0).
hipError_t launch_quant_act_i8(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* ascale, float* xsum,
                               hipStream_t stream);
hipError_t launch_gemm_w4a8(const int8_t* xq, const float* ascale, const float* xsum, int64_t M,
                            const uint32_t* codes, const uint16_t* scales, const uint16_t* mins, int64_t N, int64_t K,
                            uint16_t* y, hipStream_t stream);
// The same product for one bf16 row x [K] (M == 1), quantized inside the product's kernel.
hipError_t launch_matmul_w4a8_fused(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                                    const uint16_t* mins, int64_t N, int64_t K, uint16_t* y, hipStream_t stream);

}  // namespace w4a16
