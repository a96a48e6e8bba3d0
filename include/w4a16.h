/*
 * w4a16.h -- C ABI of libw4a16: 4-bit-weight, 16-bit-activation matmul y = x . W_hat^T on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation and the two weight formats follow:
 *  - vidyal.ai, "Low-Precision Kernels: INT4, INT8 and FP8 Matmuls, Measured", section
 *    "Step 2: a W4A16 kernel in Triton": groups of 128 consecutive weights along K with a bf16
 *    scale (max - min)/15 and a bf16 minimum; codes round((w - min)/scale) in 0..15; eight
 *    codes per 32-bit word along K, first k in the lowest nibble, giving a K/8 x N word matrix
 *    and K/128 x N scales and minimums; dequantized in registers as q*scale + min; bf16
 *    activations, fp32 accumulation, bf16 output.  (Format W4A16_FMT_G128_ASYM_BF16.)
 *  - thuongvuho.com, "Why My 4-Bit CUDA Kernel Wasn't Faster", sections "Why fewer bytes should
 *    have helped" and "Loading the same bytes differently": blocks of 32 weights with 16 bytes
 *    of codes and one fp16 scale, decoded as (code - bias) * scale, code byte j holding weight
 *    2j in its low nibble and 2j+1 in its high nibble; fp16 activations.  The bias is 8 and the
 *    scale max|w|/7.  (Format W4A16_FMT_Q4_B32_SYM_FP16.)
 *  - anrans.github.io, "Quantization and GEMV", sections "Writing a GEMV kernel" and
 *    "W4A16: dequantizing in registers": the small-batch GEMV structure and the zero-range
 *    rule (a group whose max equals its min gets scale 1).
 *
 * Rounding (both formats, identical in every entry point): codes use the STORED rounded scale
 * and minimum, IEEE fp32 division and round-half-to-even, clamped to 0..15; bf16/fp16 values
 * are rounded to nearest even; a zero min/max counts as +0.
 *
 * Conventions for every call:
 *  - All array arguments are DEVICE pointers (hipMalloc'd or equivalent) owned by the caller;
 *    the library allocates nothing, frees nothing and keeps no global mutable state.
 *  - All calls are asynchronous on `stream` (NULL = the default stream).  A returned
 *    W4A16_OK means the work was enqueued; device-side completion is the caller's to await.
 *  - Arguments are validated on the host, before anything is enqueued.  A failed check
 *    returns W4A16_ERR_INVALID (bad value, null or misaligned pointer) or
 *    W4A16_ERR_UNSUPPORTED (a valid combination this build does not implement) and touches
 *    no memory.  A HIP error while enqueuing returns W4A16_ERR_DEVICE.  Before it enqueues,
 *    a call clears the calling thread's pending HIP error (hipGetLastError), which may have
 *    been left by an earlier, unrelated runtime call, so that only its own launches are judged.
 *  - Every pointer must be 16-byte aligned; arrays are dense and row-major as documented.
 *  - Sizes are int64_t; M, N, K must be positive and at most 2^30 (W4A16_ERR_INVALID otherwise).
 *    N needs no particular multiple.  N above 2^26 or K above 2^22 returns
 *    W4A16_ERR_UNSUPPORTED: the kernels address operands as a 64-bit base plus a 32-bit
 *    per-lane byte offset.
 *  - Weights given to the quantizers must be finite (non-finite input is undefined).
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W4A16_OK = 0,
    W4A16_ERR_INVALID = 1,      /* a bad argument: value, null or misaligned pointer, size */
    W4A16_ERR_UNSUPPORTED = 2,  /* a valid request outside what this build implements */
    W4A16_ERR_DEVICE = 3        /* the HIP runtime refused a launch */
} w4a16_status_t;

typedef enum {
    /* codes  uint32 [K/8][N]  word (r, n) = codes of k = 8r..8r+7 of column n, k = 8r in bits 0..3
     * scales bf16   [K/128][N]
     * mins   bf16   [K/128][N]
     * w_hat = bf16-or-fp32 of fmaf(q, scale, min); K % 128 == 0 */
    W4A16_FMT_G128_ASYM_BF16 = 0,
    /* codes  uint8  [N][K/32][16]  byte j of block b = code of k = 32b+2j (low nibble) and
     *                              k = 32b+2j+1 (high nibble)
     * scales fp16   [N][K/32]
     * mins   unused (pass NULL)
     * w_hat = (q - 8) * scale (exact in fp32); K % 32 == 0 */
    W4A16_FMT_Q4_B32_SYM_FP16 = 1,
    /* anrans.github.io "Quantization and GEMV", "The quantization formulas" and "W4A16:
     * dequantizing in registers" (an integer zero point per group):
     * codes  uint32 [N][K/8]  word (n, r) = codes of k = 8r..8r+7 of row n, k = 8r in bits 0..3
     * scales fp16   [N][K/128]  s = fp16((max - min)/15), 1.0 for a zero range
     * mins   fp16   [N][K/128]  the zero points z = round(-min/s) (integers, clamped to
     *                           [-2048, 2048]), passed in the `mins` argument
     * q = clamp(round(w/s) + z, 0, 15) with round half away from zero (the page's std::round);
     * w_hat = (q - z) * scale (exact in fp32); K % 128 == 0.  The code bytes of a row are laid
     * out as those of the Q4 format. */
    W4A16_FMT_G128_ZP_FP16 = 2,
    /* anrans.github.io "Quantization and GEMV", "Exercises", 1 (W8A16, symmetric per channel):
     * codes  int8   [N][K]  q = clamp(round(w/s), -127, 127), round half away from zero
     * scales fp32   [N]     s = max|w| / 127 per row (1.0 for an all-zero row)
     * mins   unused (pass NULL)
     * w_hat = q * s; K % 16 == 0; fp16 activations only.  Packed sizes: N*K and 4*N bytes. */
    W4A16_FMT_W8_ROW_FP32 = 3
} w4a16_format_t;

typedef enum {
    W4A16_BF16 = 0,
    W4A16_FP16 = 1,
    W4A16_FP32 = 2
} w4a16_dtype_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* w4a16_status_string(w4a16_status_t status);

/* Bytes to allocate for the three packed arrays of an N x K weight in `fmt` (mins is 0 for the
 * Q4 and W8 formats).  G128 and the zero-point format store N*K/2 bytes of codes and two 2-byte
 * values per group of 128, 4 + 32/128 = 4.25 bits per weight (vidyal.ai "Low-Precision Kernels",
 * "Step 1": the 4.25 bits per weight behind the 3.76x ceiling over bf16, and "Step 2": a K/8 x N
 * word matrix with K/128 x N scales and minimums).  Q4 stores 16 code bytes and a 2-byte fp16
 * scale per block of 32 weights, 18 bytes or 4.5 bits per weight (thuongvuho.com "Why My 4-Bit
 * CUDA Kernel Wasn't Faster", introduction and "Why fewer bytes should have helped").  W8 stores
 * one byte per weight and a 4-byte scale per row (anrans.github.io "Quantization and GEMV",
 * "Exercises", 1).  For G128 the scale and minimum sizes are the arrays' sizes rounded up to a
 * multiple of 4 bytes: the GEMM reads them as aligned 4-byte words, so when (K/128)*N is odd
 * the last word covers 2 bytes past the last element (read, never written, value unused).
 * Buffers passed to the matmul entry points must have at least these sizes.
 * Pure host arithmetic; any output pointer may be NULL.  ERR_INVALID if N, K <= 0 or K is not a
 * multiple of the format's group (128, 32, or 16 for W8). */
w4a16_status_t w4a16_packed_sizes(w4a16_format_t fmt, int64_t N, int64_t K,
                                  size_t* codes_bytes, size_t* scales_bytes, size_t* mins_bytes);

/* Quantize and pack fp32 weights W [N][K] (row-major) into `fmt`.
 * Vidyal.ai "Low-Precision Kernels", Step 2 (G128: per (n, group) min/max, scale, min, codes);
 * thuongvuho.com "Why My 4-Bit CUDA Kernel Wasn't Faster", introduction and "Loading the same
 * bytes differently" (Q4: per (n, block) absmax/7 fp16 scale, codes + 8).
 * Output arrays as described by w4a16_format_t, all written in full (mins: G128 only; NULL
 * for Q4).  The result is bit-identical to the CPU definition.  With W4A16_DEBUG_CHECKS set, the
 * call first synchronizes `stream`, copies W to host memory it allocates and frees, and returns
 * the status of w4a16_check_weights on it (ERR_INVALID before any launch). */
w4a16_status_t w4a16_quantize_pack(w4a16_format_t fmt, const float* W, int64_t N, int64_t K,
                                   void* codes, void* scales, void* mins, hipStream_t stream);

/* Debug check of weights before they are quantized, on HOST memory: W [N][K] fp32 row-major.
 * Returns W4A16_ERR_INVALID if a weight is not finite or if a group's stored parameter would
 * overflow its storage type: for Q4 a block with max|w| / 7 at or above 65520 (the fp16 scale
 * would round to infinity, i.e. max|w| > 7 x 65504 in round numbers; thuongvuho.com "Why My 4-Bit
 * CUDA Kernel Wasn't Faster", introduction: the fp16 block scale); for the zero-point format a
 * group with (max - min) / 15 at or above 65520 (anrans.github.io "Quantization and GEMV", "The
 * quantization formulas", the scale kept in fp16); for G128 a scale (max - min) / 15 or minimum
 * whose bf16 rounding overflows (vidyal.ai "Low-Precision Kernels", "Step 2").  W4A16_OK
 * otherwise.  Pure host code: no HIP call, no allocation.  Shape checks as w4a16_packed_sizes.
 * w4a16_quantize_pack runs this check itself (on a host copy of W, after synchronizing `stream`)
 * when the environment variable W4A16_DEBUG_CHECKS is set to a value other than "0"; without it
 * the quantizers do not check, and non-finite or overflowing weights give undefined codes. */
w4a16_status_t w4a16_check_weights(w4a16_format_t fmt, const float* W_host, int64_t N, int64_t K);

/* Reference dequant: W_hat [N][K] (row-major) in `out_dtype` (BF16, FP16 or FP32), each value
 * the round-to-nearest-even of the fp32 dequantized weight (fmaf(q, s, m) for G128,
 * (q - 8) * s for Q4).  Same pages as w4a16_quantize_pack. */
w4a16_status_t w4a16_dequant(w4a16_format_t fmt, const void* codes, const void* scales,
                             const void* mins, int64_t N, int64_t K, w4a16_dtype_t out_dtype,
                             void* W_hat, hipStream_t stream);

/* Small-M path: y [M][N] = x [M][K] . W_hat^T for 1 <= M <= w4a16_gemv_max_rows().
 * Streams the packed words once with 128-bit or 32-bit coalesced loads, unpacks nibbles in
 * registers, sums x.q per group in fp32 and applies the group scale and minimum once per group
 * (the factored form s * sum(x*q) + min * sum(x) that vidyal.ai's M = 1 kernel uses, section
 * "How the measurements were taken"; P3's one-row-per-warp GEMV, "Writing a GEMV kernel").
 * act: BF16 for G128; FP16 (or BF16) for Q4 and the zero-point format; FP16 for W8.  For Q4,
 * the zero-point format and W8, up to four rows of fp16 activations (two for the zero-point
 * format) take the row-major GEMV (dot2 with the scale applied once per block, all rows against
 * one weight pass); more fp16 rows share one weight pass per 16 rows on the fp16 matrix cores: Q4
 * and W8 dequantized to fp16 in registers ((q - 8) s rounded once, or q exactly, the W8 row scale
 * applied to each total), the zero-point format in the factored per-group form
 * s * sum(x*(1024+q)) - (1024 + z) s * sum(x) in fp32; bf16 activations run one weight pass per
 * four rows (two for the zero-point format).  y has
 * the activation dtype, rounded to nearest even from fp32.  Row-major x and y; x, y 16-byte
 * aligned. */
w4a16_status_t w4a16_gemv(w4a16_format_t fmt, w4a16_dtype_t act, const void* x, int64_t M,
                          const void* codes, const void* scales, const void* mins, int64_t N,
                          int64_t K, void* y, hipStream_t stream);

/* Largest M that w4a16_gemv accepts. */
int64_t w4a16_gemv_max_rows(void);

/* Bytes of device workspace w4a16_gemm needs for this shape (0 if none), or, up to 16 rows of
 * G128, what w4a16_matmul uses to split K over blocks (below).  The workspace holds split-K
 * partial sums; it is caller-owned, needs no initialisation, and must not be shared by two calls
 * that may run at the same time. */
size_t w4a16_gemm_workspace_bytes(w4a16_format_t fmt, int64_t M, int64_t N, int64_t K);

/* Large-M path: y [M][N] = x [M][K] . W_hat^T on the matrix cores with fp32 accumulation.
 * Q4, the zero-point format and W8 (fp16 activations only; ERR_UNSUPPORTED for bf16): any M, each
 * 16 rows against one pass over the weights, as for w4a16_gemv's rows (anrans.github.io
 * "Quantization and GEMV", "The quantization formulas": the zero-point format's (q - z) s, in its
 * factored per-group form); no workspace.  G128 as follows, on bf16 MFMA.
 * From 65 rows on (and at 33..64 rows when N % 4 != 0 or K % 256 != 0), packed B tiles are
 * dequantized (fmaf(q, s, m) rounded to bf16, as vidyal.ai Step 2 builds its B tile) and fed to the
 * matrix cores; otherwise, up to 64 rows, the factored per-group form of w4a16_gemv
 * (s * sum(x*(128+q)) + (min - 128 s) * sum(x), fp32) is used instead -- with K split over 2..8
 * blocks per 64 columns, the fp32 partials summed in split order, when N is small (at most 128
 * column blocks), the codes are at least 8 MiB and the workspace holds the partials
 * (w4a16_gemm_workspace_bytes); without one that path runs unsplit.  When a K
 * split is used, partial sums go to `workspace` and are added in a fixed order; every path is
 * bitwise reproducible run to run.  workspace_bytes must be >= w4a16_gemm_workspace_bytes(...);
 * workspace may be NULL if that is 0. */
w4a16_status_t w4a16_gemm(w4a16_format_t fmt, w4a16_dtype_t act, const void* x, int64_t M,
                          const void* codes, const void* scales, const void* mins, int64_t N,
                          int64_t K, void* y, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Dispatch on M (vidyal.ai "How the measurements were taken": a GEMV kernel for one row, tiles
 * chosen per M; anrans "Exercises": kernels chosen by batch size): M <= w4a16_matmul_gemv_cutoff()
 * goes to w4a16_gemv, larger M to w4a16_gemm.  Q4, the zero-point format and W8 take the GEMV
 * path up to w4a16_gemv_max_rows() rows and w4a16_gemm above (fp16 activations).  Workspace as for
 * w4a16_gemm (w4a16_gemm_workspace_bytes of the same shape is always enough).  Up to 16 rows of
 * G128, where N is small enough that the GEMV's column blocks would leave CUs idle (fewer than
 * 192 blocks of 32 columns) and the codes are at least 16 MiB, a workspace of that size lets the
 * small-M kernel split K over 2..8 blocks per 64 columns, the fp32 partials summed in split order
 * by a second launch; without one (NULL or too small) the call runs w4a16_gemv.  Both results
 * are bitwise reproducible; they differ from each other in fp32 rounding only. */
w4a16_status_t w4a16_matmul(w4a16_format_t fmt, w4a16_dtype_t act, const void* x, int64_t M,
                            const void* codes, const void* scales, const void* mins, int64_t N,
                            int64_t K, void* y, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* The M at and below which w4a16_matmul takes the GEMV path for the G128 format. */
int64_t w4a16_matmul_gemv_cutoff(void);

/* ---- A prepared copy of the zero-point format -------------------------------------------------
 * The weights rearranged once, at load time, into the order the small-M kernel reads them, with
 * the group parameters decoded to fp32 beside them (anrans.github.io "Quantization and GEMV",
 * "What production kernels do": reorder the weights offline so that the kernel's loads land the
 * data its matrix-core fragments need; secemp.blog "Hardware-invariant NVFP4 progress report 1",
 * "Is it faster?": decode the scales once at load time and keep them as plain fp32 next to the
 * packed weights).  The canonical zero-point arrays stay the format and the reference: the copy
 * holds word (r, n) = codes[n][r] in [K/8][N] order, s[g][n] = scales[n][g] and
 * m[g][n] = -zeros[n][g] * s[g][n] as fp32 [K/128][N], each part starting 16-byte aligned.
 * With z an integer of magnitude at most 2048 (as the quantizer stores it), (q - z) s = q s + m is
 * exact in fp32 (|q - z| has at most 12 significant bits and s 11), so fmaf(q, s, m) reproduces
 * the format's decode bit for bit.  The copy costs 4 + 64/128 = 4.5 bits per weight against the
 * canonical 4 + 32/128 = 4.25.
 * Only W4A16_FMT_G128_ZP_FP16 has a prepared form; the others return 0 / W4A16_ERR_UNSUPPORTED
 * (the G128 format is already stored in that order, so a copy would change nothing). */

/* Bytes of the prepared copy of an N x K weight in `fmt` (0 if the format or shape has none). */
size_t w4a16_prepared_bytes(w4a16_format_t fmt, int64_t N, int64_t K);

/* Write the prepared copy of the packed weights (codes, scales, mins = zero points, as
 * w4a16_quantize_pack wrote them) into `prepared` (device, caller-owned, 16-byte aligned,
 * prepared_bytes >= w4a16_prepared_bytes(fmt, N, K)).  Asynchronous on `stream`; the copy is a
 * pure function of the packed arrays and is valid until they change.  Errors: ERR_INVALID (shape,
 * alignment, size), ERR_UNSUPPORTED (a format with no prepared form, N or K past the limits),
 * ERR_DEVICE. */
w4a16_status_t w4a16_prepare(w4a16_format_t fmt, const void* codes, const void* scales, const void* mins,
                             int64_t N, int64_t K, void* prepared, size_t prepared_bytes,
                             hipStream_t stream);

/* y [M][N] = x [M][K] . W_hat^T from the prepared copy, any M >= 1, for bf16 or fp16 activations;
 * y has the activations' type.  The kernels are the G128 ones for up to 16, 17..32 and 33..64 rows
 * (one pass over the copy per 64 rows where N % 4 == 0 and K % 256 == 0, else per 32 rows; the last
 * 1..16 rows in a pass of their own): the inner sums run on
 * the matrix cores against 128 + q (bf16) or 1024 + q (fp16), and each group adds
 * s * sum(x (offset + q)) + (m - offset s) * sum(x) in fp32.
 * Up to the order of fp32 additions this is the product on the canonical zero-point arrays; it is
 * bitwise reproducible run to run.  Errors: ERR_INVALID (shape, M, alignment, act),
 * ERR_UNSUPPORTED (fp32 activations, other formats, N or K past the limits), ERR_DEVICE. */
w4a16_status_t w4a16_gemv_prepared(w4a16_format_t fmt, w4a16_dtype_t act, const void* x, int64_t M,
                                   const void* prepared, int64_t N, int64_t K, void* y,
                                   hipStream_t stream);

/* For callers that cannot allocate device memory -- code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc: w4a16_matmul with no workspace argument.  Where the
 * large-M GEMM splits K, its partial sums go to a scratch array inside the library: one per GPU,
 * w4a16_matmul_noalloc_max_scratch_bytes() (16 MiB) in size, part of the library's device data from
 * the first call on that GPU until the process ends.  A shape whose split needs more than that
 * (w4a16_gemm_workspace_bytes of the shape) returns W4A16_ERR_UNSUPPORTED before any launch: use
 * w4a16_matmul with a workspace.  Every call on one GPU shares that GPU's array, so calls that may
 * run at the same time on one GPU (different streams, different host threads) race on it and
 * must not overlap.  No call allocates or frees anything; the first call on each GPU looks up the
 * array's device address (hipGetSymbolAddress, with that GPU current) and keeps it.  Results are
 * bit-identical to w4a16_matmul's; other arguments and errors as for w4a16_matmul. */
w4a16_status_t w4a16_matmul_noalloc(w4a16_format_t fmt, w4a16_dtype_t act, const void* x, int64_t M,
                                    const void* codes, const void* scales, const void* mins, int64_t N,
                                    int64_t K, void* y, hipStream_t stream);

/* Size of w4a16_matmul_noalloc's per-GPU scratch array in bytes. */
size_t w4a16_matmul_noalloc_max_scratch_bytes(void);

/* ---- W4A8: int8 activations against the same 4-bit weights ------------------------------------
 * vidyal.ai "Low-Precision Kernels", "INT8 on a GeForce chip" and "The cost of quantizing
 * activations": the activations are quantized to int8 per row on every call, the integer
 * products are summed in 32 bits on the matrix cores, and the activation and weight scales are
 * applied to those sums in the epilogue. */

/* Per-row symmetric int8 quantization of bf16 activations x [M][K] (K % 128 == 0):
 *   ascale [M]         a_m = max_k |x[m][k]| / 127 in fp32 (IEEE division); 1.0 for a zero row
 *   xq     [M][K] int8 clamp(rint(x / a_m), -127, 127), ties to even (IEEE division)
 *   xsum   [K/128][M]  fp32, the exact integer sum of xq over each group of 128 k (for the
 *                      minimum term of the G128 weights)
 * Bit-identical to the CPU definition.  All pointers 16-byte aligned device memory; M*K < 2^31.
 * x must be finite (non-finite input is undefined). */
w4a16_status_t w4a16_quantize_act_i8(const void* x, int64_t M, int64_t K, int8_t* xq, float* ascale, float* xsum,
                                     hipStream_t stream);

/* W4A8 product with G128 weights: y [M][N] bf16 = round_to_nearest_even(
 *     a_m * sum_g (s[g][n] * sum_{k in g} xq[m][k] q[k][n] + min[g][n] * xsum[g][m])),
 * the integer sums exact (on the int8 matrix cores: v_mfma_i32_16x16x64_i8 in blocks of 16 rows
 * for up to 64 rows, where the weight stream sets the time, v_mfma_i32_32x32x32_i8 tiles above),
 * the rest in fp32.
 * Inputs as written by
 * w4a16_quantize_act_i8 for the same M and K.  G128 only (ERR_UNSUPPORTED otherwise); N % 4 == 0
 * and the 32-bit offset limits M*K, K*N/2, (K/128)*M*4 < 2^31 (ERR_UNSUPPORTED otherwise).  No
 * workspace; bitwise reproducible run to run. */
w4a16_status_t w4a16_gemm_w4a8(w4a16_format_t fmt, const int8_t* xq, const float* ascale, const float* xsum,
                               int64_t M, const void* codes, const void* scales, const void* mins, int64_t N,
                               int64_t K, void* y, hipStream_t stream);

/* W4A8 with the activation quantization fused into the product, for one activation row:
 * y [M][N] bf16 = w4a16_gemm_w4a8 of the codes, row scales and group sums that
 * w4a16_quantize_act_i8 would write for x, bit for bit, in one launch and with no intermediate
 * buffers (vidyal.ai "Low-Precision Kernels", "The cost of quantizing activations": the
 * quantization is paid on every call).  x: bf16 [M][K] with M == 1 (ERR_UNSUPPORTED above: use
 * the two calls).  G128 only, N % 4 == 0, K*N/2 < 2^31 (ERR_UNSUPPORTED otherwise).  No workspace;
 * bitwise reproducible run to run. */
w4a16_status_t w4a16_matmul_w4a8(w4a16_format_t fmt, const void* x, int64_t M, const void* codes, const void* scales,
                                 const void* mins, int64_t N, int64_t K, void* y, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
