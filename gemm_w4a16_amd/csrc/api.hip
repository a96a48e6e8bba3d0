// api.hip -- the C ABI of libw4a16: argument validation, dispatch by M, launches.
// Every check runs on the host before anything is enqueued; see include/w4a16.h for the
// contract of each entry point.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/w4a16.h"
#include "launch.h"

namespace {

constexpr int64_t kGroupG128 = 128;
constexpr int64_t kBlockQ4 = 32;
constexpr int64_t kW8RowAlign = 16;  // int8 rows are whole 16-byte loads
// Largest extents the kernels index with 32-bit ints (element offsets stay 64-bit).
constexpr int64_t kMaxDim = (int64_t)1 << 30;
// Largest N and K this build runs: the kernels address a tile's operands as a 64-bit base plus a
// 32-bit per-lane byte offset, which spans up to 16 * N bytes of packed words (a lane's rows in
// the small-M kernels) and 512 * K bytes of activations (a 256-row GEMM tile).  Both limits are
// far above any layer shape (67 M output columns, 4 M inputs).
constexpr int64_t kMaxN = (int64_t)1 << 26;
constexpr int64_t kMaxK = (int64_t)1 << 22;
// M at and below which w4a16_matmul uses the GEMV path for G128 (from the batch sweep).
constexpr int64_t kGemvCutoff = 16;
// Rows the fused W4A8 product quantizes inside its kernel: one, the batch-one case (each wave
// quantizes every row of its groups, so the work and the registers grow with M).
constexpr int64_t kW4A8FusedMaxRows = 1;

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t group_of(w4a16_format_t fmt) {
    return fmt == W4A16_FMT_Q4_B32_SYM_FP16 ? kBlockQ4 : fmt == W4A16_FMT_W8_ROW_FP32 ? kW8RowAlign : kGroupG128;
}

// Formats with no third array (Q4, W8): `mins` must be NULL.
bool has_mins(w4a16_format_t fmt) { return fmt == W4A16_FMT_G128_ASYM_BF16 || fmt == W4A16_FMT_G128_ZP_FP16; }

bool valid_format(w4a16_format_t fmt) {
    return fmt == W4A16_FMT_G128_ASYM_BF16 || fmt == W4A16_FMT_Q4_B32_SYM_FP16 || fmt == W4A16_FMT_G128_ZP_FP16 ||
           fmt == W4A16_FMT_W8_ROW_FP32;
}

w4a16_status_t check_shape(w4a16_format_t fmt, int64_t N, int64_t K) {
    if (!valid_format(fmt)) return W4A16_ERR_INVALID;
    if (N <= 0 || K <= 0 || N > kMaxDim || K > kMaxDim) return W4A16_ERR_INVALID;
    if (K % group_of(fmt) != 0) return W4A16_ERR_INVALID;
    if (N > kMaxN || K > kMaxK) return W4A16_ERR_UNSUPPORTED;
    return W4A16_OK;
}

// Packed weights: codes and scales always; minimums (G128) or zero points (ZP), NULL otherwise.
w4a16_status_t check_packed(w4a16_format_t fmt, const void* codes, const void* scales, const void* mins) {
    if (!aligned16(codes) || !aligned16(scales)) return W4A16_ERR_INVALID;
    if (has_mins(fmt) ? !aligned16(mins) : mins != nullptr) return W4A16_ERR_INVALID;
    return W4A16_OK;
}

w4a16_status_t check_act(w4a16_format_t fmt, w4a16_dtype_t act) {
    if (act != W4A16_BF16 && act != W4A16_FP16 && act != W4A16_FP32) return W4A16_ERR_INVALID;
    if (fmt == W4A16_FMT_G128_ASYM_BF16 && act != W4A16_BF16) return W4A16_ERR_UNSUPPORTED;
    if (fmt != W4A16_FMT_G128_ASYM_BF16 && act == W4A16_FP32) return W4A16_ERR_UNSUPPORTED;
    if (fmt == W4A16_FMT_W8_ROW_FP32 && act != W4A16_FP16) return W4A16_ERR_UNSUPPORTED;
    return W4A16_OK;
}

w4a16_status_t from_hip(hipError_t e) { return e == hipSuccess ? W4A16_OK : W4A16_ERR_DEVICE; }

// Largest fp32 values that still round to a finite 16-bit value under round-to-nearest-even: the
// midpoints between each format's largest finite value and the next power of two round up (to
// even, i.e. to infinity).  fp16: 65504 and 65536 -> 65520.  bf16: 0x7F7F and 2^128 -> fp32 bits
// 0x7F7F8000.
bool fits_fp16(float v) { return std::fabs(v) < 65520.0f; }
bool fits_bf16(float v) {
    uint32_t u;
    std::memcpy(&u, &v, 4);
    return (u & 0x7FFFFFFFu) < 0x7F7F8000u;
}

// W4A16_DEBUG_CHECKS set to anything but "0" turns on the quantizers' host-side weight check.
bool debug_checks_enabled() {
    const char* v = std::getenv("W4A16_DEBUG_CHECKS");
    return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
}

w4a16_status_t check_matmul_common(w4a16_format_t fmt, w4a16_dtype_t act, const void* x, int64_t M,
                                   const void* codes, const void* scales, const void* mins, int64_t N, int64_t K,
                                   const void* y) {
    w4a16_status_t st = check_shape(fmt, N, K);
    if (st != W4A16_OK) return st;
    if (M <= 0 || M > kMaxDim) return W4A16_ERR_INVALID;
    if (!aligned16(x) || !aligned16(y)) return W4A16_ERR_INVALID;
    st = check_packed(fmt, codes, scales, mins);
    if (st != W4A16_OK) return st;
    return check_act(fmt, act);
}

// Q4, the zero-point format and W8 with fp16 activations: every row of x against one weight pass
// (16 rows per pass over the weights) on the fp16 matrix cores.
w4a16_status_t launch_rowmajor_rows(w4a16_format_t fmt, const void* x, int64_t M, const void* codes,
                                    const void* scales, const void* mins, int64_t N, int64_t K, void* y,
                                    hipStream_t stream) {
    const uint16_t* xa = static_cast<const uint16_t*>(x);
    uint16_t* ya = static_cast<uint16_t*>(y);
    if (fmt == W4A16_FMT_Q4_B32_SYM_FP16)
        return from_hip(w4a16::launch_rowmma_q4b32(xa, M, static_cast<const uint8_t*>(codes),
                                                   static_cast<const uint16_t*>(scales), N, K, ya, stream));
    if (fmt == W4A16_FMT_G128_ZP_FP16)
        return from_hip(w4a16::launch_rowmma_g128zp(xa, M, static_cast<const uint32_t*>(codes),
                                                    static_cast<const uint16_t*>(scales),
                                                    static_cast<const uint16_t*>(mins), N, K, ya, stream));
    return from_hip(w4a16::launch_rowmma_w8row(xa, M, static_cast<const int8_t*>(codes),
                                               static_cast<const float*>(scales), N, K, ya, stream));
}

// ---- The no-allocation entry point's scratch buffer -------------------------------------------
// Split-K partial sums of the large-M GEMM for callers that cannot allocate a workspace.  One
// array per GPU, in the code object's zero-initialised device data, held until the process ends.
constexpr size_t kScratchBytes = (size_t)16 << 20;
__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

// `scratch` names a host-side stand-in in host code: its device address is looked up once per
// device, with that device current, and only that address is passed to kernels.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the device that runs `stream` (the current device for the null stream).
w4a16_status_t scratch_for_stream(hipStream_t stream, float** out) {
    int cur = 0, dev = 0;
    if (hipGetDevice(&cur) != hipSuccess) return W4A16_ERR_DEVICE;
    dev = cur;
    if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) return W4A16_ERR_DEVICE;
    if (dev < 0 || dev >= kMaxDevices) return W4A16_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return W4A16_ERR_DEVICE;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return W4A16_ERR_DEVICE;
        if (e != hipSuccess || p == nullptr) return W4A16_ERR_DEVICE;
        g_scratch_ptr[dev] = static_cast<float*>(p);
    }
    *out = g_scratch_ptr[dev];
    return W4A16_OK;
}

}  // namespace

extern "C" {

const char* w4a16_status_string(w4a16_status_t status) {
    switch (status) {
        case W4A16_OK: return "ok";
        case W4A16_ERR_INVALID: return "invalid argument";
        case W4A16_ERR_UNSUPPORTED: return "unsupported combination";
        case W4A16_ERR_DEVICE: return "HIP launch error";
    }
    return "unknown status";
}

w4a16_status_t w4a16_packed_sizes(w4a16_format_t fmt, int64_t N, int64_t K, size_t* codes_bytes,
                                  size_t* scales_bytes, size_t* mins_bytes) {
    const w4a16_status_t st = check_shape(fmt, N, K);
    if (st != W4A16_OK) return st;
    if (fmt == W4A16_FMT_W8_ROW_FP32) {  // one byte per weight and an fp32 scale per row
        if (codes_bytes) *codes_bytes = (size_t)N * (size_t)K;
        if (scales_bytes) *scales_bytes = (size_t)N * 4;
        if (mins_bytes) *mins_bytes = 0;
        return W4A16_OK;
    }
    const size_t codes = (size_t)N * (size_t)K / 2;  // 4 bits per weight in the other formats
    size_t scales = (size_t)N * (size_t)(K / group_of(fmt)) * 2;
    // G128: the GEMM reads scales and minimums as aligned 4-byte words, so an odd element count
    // gets 2 bytes of padding (never written, never used)
    if (fmt == W4A16_FMT_G128_ASYM_BF16) scales = (scales + 3) & ~(size_t)3;
    const size_t mins = has_mins(fmt) ? scales : 0;  // minimums or zero points
    if (codes_bytes) *codes_bytes = codes;
    if (scales_bytes) *scales_bytes = scales;
    if (mins_bytes) *mins_bytes = mins;
    return W4A16_OK;
}

w4a16_status_t w4a16_check_weights(w4a16_format_t fmt, const float* W, int64_t N, int64_t K) {
    const w4a16_status_t st = check_shape(fmt, N, K);
    if (st != W4A16_OK) return st;
    if (W == nullptr) return W4A16_ERR_INVALID;
    // one pass per row and group: the group's range (G128, zero point) or largest magnitude
    // (Q4, W8), then the stored parameter the quantizer would form from it
    const int64_t span = fmt == W4A16_FMT_W8_ROW_FP32 ? K : group_of(fmt);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g0 = 0; g0 < K; g0 += span) {
            const float* w = W + n * K + g0;
            float lo = w[0], hi = w[0], amax = 0.0f;
            for (int64_t j = 0; j < span; ++j) {
                if (!std::isfinite(w[j])) return W4A16_ERR_INVALID;
                lo = std::min(lo, w[j]);
                hi = std::max(hi, w[j]);
                amax = std::max(amax, std::fabs(w[j]));
            }
            switch (fmt) {
                case W4A16_FMT_G128_ASYM_BF16:
                    if (!fits_bf16((hi - lo) / 15.0f) || !fits_bf16(lo)) return W4A16_ERR_INVALID;
                    break;
                case W4A16_FMT_G128_ZP_FP16:
                    if (!fits_fp16((hi - lo) / 15.0f)) return W4A16_ERR_INVALID;
                    break;
                case W4A16_FMT_Q4_B32_SYM_FP16:
                    if (!fits_fp16(amax / 7.0f)) return W4A16_ERR_INVALID;
                    break;
                default:  // W8: an fp32 scale max|w| / 127 is always finite
                    break;
            }
        }
    }
    return W4A16_OK;
}

w4a16_status_t w4a16_quantize_pack(w4a16_format_t fmt, const float* W, int64_t N, int64_t K, void* codes,
                                   void* scales, void* mins, hipStream_t stream) {
    w4a16_status_t st = check_shape(fmt, N, K);
    if (st != W4A16_OK) return st;
    if (!aligned16(W)) return W4A16_ERR_INVALID;
    st = check_packed(fmt, codes, scales, mins);
    if (st != W4A16_OK) return st;
    w4a16::clear_stale_error();
    if (debug_checks_enabled()) {  // debug only: a synchronous copy of W to the host
        std::vector<float> host((size_t)N * (size_t)K);
        if (hipStreamSynchronize(stream) != hipSuccess ||
            hipMemcpy(host.data(), W, host.size() * sizeof(float), hipMemcpyDeviceToHost) != hipSuccess)
            return W4A16_ERR_DEVICE;
        st = w4a16_check_weights(fmt, host.data(), N, K);
        if (st != W4A16_OK) return st;
    }
    if (fmt == W4A16_FMT_G128_ASYM_BF16)
        return from_hip(w4a16::launch_pack_g128(W, N, K, static_cast<uint32_t*>(codes), static_cast<uint16_t*>(scales),
                                                static_cast<uint16_t*>(mins), stream));
    if (fmt == W4A16_FMT_W8_ROW_FP32)
        return from_hip(w4a16::launch_pack_w8row(W, N, K, static_cast<int8_t*>(codes), static_cast<float*>(scales),
                                                 stream));
    if (fmt == W4A16_FMT_G128_ZP_FP16)
        return from_hip(w4a16::launch_pack_g128zp(W, N, K, static_cast<uint32_t*>(codes),
                                                  static_cast<uint16_t*>(scales), static_cast<uint16_t*>(mins),
                                                  stream));
    return from_hip(w4a16::launch_pack_q4b32(W, N, K, static_cast<uint8_t*>(codes), static_cast<uint16_t*>(scales),
                                             stream));
}

w4a16_status_t w4a16_dequant(w4a16_format_t fmt, const void* codes, const void* scales, const void* mins, int64_t N,
                             int64_t K, w4a16_dtype_t out_dtype, void* W_hat, hipStream_t stream) {
    w4a16_status_t st = check_shape(fmt, N, K);
    if (st != W4A16_OK) return st;
    st = check_packed(fmt, codes, scales, mins);
    if (st != W4A16_OK) return st;
    if (!aligned16(W_hat)) return W4A16_ERR_INVALID;
    if (out_dtype != W4A16_BF16 && out_dtype != W4A16_FP16 && out_dtype != W4A16_FP32) return W4A16_ERR_INVALID;
    const int dt = (int)out_dtype;
    w4a16::clear_stale_error();
    if (fmt == W4A16_FMT_G128_ASYM_BF16)
        return from_hip(w4a16::launch_dequant_g128(static_cast<const uint32_t*>(codes),
                                                   static_cast<const uint16_t*>(scales),
                                                   static_cast<const uint16_t*>(mins), N, K, dt, W_hat, stream));
    if (fmt == W4A16_FMT_W8_ROW_FP32)
        return from_hip(w4a16::launch_dequant_w8row(static_cast<const int8_t*>(codes), static_cast<const float*>(scales),
                                                    N, K, dt, W_hat, stream));
    if (fmt == W4A16_FMT_G128_ZP_FP16)
        return from_hip(w4a16::launch_dequant_g128zp(static_cast<const uint32_t*>(codes),
                                                     static_cast<const uint16_t*>(scales),
                                                     static_cast<const uint16_t*>(mins), N, K, dt, W_hat, stream));
    return from_hip(w4a16::launch_dequant_q4b32(static_cast<const uint8_t*>(codes),
                                                static_cast<const uint16_t*>(scales), N, K, dt, W_hat, stream));
}

int64_t w4a16_gemv_max_rows(void) { return w4a16::kGemvMaxRows; }

int64_t w4a16_matmul_gemv_cutoff(void) { return kGemvCutoff; }

w4a16_status_t w4a16_gemv(w4a16_format_t fmt, w4a16_dtype_t act, const void* x, int64_t M, const void* codes,
                          const void* scales, const void* mins, int64_t N, int64_t K, void* y, hipStream_t stream) {
    const w4a16_status_t st = check_matmul_common(fmt, act, x, M, codes, scales, mins, N, K, y);
    if (st != W4A16_OK) return st;
    if (M > w4a16::kGemvMaxRows) return W4A16_ERR_UNSUPPORTED;
    w4a16::clear_stale_error();
    if (fmt == W4A16_FMT_G128_ASYM_BF16) {
        return from_hip(w4a16::launch_skinny_g128(static_cast<const uint16_t*>(x), M,
                                                  static_cast<const uint32_t*>(codes),
                                                  static_cast<const uint16_t*>(scales),
                                                  static_cast<const uint16_t*>(mins), N, K, static_cast<uint16_t*>(y),
                                                  stream));
    }
    // up to four fp16 rows (two for the zero-point format): one pass of the row-major GEMV with
    // all of them (faster than the matrix-core kernel's 16-row pass); more rows: the matrix cores
    const int64_t gemv_rows = fmt == W4A16_FMT_G128_ZP_FP16 ? w4a16::kRowGemvRowsZP : w4a16::kRowGemvRows;
    if (M > gemv_rows && act == W4A16_FP16) return launch_rowmajor_rows(fmt, x, M, codes, scales, mins, N, K, y, stream);
    if (fmt == W4A16_FMT_W8_ROW_FP32)
        return from_hip(w4a16::launch_gemv_w8row(static_cast<const uint16_t*>(x), M, static_cast<const int8_t*>(codes),
                                                 static_cast<const float*>(scales), N, K, static_cast<uint16_t*>(y),
                                                 stream));
    if (fmt == W4A16_FMT_G128_ZP_FP16)
        return from_hip(w4a16::launch_gemv_g128zp(static_cast<const uint16_t*>(x), M, act == W4A16_FP16,
                                                  static_cast<const uint32_t*>(codes), static_cast<const uint16_t*>(scales),
                                                  static_cast<const uint16_t*>(mins), N, K, static_cast<uint16_t*>(y),
                                                  stream));
    return from_hip(w4a16::launch_gemv_q4b32(static_cast<const uint16_t*>(x), M, act == W4A16_FP16,
                                             static_cast<const uint8_t*>(codes), static_cast<const uint16_t*>(scales),
                                             N, K, static_cast<uint16_t*>(y), stream));
}

size_t w4a16_gemm_workspace_bytes(w4a16_format_t fmt, int64_t M, int64_t N, int64_t K) {
    if (fmt != W4A16_FMT_G128_ASYM_BF16 || check_shape(fmt, N, K) != W4A16_OK || M <= 0 || M > kMaxDim) return 0;
    // the large-M GEMM's split-K partials, or the optional K split of the small-M (w4a16_matmul)
    // and 17..64-row kernels
    return std::max({w4a16::gemm_g128_workspace_bytes(M, N, K), w4a16::skinny_split_workspace_bytes(M, N, K),
                     w4a16::mid_split_workspace_bytes(M, N, K)});
}

w4a16_status_t w4a16_gemm(w4a16_format_t fmt, w4a16_dtype_t act, const void* x, int64_t M, const void* codes,
                          const void* scales, const void* mins, int64_t N, int64_t K, void* y, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    const w4a16_status_t st = check_matmul_common(fmt, act, x, M, codes, scales, mins, N, K, y);
    if (st != W4A16_OK) return st;
    if (fmt != W4A16_FMT_G128_ASYM_BF16) {  // the row-major formats: fp16 activations, no workspace
        if (act != W4A16_FP16) return W4A16_ERR_UNSUPPORTED;
        w4a16::clear_stale_error();
        return launch_rowmajor_rows(fmt, x, M, codes, scales, mins, N, K, y, stream);
    }
    const size_t need = w4a16::gemm_g128_workspace_bytes(M, N, K);
    if (need > 0 && (workspace_bytes < need || !aligned16(workspace))) return W4A16_ERR_INVALID;
    w4a16::clear_stale_error();
    // 17..64 rows at small N: K split over blocks when the workspace holds the partials (else the
    // unsplit kernel, which needs none)
    const size_t mid_need = w4a16::mid_split_workspace_bytes(M, N, K);
    if (mid_need > 0 && workspace_bytes >= mid_need && aligned16(workspace))
        return from_hip(w4a16::launch_mid_g128_split(static_cast<const uint16_t*>(x), M,
                                                     static_cast<const uint32_t*>(codes),
                                                     static_cast<const uint16_t*>(scales),
                                                     static_cast<const uint16_t*>(mins), N, K,
                                                     static_cast<uint16_t*>(y), static_cast<float*>(workspace), stream));
    return from_hip(w4a16::launch_gemm_g128(static_cast<const uint16_t*>(x), M, static_cast<const uint32_t*>(codes),
                                            static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(mins),
                                            N, K, static_cast<uint16_t*>(y), static_cast<float*>(workspace), stream));
}

w4a16_status_t w4a16_matmul(w4a16_format_t fmt, w4a16_dtype_t act, const void* x, int64_t M, const void* codes,
                            const void* scales, const void* mins, int64_t N, int64_t K, void* y, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    // G128 by the cutoff; the row-major formats take the GEMV up to its row limit, and above it
    // w4a16_gemm (fp16 activations)
    const int64_t cut = fmt == W4A16_FMT_G128_ASYM_BF16 ? kGemvCutoff : w4a16::kGemvMaxRows;
    if (M > 0 && M <= cut) {
        // G128 with a workspace: the small-M kernel with K split over blocks where its column
        // blocks alone would leave CUs idle; without one (or short of it), the GEMV
        const size_t need = fmt == W4A16_FMT_G128_ASYM_BF16 ? w4a16::skinny_split_workspace_bytes(M, N, K) : 0;
        if (need > 0 && workspace_bytes >= need && aligned16(workspace)) {
            const w4a16_status_t st = check_matmul_common(fmt, act, x, M, codes, scales, mins, N, K, y);
            if (st != W4A16_OK) return st;
            w4a16::clear_stale_error();
            return from_hip(w4a16::launch_skinny_g128_split(
                static_cast<const uint16_t*>(x), M, static_cast<const uint32_t*>(codes),
                static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(mins), N, K, static_cast<uint16_t*>(y),
                static_cast<float*>(workspace), w4a16::skinny_splits(M, N, K), stream));
        }
        return w4a16_gemv(fmt, act, x, M, codes, scales, mins, N, K, y, stream);
    }
    return w4a16_gemm(fmt, act, x, M, codes, scales, mins, N, K, y, workspace, workspace_bytes, stream);
}

// The prepared copy's three parts, each starting 16-byte aligned: words, fp32 scales, fp32 minimums.
struct PreparedLayout {
    size_t words, scales, mins, total;
};
static PreparedLayout prepared_layout(int64_t N, int64_t K) {
    auto a16 = [](size_t b) { return (b + 15) & ~(size_t)15; };
    PreparedLayout L;
    L.words = 0;
    L.scales = a16((size_t)(K / 8) * (size_t)N * 4);
    L.mins = L.scales + a16((size_t)(K / 128) * (size_t)N * 4);
    L.total = L.mins + a16((size_t)(K / 128) * (size_t)N * 4);
    return L;
}

size_t w4a16_prepared_bytes(w4a16_format_t fmt, int64_t N, int64_t K) {
    if (fmt != W4A16_FMT_G128_ZP_FP16 || check_shape(fmt, N, K) != W4A16_OK) return 0;
    return prepared_layout(N, K).total;
}

w4a16_status_t w4a16_prepare(w4a16_format_t fmt, const void* codes, const void* scales, const void* mins, int64_t N,
                             int64_t K, void* prepared, size_t prepared_bytes, hipStream_t stream) {
    w4a16_status_t st = check_shape(fmt, N, K);
    if (st != W4A16_OK) return st;
    if (fmt != W4A16_FMT_G128_ZP_FP16) return W4A16_ERR_UNSUPPORTED;
    if ((st = check_packed(fmt, codes, scales, mins)) != W4A16_OK) return st;
    const PreparedLayout L = prepared_layout(N, K);
    if (!aligned16(prepared) || prepared_bytes < L.total) return W4A16_ERR_INVALID;
    char* base = static_cast<char*>(prepared);
    w4a16::clear_stale_error();
    return from_hip(w4a16::launch_prepare_zp(static_cast<const uint32_t*>(codes), static_cast<const uint16_t*>(scales),
                                             static_cast<const uint16_t*>(mins), N, K,
                                             reinterpret_cast<uint32_t*>(base + L.words),
                                             reinterpret_cast<float*>(base + L.scales),
                                             reinterpret_cast<float*>(base + L.mins), stream));
}

w4a16_status_t w4a16_gemv_prepared(w4a16_format_t fmt, w4a16_dtype_t act, const void* x, int64_t M,
                                   const void* prepared, int64_t N, int64_t K, void* y, hipStream_t stream) {
    w4a16_status_t st = check_shape(fmt, N, K);
    if (st != W4A16_OK) return st;
    if (M <= 0 || M > kMaxDim) return W4A16_ERR_INVALID;
    if (!aligned16(x) || !aligned16(y) || !aligned16(prepared)) return W4A16_ERR_INVALID;
    if (act != W4A16_BF16 && act != W4A16_FP16 && act != W4A16_FP32) return W4A16_ERR_INVALID;
    if (fmt != W4A16_FMT_G128_ZP_FP16 || act == W4A16_FP32) return W4A16_ERR_UNSUPPORTED;
    const PreparedLayout L = prepared_layout(N, K);
    const char* base = static_cast<const char*>(prepared);
    w4a16::clear_stale_error();
    const bool f16 = act == W4A16_FP16;
    const uint32_t* words = reinterpret_cast<const uint32_t*>(base + L.words);
    const float* sp = reinterpret_cast<const float*>(base + L.scales);
    const float* mp = reinterpret_cast<const float*>(base + L.mins);
    // one pass over the copy per 64 rows (the 64-row kernel, where the shape fits) or 32 rows (the
    // 17..32-row kernel), the last 1..16 rows on the small-M kernel; after the first pass the copy
    // is read from the Infinity Cache when it fits
    const bool rows64 = w4a16::midr_fits(64, N, K);
    for (int64_t m0 = 0; m0 < M;) {
        const int64_t rem = M - m0;
        const int64_t mc = rem <= 32 ? rem : (rows64 ? std::min<int64_t>(rem, 64) : 32);
        const uint16_t* xa = static_cast<const uint16_t*>(x) + m0 * K;
        uint16_t* ya = static_cast<uint16_t*>(y) + m0 * N;
        hipError_t e;
        if (mc <= w4a16::kGemvMaxRows) e = w4a16::launch_skinny_prepared_zp(xa, mc, f16, words, sp, mp, N, K, ya, stream);
        else if (mc <= 32) e = w4a16::launch_rows32_prepared_zp(xa, mc, f16, words, sp, mp, N, K, ya, stream);
        else e = w4a16::launch_rows64_prepared_zp(xa, mc, f16, words, sp, mp, N, K, ya, stream);
        const w4a16_status_t st = from_hip(e);
        if (st != W4A16_OK) return st;
        m0 += mc;
    }
    return W4A16_OK;
}

size_t w4a16_matmul_noalloc_max_scratch_bytes(void) { return kScratchBytes; }

w4a16_status_t w4a16_matmul_noalloc(w4a16_format_t fmt, w4a16_dtype_t act, const void* x, int64_t M,
                                    const void* codes, const void* scales, const void* mins, int64_t N, int64_t K,
                                    void* y, hipStream_t stream) {
    w4a16_status_t st = check_matmul_common(fmt, act, x, M, codes, scales, mins, N, K, y);
    if (st != W4A16_OK) return st;
    const size_t need = w4a16_gemm_workspace_bytes(fmt, M, N, K);
    if (need > kScratchBytes) return W4A16_ERR_UNSUPPORTED;
    float* ws = nullptr;
    if (need > 0 && (st = scratch_for_stream(stream, &ws)) != W4A16_OK) return st;
    return w4a16_matmul(fmt, act, x, M, codes, scales, mins, N, K, y, ws, need, stream);
}

w4a16_status_t w4a16_quantize_act_i8(const void* x, int64_t M, int64_t K, int8_t* xq, float* ascale, float* xsum,
                                     hipStream_t stream) {
    if (M <= 0 || K <= 0 || M > kMaxDim || K > kMaxDim || K % kGroupG128 != 0) return W4A16_ERR_INVALID;
    if (M * K >= ((int64_t)1 << 31)) return W4A16_ERR_INVALID;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(ascale) || !aligned16(xsum)) return W4A16_ERR_INVALID;
    w4a16::clear_stale_error();
    return from_hip(w4a16::launch_quant_act_i8(static_cast<const uint16_t*>(x), M, K, xq, ascale, xsum, stream));
}

w4a16_status_t w4a16_gemm_w4a8(w4a16_format_t fmt, const int8_t* xq, const float* ascale, const float* xsum,
                               int64_t M, const void* codes, const void* scales, const void* mins, int64_t N,
                               int64_t K, void* y, hipStream_t stream) {
    if (w4a16_status_t st = check_shape(fmt, N, K); st != W4A16_OK) return st;
    if (M <= 0 || M > kMaxDim) return W4A16_ERR_INVALID;
    if (w4a16_status_t st = check_packed(fmt, codes, scales, mins); st != W4A16_OK) return st;
    if (!aligned16(xq) || !aligned16(ascale) || !aligned16(xsum) || !aligned16(y)) return W4A16_ERR_INVALID;
    if (fmt != W4A16_FMT_G128_ASYM_BF16 || N % 4 != 0) return W4A16_ERR_UNSUPPORTED;
    // the kernel's per-lane byte offsets are 32-bit
    if (M * K >= ((int64_t)1 << 31) || (K / 8) * N * 4 >= ((int64_t)1 << 31) || (K / 128) * M * 4 >= ((int64_t)1 << 31))
        return W4A16_ERR_UNSUPPORTED;
    w4a16::clear_stale_error();
    return from_hip(w4a16::launch_gemm_w4a8(xq, ascale, xsum, M, static_cast<const uint32_t*>(codes),
                                            static_cast<const uint16_t*>(scales), static_cast<const uint16_t*>(mins),
                                            N, K, static_cast<uint16_t*>(y), stream));
}

w4a16_status_t w4a16_matmul_w4a8(w4a16_format_t fmt, const void* x, int64_t M, const void* codes, const void* scales,
                                 const void* mins, int64_t N, int64_t K, void* y, hipStream_t stream) {
    if (w4a16_status_t st = check_shape(fmt, N, K); st != W4A16_OK) return st;
    if (M <= 0 || M > kMaxDim) return W4A16_ERR_INVALID;
    if (w4a16_status_t st = check_packed(fmt, codes, scales, mins); st != W4A16_OK) return st;
    if (!aligned16(x) || !aligned16(y)) return W4A16_ERR_INVALID;
    if (fmt != W4A16_FMT_G128_ASYM_BF16 || N % 4 != 0 || M > kW4A8FusedMaxRows) return W4A16_ERR_UNSUPPORTED;
    if ((K / 8) * N * 4 >= ((int64_t)1 << 31)) return W4A16_ERR_UNSUPPORTED;  // as w4a16_gemm_w4a8
    w4a16::clear_stale_error();
    return from_hip(w4a16::launch_matmul_w4a8_fused(static_cast<const uint16_t*>(x), M,
                                                    static_cast<const uint32_t*>(codes),
                                                    static_cast<const uint16_t*>(scales),
                                                    static_cast<const uint16_t*>(mins), N, K, static_cast<uint16_t*>(y),
                                                    stream));
}

}  // extern "C"
