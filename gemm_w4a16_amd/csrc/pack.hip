// pack.hip -- quantize/pack and reference dequant kernels for both weight formats.
//
// G128 (vidyal.ai "Low-Precision Kernels", Step 2): per (column n, group of 128 k):
//   lo/hi = min/max (a zero taken as +0), s = (hi - lo)/15 in fp32, s_b = bf16(s) (1.0 if 0),
//   m_b = bf16(lo), q = clamp(rint((w - m_b)/s_b), 0, 15), eight codes per word along k with
//   k = 8r in the lowest nibble, words stored [K/8][N].
// Q4B32 (thuongvuho.com "Why My 4-Bit CUDA Kernel Wasn't Faster", introduction and "Loading the
//   same bytes differently"): per (row n, block of 32 k): s = max|w|/7, s_h = fp16(s) (1.0 if
//   0), q = clamp(rint(w/s_h) + 8, 0, 15), byte j = q[2j] | q[2j+1] << 4.
//
// G128-ZP (anrans.github.io "Quantization and GEMV", "The quantization formulas" and "W4A16:
//   dequantizing in registers"): per (row n, group of 128 k): lo/hi as for G128, s = (hi-lo)/15,
//   s_h = fp16(s) (1.0 if 0), z = clamp(round(-lo/s_h), -2048, 2048) as fp16, q = clamp(round(w/s_h)
//   + z, 0, 15) with round half away from zero (the page's std::round), eight codes per word along
//   k, words stored [N][K/8].
// W8 (anrans.github.io "Quantization and GEMV", "Exercises", 1): per row n: s = max|w|/127 in
//   fp32 (1.0 for an all-zero row), q = clamp(round(w/s), -127, 127) as int8 [N][K], round half
//   away from zero.
//
// The arithmetic is IEEE fp32 with a correctly rounded divide (-fhip-fp32-correctly-rounded-
// divide-sqrt), rint = round-half-to-even, and no expression here is eligible for FMA
// contraction, so the codes are bit-identical to any other IEEE implementation of the rule.
#include "device_common.h"
#include "launch.h"

namespace w4a16 {

// ---- G128 quantize/pack -------------------------------------------------------------------
// Block: 256 threads = 64 columns x 4 quarters of a 128-k group; grid (ceil(N/64), K/128).
// Thread (c, p) reads W[n][128g + 32p .. +31] (8 x 16-byte loads), the 4 quarters of a column
// combine their min/max with two lane swaps, then each thread writes the 4 words of its
// quarter: packed rows 16g + 4p + i, column n.
__global__ __launch_bounds__(256) void pack_g128_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                        uint32_t* __restrict__ codes, uint16_t* __restrict__ scales,
                                                        uint16_t* __restrict__ mins) {
    const int c = threadIdx.x >> 2, p = threadIdx.x & 3;
    const int64_t n = (int64_t)blockIdx.x * 64 + c;
    const int64_t g = blockIdx.y;
    const bool live = n < N;
    const int64_t nr = live ? n : N - 1;  // clamped row for the loads; dead lanes store nothing
    const float4* src = reinterpret_cast<const float4*>(W + nr * K + g * 128 + p * 32);
    float w[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 v = src[i];
        w[4 * i] = v.x;
        w[4 * i + 1] = v.y;
        w[4 * i + 2] = v.z;
        w[4 * i + 3] = v.w;
    }
    float lo = w[0], hi = w[0];
#pragma unroll
    for (int j = 1; j < 32; ++j) {
        lo = fminf(lo, w[j]);
        hi = fmaxf(hi, w[j]);
    }
    lo = fminf(lo, __shfl_xor(lo, 1));
    hi = fmaxf(hi, __shfl_xor(hi, 1));
    lo = fminf(lo, __shfl_xor(lo, 2));
    hi = fmaxf(hi, __shfl_xor(hi, 2));
    if (lo == 0.0f) lo = 0.0f;  // -0 -> +0
    if (hi == 0.0f) hi = 0.0f;
    const float s = (hi - lo) / 15.0f;
    uint16_t s_b = f32_to_bf16_bits(s);
    if (bf16_bits_to_f32(s_b) == 0.0f) s_b = 0x3F80;
    const uint16_t m_b = f32_to_bf16_bits(lo);
    const float sf = bf16_bits_to_f32(s_b), mf = bf16_bits_to_f32(m_b);
    if (!live) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float t = __builtin_rintf((w[8 * i + j] - mf) / sf);
            const uint32_t q = t < 0.0f ? 0u : (t > 15.0f ? 15u : (uint32_t)t);
            word |= q << (4 * j);
        }
        codes[(g * 16 + p * 4 + i) * N + n] = word;
    }
    if (p == 0) {
        scales[g * N + n] = s_b;
        mins[g * N + n] = m_b;
    }
}

// ---- Q4B32 quantize/pack ------------------------------------------------------------------
// One thread per (row, block of 32); consecutive threads take consecutive blocks of a row, so
// the 128-byte reads and the 16-byte code stores are contiguous across the wave.
__global__ __launch_bounds__(256) void pack_q4b32_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                         uint8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
    const int64_t B = K / 32;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= N * B) return;
    const float4* src = reinterpret_cast<const float4*>(W + i * 32);  // row n, block b = i / B, i % B
    float w[32];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float4 v = src[j];
        w[4 * j] = v.x;
        w[4 * j + 1] = v.y;
        w[4 * j + 2] = v.z;
        w[4 * j + 3] = v.w;
    }
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) a = fmaxf(a, fabsf(w[j]));
    const float s = a / 7.0f;
    uint16_t s_h = f32_to_f16_bits(s);
    if (f16_bits_to_f32(s_h) == 0.0f) s_h = 0x3C00;
    const float sf = f16_bits_to_f32(s_h);
    uint32_t out[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float t = __builtin_rintf(w[8 * d + j] / sf) + 8.0f;
            const uint32_t q = t < 0.0f ? 0u : (t > 15.0f ? 15u : (uint32_t)t);
            word |= q << (4 * j);  // k = 8d + j: byte j/2, low nibble for even j
        }
        out[d] = word;
    }
    *reinterpret_cast<uint4*>(codes + i * 16) = make_uint4(out[0], out[1], out[2], out[3]);
    scales[i] = s_h;
}

// ---- G128-ZP quantize/pack ----------------------------------------------------------------
// Four consecutive threads per (row, group of 128): thread p reads k = 32p .. 32p+31 of the
// group (8 x 16-byte loads), the four combine their min/max with two lane swaps, and each writes
// its 4 words: the group's 16 words are 64 contiguous bytes of the row.
__global__ __launch_bounds__(256) void pack_g128zp_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                          uint32_t* __restrict__ codes, uint16_t* __restrict__ scales,
                                                          uint16_t* __restrict__ zeros) {
    const int64_t G = K / 128;
    const int64_t i = (int64_t)blockIdx.x * 64 + (threadIdx.x >> 2);  // (row, group) index
    const int p = threadIdx.x & 3;
    const bool live = i < N * G;
    const int64_t ii = live ? i : N * G - 1;  // clamped for the loads; dead lanes store nothing
    const float4* src = reinterpret_cast<const float4*>(W + ii * 128 + p * 32);  // row n = ii / G
    float w[32];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float4 v = src[j];
        w[4 * j] = v.x;
        w[4 * j + 1] = v.y;
        w[4 * j + 2] = v.z;
        w[4 * j + 3] = v.w;
    }
    float lo = w[0], hi = w[0];
#pragma unroll
    for (int j = 1; j < 32; ++j) {
        lo = fminf(lo, w[j]);
        hi = fmaxf(hi, w[j]);
    }
    lo = fminf(lo, __shfl_xor(lo, 1));
    hi = fmaxf(hi, __shfl_xor(hi, 1));
    lo = fminf(lo, __shfl_xor(lo, 2));
    hi = fmaxf(hi, __shfl_xor(hi, 2));
    if (lo == 0.0f) lo = 0.0f;  // -0 -> +0
    if (hi == 0.0f) hi = 0.0f;
    const float s = (hi - lo) / 15.0f;
    uint16_t s_h = f32_to_f16_bits(s);
    if ((s_h & 0x7FFFu) == 0) s_h = 0x3C00;  // a zero scale becomes 1.0
    const float sf = f16_bits_to_f32(s_h);
    float z = __builtin_roundf(-lo / sf);
    z = fminf(fmaxf(z, -2048.0f), 2048.0f);
    if (z == 0.0f) z = 0.0f;  // -0 -> +0
    const uint16_t z_h = f32_to_f16_bits(z);  // exact: an integer of magnitude <= 2048
    const float zf = f16_bits_to_f32(z_h);
    if (!live) return;
    uint32_t out[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float t = __builtin_roundf(w[8 * d + j] / sf) + zf;
            const uint32_t q = t < 0.0f ? 0u : (t > 15.0f ? 15u : (uint32_t)t);
            word |= q << (4 * j);
        }
        out[d] = word;
    }
    *reinterpret_cast<uint4*>(codes + i * 16 + p * 4) = make_uint4(out[0], out[1], out[2], out[3]);
    if (p == 0) {
        scales[i] = s_h;
        zeros[i] = z_h;
    }
}

// ---- W8 quantize/pack -------------------------------------------------------------------------
// One 256-thread block per row: a max-|w| reduction over the row (16-byte loads, lane swaps, LDS),
// then each thread writes 4 codes at a time.  K % 16 == 0.
__global__ __launch_bounds__(256) void pack_w8row_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                                                         int8_t* __restrict__ codes, float* __restrict__ scales) {
    __shared__ float wmax[4];
    const int64_t n = blockIdx.x;
    const float4* row = reinterpret_cast<const float4*>(W + n * K);
    const int64_t K4 = K / 4;
    float a = 0.0f;
    for (int64_t i = threadIdx.x; i < K4; i += 256) {
        const float4 v = row[i];
        a = fmaxf(a, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) a = fmaxf(a, __shfl_xor(a, o));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    float s = a / 127.0f;
    if (s == 0.0f) s = 1.0f;
    uint32_t* out = reinterpret_cast<uint32_t*>(codes + n * K);
    for (int64_t i = threadIdx.x; i < K4; i += 256) {
        const float4 v = row[i];
        const float w4[4] = {v.x, v.y, v.z, v.w};
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float r = fminf(fmaxf(__builtin_roundf(w4[j] / s), -127.0f), 127.0f);
            word |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * j);
        }
        out[i] = word;
    }
    if (threadIdx.x == 0) scales[n] = s;
}

// ---- reference dequant ----------------------------------------------------------------------
// Eight fp32 values -> out[idx .. idx+7] as bf16 (dtype 0), fp16 (1) or fp32 (2), each rounded
// to nearest even.
__device__ __forceinline__ void store8(void* out, int64_t idx, const float* v, int dtype) {
    if (dtype == 2) {  // fp32
        float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + idx);
        o[0] = make_float4(v[0], v[1], v[2], v[3]);
        o[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
        uint32_t p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            p[j] = dtype == 0 ? pack2_bf16(v[2 * j], v[2 * j + 1])
                              : ((uint32_t)f32_to_f16_bits(v[2 * j]) | ((uint32_t)f32_to_f16_bits(v[2 * j + 1]) << 16));
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + idx) = make_uint4(p[0], p[1], p[2], p[3]);
    }
}

// One thread per packed word (r, n): w_hat[n][8r .. 8r+7] = fmaf(q, s_b, m_b), then rounded.
__global__ __launch_bounds__(256) void dequant_g128_kernel(const uint32_t* __restrict__ codes,
                                                           const uint16_t* __restrict__ scales,
                                                           const uint16_t* __restrict__ mins, int64_t N, int64_t K,
                                                           int dtype, void* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (K / 8) * N) return;
    const int64_t r = i / N, n = i % N;
    const uint32_t word = codes[i];
    const float s = bf16_bits_to_f32(scales[(r / 16) * N + n]);
    const float m = bf16_bits_to_f32(mins[(r / 16) * N + n]);
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_fmaf((float)((word >> (4 * j)) & 0xFu), s, m);
    store8(out, n * K + r * 8, v, dtype);
}

// One thread per 8 codes of a Q4 block: w_hat = (q - 8) * s_h, exact in fp32, then rounded.
__global__ __launch_bounds__(256) void dequant_q4b32_kernel(const uint32_t* __restrict__ codes,
                                                            const uint16_t* __restrict__ scales, int64_t N, int64_t K,
                                                            int dtype, void* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // dword index = k/8 over all rows
    if (i >= N * (K / 8)) return;
    const uint32_t word = codes[i];
    const float s = f16_bits_to_f32(scales[i / 4]);  // 4 dwords per 32-k block
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (float)((int)((word >> (4 * j)) & 0xFu) - 8) * s;
    store8(out, i * 8, v, dtype);
}

// One thread per packed word (n, r): w_hat[n][8r .. 8r+7] = (q - z) * s (exact), then rounded.
__global__ __launch_bounds__(256) void dequant_g128zp_kernel(const uint32_t* __restrict__ codes,
                                                             const uint16_t* __restrict__ scales,
                                                             const uint16_t* __restrict__ zeros, int64_t N, int64_t K,
                                                             int dtype, void* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // word index over all rows
    if (i >= N * (K / 8)) return;
    const uint32_t word = codes[i];
    const float s = f16_bits_to_f32(scales[i / 16]), z = f16_bits_to_f32(zeros[i / 16]);  // 16 words per group
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ((float)((word >> (4 * j)) & 0xFu) - z) * s;
    store8(out, i * 8, v, dtype);
}

// One thread per 8 codes of a row: w_hat = q * s in fp32 (one rounding), then rounded to 16 bits.
__global__ __launch_bounds__(256) void dequant_w8row_kernel(const int8_t* __restrict__ codes,
                                                            const float* __restrict__ scales, int64_t N, int64_t K,
                                                            int dtype, void* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // index of 8 codes over all rows
    if (i >= N * (K / 8)) return;
    const uint2 c = reinterpret_cast<const uint2*>(codes)[i];
    const float s = scales[i / (K / 8)];
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (float)(int8_t)(((j < 4 ? c.x : c.y) >> (8 * (j & 3))) & 0xFFu) * s;
    store8(out, i * 8, v, dtype);
}

hipError_t launch_pack_w8row(const float* W, int64_t N, int64_t K, int8_t* codes, float* scales, hipStream_t stream) {
    hipLaunchKernelGGL(pack_w8row_kernel, dim3((unsigned)N), dim3(256), 0, stream, W, N, K, codes, scales);
    return hipGetLastError();
}

hipError_t launch_dequant_w8row(const int8_t* codes, const float* scales, int64_t N, int64_t K, int dtype, void* out,
                                hipStream_t stream) {
    const int64_t blocks = (N * (K / 8) + 255) / 256;
    hipLaunchKernelGGL(dequant_w8row_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, codes, scales, N, K, dtype,
                       out);
    return hipGetLastError();
}

hipError_t launch_pack_g128zp(const float* W, int64_t N, int64_t K, uint32_t* codes, uint16_t* scales,
                              uint16_t* zeros, hipStream_t stream) {
    const int64_t groups = N * (K / 128);
    hipLaunchKernelGGL(pack_g128zp_kernel, dim3((unsigned)((groups + 63) / 64)), dim3(256), 0, stream, W, N, K, codes,
                       scales, zeros);
    return hipGetLastError();
}

hipError_t launch_dequant_g128zp(const uint32_t* codes, const uint16_t* scales, const uint16_t* zeros, int64_t N,
                                 int64_t K, int dtype, void* out, hipStream_t stream) {
    const int64_t blocks = (N * (K / 8) + 255) / 256;
    hipLaunchKernelGGL(dequant_g128zp_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, codes, scales, zeros, N,
                       K, dtype, out);
    return hipGetLastError();
}

hipError_t launch_pack_g128(const float* W, int64_t N, int64_t K, uint32_t* codes, uint16_t* scales,
                            uint16_t* mins, hipStream_t stream) {
    const dim3 grid((unsigned)((N + 63) / 64), (unsigned)(K / 128));
    hipLaunchKernelGGL(pack_g128_kernel, grid, dim3(256), 0, stream, W, N, K, codes, scales, mins);
    return hipGetLastError();
}

hipError_t launch_pack_q4b32(const float* W, int64_t N, int64_t K, uint8_t* codes, uint16_t* scales,
                             hipStream_t stream) {
    const int64_t blocks = (N * (K / 32) + 255) / 256;
    hipLaunchKernelGGL(pack_q4b32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, W, N, K, codes, scales);
    return hipGetLastError();
}

hipError_t launch_dequant_g128(const uint32_t* codes, const uint16_t* scales, const uint16_t* mins, int64_t N,
                               int64_t K, int dtype, void* out, hipStream_t stream) {
    const int64_t blocks = ((K / 8) * N + 255) / 256;
    hipLaunchKernelGGL(dequant_g128_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, codes, scales, mins, N, K,
                       dtype, out);
    return hipGetLastError();
}

hipError_t launch_dequant_q4b32(const uint8_t* codes, const uint16_t* scales, int64_t N, int64_t K, int dtype,
                                void* out, hipStream_t stream) {
    const int64_t blocks = (N * (K / 8) + 255) / 256;
    hipLaunchKernelGGL(dequant_q4b32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const uint32_t*>(codes), scales, N, K, dtype, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// The prepared copy of the zero-point format: its words reordered into the [K/8][N] column order
// the small-M kernel streams (word (r, n) of the copy is word (n, r) of the format), with each
// group's parameters as fp32 s and m = -z s.  (q - z) s = q s + m exactly in fp32: |q - z| needs
// at most 12 bits and s 11, so q s, z s and their sum are all exact, and fmaf(q, s, m) is the
// format's decode bit for bit.
// ---------------------------------------------------------------------------------------------
// The word transpose goes through a 64 x 64-word LDS tile, so that both the reads (256 bytes of
// one weight row per 64 lanes) and the writes (256 bytes of one packed row) are whole lines.
constexpr int kTr = 64;
__global__ __launch_bounds__(256) void prepare_zp_words_kernel(const uint32_t* __restrict__ codes, int64_t N, int64_t K8,
                                                               uint32_t* __restrict__ out) {
    __shared__ uint32_t tile[kTr][kTr + 1];  // [n][r], padded: column reads hit distinct banks
    const int64_t n0 = (int64_t)blockIdx.x * kTr, r0 = (int64_t)blockIdx.y * kTr;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 lanes x 4 rows per step
#pragma unroll
    for (int i = 0; i < kTr / 4; ++i) {
        const int nn = 4 * i + ty;
        const int64_t n = n0 + nn, r = r0 + tx;
        if (n < N && r < K8) tile[nn][tx] = codes[n * K8 + r];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kTr / 4; ++i) {
        const int rr = 4 * i + ty;
        const int64_t r = r0 + rr, n = n0 + tx;
        if (n < N && r < K8) out[r * N + n] = tile[tx][rr];
    }
}

__global__ __launch_bounds__(256) void prepare_zp_params_kernel(const uint16_t* __restrict__ scales,
                                                                const uint16_t* __restrict__ zeros, int64_t N,
                                                                int64_t G, float* __restrict__ s_out,
                                                                float* __restrict__ m_out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // output (g, n), n fastest
    if (i >= N * G) return;
    const int64_t g = i / N, n = i % N;
    const float s = f16_bits_to_f32(scales[n * G + g]);
    const float z = f16_bits_to_f32(zeros[n * G + g]);
    s_out[i] = s;
    m_out[i] = -z * s;  // exact: an integer of at most 12 bits times 11 significant bits
}

hipError_t launch_prepare_zp(const uint32_t* codes, const uint16_t* scales, const uint16_t* zeros, int64_t N, int64_t K,
                             uint32_t* words, float* s_out, float* m_out, hipStream_t stream) {
    const int64_t K8 = K / 8, G = K / 128;
    hipLaunchKernelGGL(prepare_zp_words_kernel, dim3((unsigned)((N + kTr - 1) / kTr), (unsigned)((K8 + kTr - 1) / kTr)),
                       dim3(256), 0, stream, codes, N, K8, words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prepare_zp_params_kernel, dim3((unsigned)((N * G + 255) / 256)), dim3(256), 0, stream, scales, zeros,
                       N, G, s_out, m_out);
    return hipGetLastError();
}

}  // namespace w4a16
