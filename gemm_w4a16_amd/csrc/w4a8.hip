// w4a8.hip -- W4A8: int8 activations (quantized per row) against the G128 4-bit weights, on the
// int8 matrix cores.
//
// vidyal.ai "Low-Precision Kernels", "INT8 on a GeForce chip" and "The cost of quantizing
// activations": 8-bit integer products summed in 32 bits run at twice the rate of bf16 on the
// matrix cores; the activations have to be quantized on every call (absolute value, maximum per
// row, divide, round, convert), and both scales are applied to the integer sums in the matmul's
// epilogue rather than in a separate pass over an int32 result.
//
// quant_act_i8_kernel -- one block per row: a = max|x| / 127 (IEEE fp32 division, 1.0 for a zero
// row), xq = clamp(rint(x / a), -127, 127) with ties to even, and for each group of 128 k the exact
// sum of its xq (the epilogue's minimum term needs it, and the producer has the codes in hand).
//
// w4a8_gemm_kernel -- y = a_m * sum_g (s_g,n * sum_k xq q + min_g,n * X_g,m), one group of 128 k
// per k-tile:
//  * block tile 128 x 128, 4 waves side by side along N; a wave owns 128 rows x 32 columns as four
//    v_mfma_i32_32x32x32_i8 accumulators, restarted at zero every group, so each packed word is
//    unpacked once per block;
//  * every operand reaches LDS through direct-to-LDS copies issued two k-tiles ahead (three
//    stages): the 128 x 128-byte activation tile (16-byte chunks XOR-swizzled by row pair, so
//    the fragment reads are conflict-free), the 16 packed rows x 128 columns of weights as they
//    are stored (each copy of two packed rows 1152 bytes after the previous one, so that the two
//    copies a k-step reads sit on different banks), the group's 128 scales and minimums, and the
//    128 row sums X.  Each wave issues
//    seven copies per k-tile and one `s_waitcnt vmcnt` before the k-tile's barrier waits for
//    exactly its own copies of that k-tile;
//  * a lane's B fragment (32 k x 32 columns: 16 k of one column) is two consecutive packed words:
//    w & 0x0F0F0F0F and (w >> 4) & 0x0F0F0F0F hold the even and odd codes as bytes, and two
//    v_perm_b32 put them back in k order, matching the activation bytes;
//  * after a group's 4 k-steps each int32 sum becomes fp32 (exact: |sum| < 2^18) and enters the
//    fp32 accumulator as s * sum (one convert and one fma per output); the minimum term
//    sum_g min_g X_g is a [128 x G] x [G x 128] product of its own, run on v_mfma_f32_32x32x2f32
//    two groups at a time into the same accumulators, so it costs no VALU work per output;
//  * the row scale multiplies the total once at the end, and the tile leaves through LDS as
//    whole rows (16-byte stores of consecutive columns).
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace w4a16 {

namespace {

// ---- activation quantization ------------------------------------------------------------------

__global__ __launch_bounds__(256) void quant_act_i8_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                           int8_t* __restrict__ xq, float* __restrict__ ascale,
                                                           float* __restrict__ xsum) {
    __shared__ float red[4];
    const int m = blockIdx.x;
    const int t = threadIdx.x;
    const uint16_t* row = x + (size_t)m * K;
    const int chunks = K / 8;  // 16-byte chunks of 8 activations; 16 per group

    float amax = 0.0f;
    for (int c = t; c < chunks; c += 256) {
        const uint4 v = *reinterpret_cast<const uint4*>(row + 8 * c);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[i] & 0xFFFFu)));
            amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[i] >> 16)));
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if ((t & 63) == 0) red[t >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float a = amax / 127.0f;  // correctly rounded division (the library is built for it)
    if (a == 0.0f) a = 1.0f;
    if (t == 0) ascale[m] = a;

    for (int c = t; c < chunks; c += 256) {
        const uint4 v = *reinterpret_cast<const uint4*>(row + 8 * c);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t packed[2] = {0u, 0u};
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t bits = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
            const float r = rintf(bf16_bits_to_f32(bits) / a);
            const int q = r < -127.0f ? -127 : (r > 127.0f ? 127 : (int)r);
            packed[i >> 2] |= ((uint32_t)q & 0xFFu) << (8 * (i & 3));
            sum += q;
        }
        *reinterpret_cast<uint2*>(xq + (size_t)m * K + 8 * c) = make_uint2(packed[0], packed[1]);
        // the 16 chunks of a group are 16 consecutive threads (256 is a multiple of 16)
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
        if ((c & 15) == 0) xsum[(size_t)(c / 16) * M + m] = (float)sum;  // |sum| <= 127 * 128: exact
    }
}

// ---- GEMM ------------------------------------------------------------------------------------

constexpr int kT = 128;                                // block tile (rows and columns), and BK
constexpr int kOffA = 0;                               // 128 rows x 128 bytes
constexpr int kOffB = kOffA + kT * kT;                 // 8 copies of 2 packed rows x 512 bytes,
constexpr int kBCopy = 1152;                           //   1152 bytes apart
constexpr int kOffS = kOffB + 8 * kBCopy;
constexpr int kOffMn = kOffS + kT * 2;                 // 128 bf16 scales, then 128 bf16 minimums
constexpr int kOffX = kOffMn + kT * 2;                 // 128 fp32 row sums
constexpr int kStage = kOffX + kT * 4;                 // 26,624 bytes
constexpr int kStages = 3;
static_assert(kStage % 16 == 0, "stage alignment");

__device__ __forceinline__ uint32_t w8_lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Direct-to-LDS copies from inline assembly, so that the compiler does not track them (it cannot
// tell the LDS stages apart and would wait for every copy in flight before any LDS read): lane l
// reads 16 (or 4) bytes at sbase + voff, and the load unit writes them to LDS byte m0 + 16 l
// (or 4 l).  The only waits for them are the explicit ones before each k-tile's barrier.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void w8_dma16(uint32_t voff, const void* sbase, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void w8_dma4(uint32_t voff, const void* sbase, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

template <int n>
__device__ __forceinline__ void w8_wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | 0x0F70 /* expcnt, lgkmcnt: no wait */);
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void w4a8_gemm_kernel(const int8_t* __restrict__ xq, const float* __restrict__ ascale, const float* __restrict__ xsum,
                      const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                      const uint16_t* __restrict__ mins, uint16_t* __restrict__ y, int M, int N, int K) {
    __shared__ __attribute__((aligned(16))) char smem[kStages * kStage];
    __shared__ float arow[kT];  // the block's row scales
    const int lane = lane_id(), wave = wave_id();
    const int l32 = lane & 31, kg = lane >> 5;
    const int n0 = blockIdx.x * kT, m0 = blockIdx.y * kT;
    const int T = K / kT;
    const uint32_t lds0 = w8_lds_addr(smem);
    const int col = 32 * wave + l32;  // this lane's column in the tile (every row tile)

    // Per-lane source offsets of this wave's copies (the k-tile adds a uniform offset):
    //  A: copies j = 4 wave + i, rows 8 j .. 8 j + 7; lane l -> row 8 j + l / 8, LDS slot l % 8,
    //     which holds chunk (l % 8) ^ ((row >> 1) & 7) of the row's 128 bytes
    uint32_t a_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * (4 * wave + i) + lane / 8;
        const int c = (lane % 8) ^ ((r >> 1) & 7);
        a_off[i] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)K + 16u * c;
    }
    //  B: copies j = 2 wave + i: packed rows 2 j + lane / 32 of the group, columns 4 (lane % 32) ..
    //     + 3 (past N: the last four columns, never stored)
    uint32_t b_off[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int pr = 2 * (2 * wave + i) + lane / 32;
        const int n = min(n0 + 4 * l32, N - 4);
        b_off[i] = ((uint32_t)pr * (uint32_t)N + (uint32_t)n) * 4u;
    }
    //  one 4-byte copy: wave 0 the scales, wave 1 the minimums (two columns per lane), waves 2
    //  and 3 the row sums of rows 64 (wave - 2) + lane
    const void* small_src;
    uint32_t small_off, small_lds;
    if (wave < 2) {
        small_src = wave == 0 ? (const void*)scales : (const void*)mins;
        small_off = (uint32_t)min(n0 + 2 * lane, N - 2) * 2u;
        small_lds = wave == 0 ? kOffS : kOffMn;
    } else {
        small_src = xsum;
        small_off = (uint32_t)min(m0 + 64 * (wave - 2) + lane, M - 1) * 4u;
        small_lds = kOffX + 256 * (wave - 2);
    }
    small_lds = __builtin_amdgcn_readfirstlane(small_lds);

    // the seven copies of k-tile t into stage st
    auto issue = [&](int t, int st) {
        const uint32_t sbase = lds0 + (uint32_t)(st * kStage);
        const int8_t* xa = xq + (size_t)t * kT;
#pragma unroll
        for (int i = 0; i < 4; ++i) w8_dma16(a_off[i], xa, sbase + kOffA + 1024u * (4 * wave + i));
        const uint32_t* cb = codes + (size_t)t * 16 * N;
#pragma unroll
        for (int i = 0; i < 2; ++i) w8_dma16(b_off[i], cb, sbase + kOffB + (uint32_t)(kBCopy * (2 * wave + i)));
        const char* sp = (const char*)small_src + (wave < 2 ? (size_t)t * N * 2 : (size_t)t * M * 4);
        w8_dma4(small_off, sp, sbase + small_lds);
    };

    issue(0, 0);
    if (T > 1) issue(1, 1);
    if (threadIdx.x < kT) arow[threadIdx.x] = ascale[min(m0 + (int)threadIdx.x, M - 1)];

    // Lane offsets inside a stage.  Row 32 rt + l32 of the activation tile keeps its chunk c at
    // slot c ^ ((l32 >> 1) & 7) (the row tile does not change the swizzle), so k-step ks reads at
    // a_lane[ks] + 4096 rt; the packed words of copy 2 ks + kg at b_lane + 2 ks kBCopy.
    uint32_t a_lane[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a_lane[ks] = kOffA + 128u * l32 + 16u * ((2 * ks + kg) ^ ((l32 >> 1) & 7));
    const uint32_t b_lane = kOffB + kBCopy * kg + 4u * col;

    // fp32 accumulators, element e of row tile rt: row 32 rt + 8 (e / 4) + 4 kg + e % 4, column col
    f32x16_t yacc[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int e = 0; e < 16; ++e) yacc[rt][e] = 0.0f;
    // the minimum term sum_g min_g X_g on v_mfma_f32_32x32x2f32, two groups per instruction: A
    // lane l holds X of row l % 32 and group 2 p + l / 32, B lane l the minimum of column l % 32 and
    // the same group; an even group's values wait in xp / mp for the odd one
    float xp[4], mp = 0.0f;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) xp[rt] = 0.0f;

    // Software pipeline over groups: the int32 sums of group t (acc[t & 1]) are computed while the
    // previous group's (acc[(t - 1) & 1]) go through the fp32 epilogue, whose scale, minimum and
    // row sums were read into registers (sv, mv, xc) before their stage could be overwritten.
    i32x16_t acc[2][4];
    float sv = 0.0f, mv = 0.0f, xc[4] = {0.0f, 0.0f, 0.0f, 0.0f};

    auto mfma_group = [&](auto par, const char* s) {
        constexpr int P = decltype(par)::value;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const uint32_t* wp = reinterpret_cast<const uint32_t*>(s + b_lane + 2 * ks * kBCopy);
            const uint32_t w0 = wp[0], w1 = wp[128];
            const uint32_t lo0 = w0 & 0x0F0F0F0Fu, hi0 = (w0 >> 4) & 0x0F0F0F0Fu;
            const uint32_t lo1 = w1 & 0x0F0F0F0Fu, hi1 = (w1 >> 4) & 0x0F0F0F0Fu;
            const i32x4_t b = {(int)__builtin_amdgcn_perm(hi0, lo0, 0x05010400u),
                               (int)__builtin_amdgcn_perm(hi0, lo0, 0x07030602u),
                               (int)__builtin_amdgcn_perm(hi1, lo1, 0x05010400u),
                               (int)__builtin_amdgcn_perm(hi1, lo1, 0x07030602u)};
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const i32x4_t av = *reinterpret_cast<const i32x4_t*>(s + a_lane[ks] + 4096 * rt);
                if (ks == 0)
                    acc[P][rt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, b, i32x16_t{}, 0, 0, 0);
                else
                    acc[P][rt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, b, acc[P][rt], 0, 0, 0);
            }
        }
    };
    // the epilogue of group g (parity P, odd when g is): s * sum, then the minimum term per pair
    auto epilogue = [&](auto par) {
        constexpr int P = decltype(par)::value;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int e = 0; e < 16; ++e) yacc[rt][e] = __builtin_fmaf(sv, (float)acc[P][rt][e], yacc[rt][e]);
        if constexpr (P == 1) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                yacc[rt] = __builtin_amdgcn_mfma_f32_32x32x2f32(kg ? xc[rt] : xp[rt], kg ? mv : mp, yacc[rt], 0, 0, 0);
        } else {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) xp[rt] = xc[rt];
            mp = mv;
        }
    };
    auto read_params = [&](const char* s) {
        sv = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(s + kOffS)[col]);
        mv = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(s + kOffMn)[col]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) xc[rt] = reinterpret_cast<const float*>(s + kOffX)[32 * rt + l32];
    };

    // one k-tile t (stage t % 3 and parity t % 2 known at compile time): wait for its copies,
    // barrier, request t + 2, the MFMAs of t, the epilogue of t - 1, then t's own parameters
    auto ktile = [&](int t, auto st_c, auto par_c) {
        constexpr int ST = decltype(st_c)::value, P = decltype(par_c)::value;
        if (t + 1 < T)
            w8_wait_vm<7>();
        else
            w8_wait_vm<0>();
        __syncthreads();
        if (t + 2 < T) issue(t + 2, (ST + 2) % kStages);
        const char* s = smem + ST * kStage;
        mfma_group(std::integral_constant<int, P>{}, s);
        if (t > 0) epilogue(std::integral_constant<int, 1 - P>{});
        read_params(s);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    for (int t0 = 0; t0 < T; t0 += 6) {
        ktile(t0, I0{}, I0{});
        if (t0 + 1 < T) ktile(t0 + 1, I1{}, I1{});
        if (t0 + 2 < T) ktile(t0 + 2, I2{}, I0{});
        if (t0 + 3 < T) ktile(t0 + 3, I0{}, I1{});
        if (t0 + 4 < T) ktile(t0 + 4, I1{}, I0{});
        if (t0 + 5 < T) ktile(t0 + 5, I2{}, I1{});
    }
    // the last group's epilogue; an unpaired last (even) group pairs with zeros
    if ((T - 1) & 1) {
        epilogue(I1{});
    } else {
        epilogue(I0{});
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
            yacc[rt] = __builtin_amdgcn_mfma_f32_32x32x2f32(kg ? 0.0f : xp[rt], kg ? 0.0f : mp, yacc[rt], 0, 0, 0);
    }

    // y = bf16(a_m * acc) through LDS (the stages are free now) as whole rows: 16-byte stores of
    // consecutive columns; rows past M and columns past N are not stored
    __syncthreads();
    uint16_t* tile = reinterpret_cast<uint16_t*>(smem);  // [128][128 + 8] bf16
    constexpr int kPitch = kT + 8;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int r = 32 * rt + 8 * (e / 4) + 4 * kg + (e % 4);
            tile[r * kPitch + col] = f32_to_bf16_bits(arow[r] * yacc[rt][e]);
        }
    __syncthreads();
    for (int idx = threadIdx.x; idx < kT * (kT / 8); idx += 256) {
        const int r = idx / (kT / 8), c8 = idx % (kT / 8);
        const int row = m0 + r, c0 = n0 + 8 * c8;
        if (row >= M || c0 >= N) continue;
        const uint4 v = *reinterpret_cast<const uint4*>(tile + r * kPitch + 8 * c8);
        uint16_t* dst = y + (size_t)row * N + c0;
        if ((N & 7) == 0) {
            *reinterpret_cast<uint4*>(dst) = v;  // N % 8 == 0: in range and 16-byte aligned
        } else {  // N % 4 == 0: 8-byte aligned halves, the second one only inside the row
            *reinterpret_cast<uint2*>(dst) = make_uint2(v.x, v.y);
            if (c0 + 4 < N) *reinterpret_cast<uint2*>(dst + 4) = make_uint2(v.z, v.w);
        }
    }
}

}  // namespace

hipError_t launch_quant_act_i8(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, float* ascale, float* xsum,
                               hipStream_t stream) {
    hipLaunchKernelGGL(quant_act_i8_kernel, dim3((unsigned)M), dim3(256), 0, stream, x, (int)M, (int)K, xq, ascale,
                       xsum);
    return hipGetLastError();
}

hipError_t launch_gemm_w4a8(const int8_t* xq, const float* ascale, const float* xsum, int64_t M,
                            const uint32_t* codes, const uint16_t* scales, const uint16_t* mins, int64_t N, int64_t K,
                            uint16_t* y, hipStream_t stream) {
    const dim3 grid((unsigned)((N + kT - 1) / kT), (unsigned)((M + kT - 1) / kT));
    hipLaunchKernelGGL(w4a8_gemm_kernel, grid, dim3(256), 0, stream, xq, ascale, xsum, codes, scales, mins, y, (int)M,
                       (int)N, (int)K);
    return hipGetLastError();
}

}  // namespace w4a16
