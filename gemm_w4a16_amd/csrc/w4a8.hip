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
//  * block tile 128 x 256 (8 waves, one block per CU) where that still gives half the CUs a block,
//    else 128 x 128 (4 waves, two blocks per CU); the waves sit side by side along N and each owns
//    128 rows x 32 columns as four v_mfma_i32_32x32x32_i8 accumulators restarted at zero every
//    group, so each packed word is unpacked once per block;
//  * every operand reaches LDS through direct-to-LDS copies issued two k-tiles ahead (three
//    stages): the 128 x 128-byte activation tile (16-byte chunks XOR-swizzled by row pair, so
//    the fragment reads are conflict-free), the 16 packed rows of weights as they are stored (the
//    pairs of packed rows 128 bytes apart, so that the two pairs a k-step reads sit on different
//    banks), the group's scales and minimums, and the 128 row sums X.  One `s_waitcnt vmcnt`
//    before each k-tile's barrier waits for exactly this wave's copies of that k-tile;
//  * a lane's B fragment (32 k x 32 columns: 16 k of one column) is two consecutive packed words:
//    w & 0x0F0F0F0F and (w >> 4) & 0x0F0F0F0F hold the even and odd codes as bytes, and two
//    v_perm_b32 put them back in k order, matching the activation bytes;
//  * after a group's 4 k-steps each int32 sum becomes fp32 (exact: |sum| < 2^18) and enters the
//    fp32 accumulator as s * sum (one convert and one fma per output); the minimum term
//    sum_g min_g X_g is a [128 x G] x [G x 128] product of its own, run on v_mfma_f32_32x32x2f32
//    two groups at a time into the same accumulators, so it costs no VALU work per output;
//  * the row scale multiplies the total once at the end, and the tile leaves through LDS as
//    whole rows (16-byte stores of consecutive columns).
//
// w4a8_rows16_kernel -- the same sum for up to 64 rows, 16 per block, where the weight stream sets
// the time (below).
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "lds_dma.h"

namespace w4a16 {

namespace {

// ---- activation quantization ------------------------------------------------------------------

// One activation (bf16 bits) to its int8 code with row scale a: rint(x / a) (IEEE division, ties to
// even), clamped to [-127, 127].  The quantizer and the fused few-row kernel both use this.
__device__ __forceinline__ int quant_i8(uint32_t bits, float a) {
    const float r = rintf(bf16_bits_to_f32(bits) / a);
    return r < -127.0f ? -127 : (r > 127.0f ? 127 : (int)r);
}

// max |x| over the 8 bf16 of a 16-byte chunk, folded into m
__device__ __forceinline__ float absmax8(uint4 v, float m) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        m = fmaxf(m, fabsf(bf16_bits_to_f32(w[i] & 0xFFFFu)));
        m = fmaxf(m, fabsf(bf16_bits_to_f32(w[i] >> 16)));
    }
    return m;
}

__global__ __launch_bounds__(256) void quant_act_i8_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                           int8_t* __restrict__ xq, float* __restrict__ ascale,
                                                           float* __restrict__ xsum) {
    __shared__ float red[4];
    const int m = blockIdx.x;
    const int t = threadIdx.x;
    const uint16_t* row = x + (size_t)m * K;
    const int chunks = K / 8;  // 16-byte chunks of 8 activations; 16 per group
    // The first kKeep chunks of each thread stay in registers between the two passes (all of a row
    // up to K = 8192), so the quantization does not wait for a second read of the row.  Chunks are
    // taken in whole 16-lane groups (chunks is a multiple of 16, 256 of 16), so every lane of a
    // group is active at the group sum's shuffles.
    constexpr int kKeep = 4;
    uint4 keep[kKeep];

    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kKeep; ++i) {
        const int c = t + 256 * i;
        if (c < chunks) {
            keep[i] = *reinterpret_cast<const uint4*>(row + 8 * c);
            amax = absmax8(keep[i], amax);
        }
    }
    for (int c = t + 256 * kKeep; c < chunks; c += 256) amax = absmax8(*reinterpret_cast<const uint4*>(row + 8 * c), amax);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if ((t & 63) == 0) red[t >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float a = amax / 127.0f;  // correctly rounded division (the library is built for it)
    if (a == 0.0f) a = 1.0f;
    if (t == 0) ascale[m] = a;

    // codes of chunk c (8 activations), and the exact code sum of its group
    auto quantize_chunk = [&](uint4 v, int c) __attribute__((always_inline)) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t packed[2] = {0u, 0u};
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int q = quant_i8((i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu), a);
            packed[i >> 2] |= ((uint32_t)q & 0xFFu) << (8 * (i & 3));
            sum += q;
        }
        *reinterpret_cast<uint2*>(xq + (size_t)m * K + 8 * c) = make_uint2(packed[0], packed[1]);
        // the 16 chunks of a group are 16 consecutive threads
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
        if ((c & 15) == 0) xsum[(size_t)(c / 16) * M + m] = (float)sum;  // |sum| <= 127 * 128: exact
    };
#pragma unroll
    for (int i = 0; i < kKeep; ++i) {
        const int c = t + 256 * i;
        if (c < chunks) quantize_chunk(keep[i], c);
    }
    for (int c = t + 256 * kKeep; c < chunks; c += 256) quantize_chunk(*reinterpret_cast<const uint4*>(row + 8 * c), c);
}

// ---- GEMM ------------------------------------------------------------------------------------

constexpr int kBM = 128;  // block rows, and the k-tile: one group of 128 k
constexpr int kStages = 3;

// LDS stage of a 128 x BN block tile.
template <int BN_>
struct W8Layout {
    static constexpr int BN = BN_;
    static constexpr int OffA = 0;                      // 128 rows x 128 bytes, chunks swizzled
    static constexpr int BCopy = 2 * BN * 4 + 128;      // packed rows 2j, 2j+1 (BN words each), 128 B apart
    static constexpr int OffB = OffA + kBM * kBM;       //   from the next pair: the two pairs a k-step reads
    static constexpr int OffS = OffB + 8 * BCopy;       //   sit on different banks
    static constexpr int OffMn = OffS + BN * 2;         // BN bf16 scales, BN bf16 minimums
    static constexpr int OffX = OffMn + BN * 2;         // 128 fp32 row sums
    static constexpr int Stage = OffX + kBM * 4;
    static constexpr int RowsPerB = 256 / BN;           // packed rows per 1-KB copy
    static constexpr int BCopies = BN / 16;             // 1-KB copies of the 16 packed rows
    static constexpr int NSmall = BN / 64 + 2;          // 256-byte copies: scales, minimums, row sums
    static_assert(Stage % 16 == 0, "stage alignment");
};

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x16_t __attribute__((ext_vector_type(16)));


// NW waves side by side along N, each owning 32 columns: the block is 128 x 32 NW.
template <int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void w4a8_gemm_kernel(const int8_t* __restrict__ xq, const float* __restrict__ ascale, const float* __restrict__ xsum,
                      const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                      const uint16_t* __restrict__ mins, uint16_t* __restrict__ y, int M, int N, int K) {
    constexpr int WCT = 1;  // 32-column MFMA tiles per wave
    using L = W8Layout<32 * WCT * NW>;
    constexpr int BN = L::BN;
    constexpr int kACopies = 16 / NW, kBCopies = L::BCopies / NW;  // 1-KB copies per wave per k-tile
    static_assert(kACopies * NW == 16 && kBCopies * NW == L::BCopies, "copies split evenly over the waves");
    __shared__ __attribute__((aligned(16))) char smem[kStages * L::Stage];
    __shared__ float arow[kBM];  // the block's row scales
    const int lane = lane_id(), wave = wave_id();
    const int l32 = lane & 31, kg = lane >> 5;
    const int n0 = blockIdx.x * BN, m0 = blockIdx.y * kBM;
    const int T = K / kBM;
    const uint32_t lds0 = lds_addr(smem);

    // ---- this wave's copies of a k-tile (per-lane source offsets; the k-tile adds a uniform one)
    //  A: copies j = kACopies wave + i, rows 8 j .. 8 j + 7; lane l -> row 8 j + l / 8, LDS slot
    //     l % 8, which holds chunk (l % 8) ^ ((row >> 1) & 7) of the row's 128 bytes
    uint32_t a_off[kACopies];
#pragma unroll
    for (int i = 0; i < kACopies; ++i) {
        const int r = 8 * (kACopies * wave + i) + lane / 8;
        const int c = (lane % 8) ^ ((r >> 1) & 7);
        a_off[i] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)K + 16u * c;
    }
    //  B: copies j = kBCopies wave + i of 1 KB: packed rows RowsPerB j + lane / (64 / RowsPerB),
    //     4 columns per lane (past N: the last four columns, never stored)
    constexpr int kLanesPerRow = 64 / L::RowsPerB;
    uint32_t b_off[kBCopies], b_lds[kBCopies];
#pragma unroll
    for (int i = 0; i < kBCopies; ++i) {
        const int j = kBCopies * wave + i;
        const int pr0 = L::RowsPerB * j;
        const int pr = pr0 + lane / kLanesPerRow;
        const int n = min(n0 + 4 * (lane % kLanesPerRow), N - 4);
        b_off[i] = ((uint32_t)pr * (uint32_t)N + (uint32_t)n) * 4u;
        b_lds[i] = __builtin_amdgcn_readfirstlane(L::OffB + L::BCopy * (pr0 / 2) + (pr0 % 2) * BN * 4);
    }
    //  small 256-byte copies i = wave, wave + NW (of NSmall): the scales (BN / 128 of them, two
    //  columns per lane), the minimums, then the row sums of rows 64 (i - BN / 64) + lane
    constexpr int kSC = BN / 128;  // 256-byte copies of the scales (and of the minimums)
    constexpr int kSmallMax = (L::NSmall + NW - 1) / NW;
    const void* sm_src[kSmallMax];
    uint32_t sm_off[kSmallMax], sm_lds[kSmallMax];
    size_t sm_step[kSmallMax];
    const int n_small = (L::NSmall - wave + NW - 1) / NW;
#pragma unroll
    for (int u = 0; u < kSmallMax; ++u) {
        const int i = wave + NW * u;
        if (i < kSC) {
            sm_src[u] = scales, sm_step[u] = (size_t)N * 2, sm_lds[u] = L::OffS + 256 * i;
            sm_off[u] = (uint32_t)min(n0 + 128 * i + 2 * lane, N - 2) * 2u;
        } else if (i < 2 * kSC) {
            sm_src[u] = mins, sm_step[u] = (size_t)N * 2, sm_lds[u] = L::OffMn + 256 * (i - kSC);
            sm_off[u] = (uint32_t)min(n0 + 128 * (i - kSC) + 2 * lane, N - 2) * 2u;
        } else {
            sm_src[u] = xsum, sm_step[u] = (size_t)M * 4, sm_lds[u] = L::OffX + 256 * (i - 2 * kSC);
            sm_off[u] = (uint32_t)min(m0 + 64 * (i - 2 * kSC) + lane, M - 1) * 4u;
        }
        sm_lds[u] = __builtin_amdgcn_readfirstlane(sm_lds[u]);
    }

    auto issue = [&](int t, int st) __attribute__((always_inline)) {
        const uint32_t sbase = lds0 + (uint32_t)(st * L::Stage);
        const int8_t* xa = xq + (size_t)t * kBM;
#pragma unroll
        for (int i = 0; i < kACopies; ++i) dma16(a_off[i], xa, sbase + L::OffA + 1024u * (kACopies * wave + i));
        const uint32_t* cb = codes + (size_t)t * 16 * N;
#pragma unroll
        for (int i = 0; i < kBCopies; ++i) dma16(b_off[i], cb, sbase + b_lds[i]);
#pragma unroll
        for (int u = 0; u < kSmallMax; ++u)
            if (u < n_small) dma4(sm_off[u], (const char*)sm_src[u] + (size_t)t * sm_step[u], sbase + sm_lds[u]);
    };
    // copies per wave per k-tile: kACopies + kBCopies + n_small (n_small is 0, 1 or 2, wave-uniform)
    constexpr int kBase = kACopies + kBCopies;
    auto wait_next_only = [&]() __attribute__((always_inline)) {  // at most this wave's copies of one k-tile in flight
        if (n_small == 2)
            wait_vm<kBase + 2>();
        else if (n_small == 1)
            wait_vm<kBase + 1>();
        else
            wait_vm<kBase>();
    };

    issue(0, 0);
    if (T > 1) issue(1, 1);
    if (threadIdx.x < kBM) arow[threadIdx.x] = ascale[min(m0 + (int)threadIdx.x, M - 1)];

    // Lane offsets inside a stage.  Row 32 rt + l32 of the activation tile keeps its chunk c at
    // slot c ^ ((l32 >> 1) & 7) (the row tile does not change the swizzle), so k-step ks reads at
    // a_lane[ks] + 4096 rt; column tile ct's packed words of k-step ks at b_lane + 2 ks BCopy + 128 ct.
    uint32_t a_lane[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a_lane[ks] = L::OffA + 128u * l32 + 16u * ((2 * ks + kg) ^ ((l32 >> 1) & 7));
    const int colw = 32 * WCT * wave + l32;  // this lane's column in column tile 0 (tile ct: + 32 ct)
    const uint32_t b_lane = L::OffB + L::BCopy * kg + 4u * colw;

    // fp32 accumulators, element e of tile (ct, rt): row 32 rt + 8 (e / 4) + 4 kg + e % 4, column colw + 32 ct
    f32x16_t yacc[WCT][4];
#pragma unroll
    for (int ct = 0; ct < WCT; ++ct)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int e = 0; e < 16; ++e) yacc[ct][rt][e] = 0.0f;
    // the minimum term sum_g min_g X_g on v_mfma_f32_32x32x2f32, two groups per instruction: A
    // lane l holds X of row l % 32 and group 2 p + l / 32, B lane l the minimum of column l % 32 and
    // the same group; an even group's values wait in xp / mp for the odd one
    float xp[4], mp[WCT];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) xp[rt] = 0.0f;
#pragma unroll
    for (int ct = 0; ct < WCT; ++ct) mp[ct] = 0.0f;

    // Software pipeline over groups: the int32 sums of group t (acc[t & 1]) are computed while the
    // previous group's (acc[(t - 1) & 1]) go through the fp32 epilogue, whose scale, minimum and
    // row sums were read into registers (sv, mv, xc) before their stage could be overwritten.
    i32x16_t acc[2][WCT][4];
    float sv[WCT], mv[WCT], xc[4];
#pragma unroll
    for (int ct = 0; ct < WCT; ++ct) sv[ct] = mv[ct] = 0.0f;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) xc[rt] = 0.0f;

    auto mfma_group = [&](auto slot, const char* s) __attribute__((always_inline)) {
        constexpr int P = decltype(slot)::value;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            i32x4_t b[WCT];
#pragma unroll
            for (int ct = 0; ct < WCT; ++ct) {
                const uint32_t* wp = reinterpret_cast<const uint32_t*>(s + b_lane + 2 * ks * L::BCopy + 128 * ct);
                const uint32_t w0 = wp[0], w1 = wp[BN];
                const uint32_t lo0 = w0 & 0x0F0F0F0Fu, hi0 = (w0 >> 4) & 0x0F0F0F0Fu;
                const uint32_t lo1 = w1 & 0x0F0F0F0Fu, hi1 = (w1 >> 4) & 0x0F0F0F0Fu;
                b[ct] = i32x4_t{(int)__builtin_amdgcn_perm(hi0, lo0, 0x05010400u),
                                (int)__builtin_amdgcn_perm(hi0, lo0, 0x07030602u),
                                (int)__builtin_amdgcn_perm(hi1, lo1, 0x05010400u),
                                (int)__builtin_amdgcn_perm(hi1, lo1, 0x07030602u)};
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const i32x4_t av = *reinterpret_cast<const i32x4_t*>(s + a_lane[ks] + 4096 * rt);
#pragma unroll
                for (int ct = 0; ct < WCT; ++ct) {
                    if (ks == 0)
                        acc[P][ct][rt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, b[ct], i32x16_t{}, 0, 0, 0);
                    else
                        acc[P][ct][rt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, b[ct], acc[P][ct][rt], 0, 0, 0);
                }
            }
        }
    };
    // the epilogue of a group of parity P whose sums are in acc[A]: s * sum (each int32 sum exact
    // in fp32: |sum| < 2^18), then the minimum term once per pair of groups
    auto epilogue = [&](auto slot, auto par) __attribute__((always_inline)) {
        constexpr int A = decltype(slot)::value, P = decltype(par)::value;
#pragma unroll
        for (int ct = 0; ct < WCT; ++ct)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    yacc[ct][rt][e] = __builtin_fmaf(sv[ct], (float)acc[A][ct][rt][e], yacc[ct][rt][e]);
        if constexpr (P == 1) {
#pragma unroll
            for (int ct = 0; ct < WCT; ++ct)
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
                    yacc[ct][rt] = __builtin_amdgcn_mfma_f32_32x32x2f32(kg ? xc[rt] : xp[rt], kg ? mv[ct] : mp[ct],
                                                                        yacc[ct][rt], 0, 0, 0);
        } else {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) xp[rt] = xc[rt];
#pragma unroll
            for (int ct = 0; ct < WCT; ++ct) mp[ct] = mv[ct];
        }
    };
    auto read_params = [&](const char* s) __attribute__((always_inline)) {
#pragma unroll
        for (int ct = 0; ct < WCT; ++ct) {
            sv[ct] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(s + L::OffS)[colw + 32 * ct]);
            mv[ct] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(s + L::OffMn)[colw + 32 * ct]);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) xc[rt] = reinterpret_cast<const float*>(s + L::OffX)[32 * rt + l32];
    };

    // one k-tile t (stage t % 3 and parity t % 2 known at compile time): wait for its copies,
    // barrier, request t + 2, the MFMAs of t, the epilogue of t - 1, then t's own parameters
    auto ktile = [&](int t, auto st_c, auto par_c) __attribute__((always_inline)) {
        constexpr int ST = decltype(st_c)::value, P = decltype(par_c)::value;
        if (t + 1 < T)
            wait_next_only();
        else
            wait_vm<0>();
        __syncthreads();
        if (t + 2 < T) issue(t + 2, (ST + 2) % kStages);
        const char* s = smem + ST * L::Stage;
        mfma_group(std::integral_constant<int, P>{}, s);
        if (t > 0) epilogue(std::integral_constant<int, 1 - P>{}, std::integral_constant<int, 1 - P>{});
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
        epilogue(I1{}, I1{});
    } else {
        epilogue(I0{}, I0{});
#pragma unroll
        for (int ct = 0; ct < WCT; ++ct)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                yacc[ct][rt] = __builtin_amdgcn_mfma_f32_32x32x2f32(kg ? 0.0f : xp[rt], kg ? 0.0f : mp[ct],
                                                                    yacc[ct][rt], 0, 0, 0);
    }

    // y = bf16(a_m * acc) through LDS (the stages are free now) as whole rows: 16-byte stores of
    // consecutive columns; rows past M and columns past N are not stored
    __syncthreads();
    constexpr int kPitch = BN + 8;
    static_assert(kBM * kPitch * 2 <= kStages * L::Stage, "the output tile fits in the stages");
    uint16_t* tile = reinterpret_cast<uint16_t*>(smem);  // [128][BN + 8] bf16
#pragma unroll
    for (int ct = 0; ct < WCT; ++ct)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = 32 * rt + 8 * (e / 4) + 4 * kg + (e % 4);
                tile[r * kPitch + colw + 32 * ct] = f32_to_bf16_bits(arow[r] * yacc[ct][rt][e]);
            }
    __syncthreads();
    for (int idx = threadIdx.x; idx < kBM * (BN / 8); idx += 64 * NW) {
        const int r = idx / (BN / 8), c8 = idx % (BN / 8);
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

// ---- 1..64 rows: the weights streamed straight into registers -----------------------------------
//
// w4a8_rows16_kernel -- the same sum, y = a_m * sum_g (s_g,n * sum_k xq q + min_g,n * X_g,m), for a
// few rows, where the work is the weight stream (HBM-bound) rather than the products.  A block of 16
// waves owns 64 columns, up to 16 rows (blockIdx.y) and all of K, the groups dealt over the waves
// (two per wave per 4096 k);
// every load of a pass (16 bytes of 4 adjacent columns of one packed row per lane, the rows' 16-byte
// activation chunks, the group's scales, minimums and row sums) is issued before any math, in the
// order it is used.  Per group, a lane's v_mfma_i32_16x16x64_i8 B fragment is 16 k of one column,
// two packed words unpacked to bytes in k order as in the GEMM, and its A fragment the same 16 k of
// one row (for a single row staged per wave in LDS: the fragments of all 16 lanes of a lane group
// are the same bytes, and loading them from memory would request them 16 times); the group
// epilogue is one convert and two fma per output.  The waves' sums are added
// through LDS in wave order, so the result is reproducible run to run.
constexpr int kR16Waves = 16;
constexpr int kW4A8Rows16Max = 64;  // rows up to which w4a8_rows16_kernel (16 rows per block) is used
constexpr int kR16Gpp = 2;  // groups per wave per pass: a pass covers 32 groups (4096 k)

// An LDS-only workgroup barrier: this wave's LDS writes complete, then s_barrier.  No memory fence,
// so the weight loads in flight stay in flight; the memory clobber keeps the compiler from moving
// LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// MR: rows the accumulator layout keeps (M <= MR; 1, 4 or 16).  N % 4 == 0.
// kFused (one row): the block quantizes the bf16 row x itself, with the quantizer's arithmetic:
// with its first pass's weight loads in flight (requested after one 16-byte chunk of x per thread),
// the block reduces max|x| (every block reads the whole row, 8 KB at K = 4096, from L2), and each
// wave then quantizes its own groups into LDS and sums their codes.  Otherwise xq, ascale and xsum
// come from w4a16_quantize_act_i8.
template <int MR, bool kFused>
__global__ __launch_bounds__(64 * kR16Waves) void w4a8_rows16_kernel(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ xq, const float* __restrict__ ascale,
    const float* __restrict__ xsum, const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ mins, uint16_t* __restrict__ y, int M, int N, int K) {
    static_assert(!kFused || MR == 1, "the fused form quantizes one row");
    constexpr int E = MR == 1 ? 1 : 4;  // D rows per lane that can be real (row 4 (lane / 16) + e)
    constexpr int TPL = 4, COLS = 64;
    constexpr bool kStageX = MR == 1 || kFused;  // activation fragments from LDS
    __shared__ float part[kR16Waves][MR][COLS];
    // each wave's groups' 128-byte activation runs, per row: for one row loaded with one 4-byte
    // load per lane (the A fragments then cost no vector-memory requests of their own), in the
    // fused form written by the quantization
    __shared__ __attribute__((aligned(16))) uint32_t xw[kStageX ? kR16Waves : 1][kStageX ? MR : 1][kR16Gpp * 32];
    __shared__ float red[kFused ? kR16Waves : 1][MR];
    float arow[MR];  // fused: the row scales a_m
#pragma unroll
    for (int m = 0; m < MR; ++m) arow[m] = 1.0f;
    const int lane = lane_id(), wave = wave_id();
    const int lr = lane & 15, lg = lane >> 4;
    const int n0 = blockIdx.x * COLS;
    const int m0 = blockIdx.y * MR;       // this block's rows m0 .. m0 + Mb - 1
    const int Mb = min(M - m0, MR);
    const int G = K >> 7;
    // this lane's 4 adjacent columns; a lane past N re-reads the last 4 and never stores
    const int cbase = min(n0 + TPL * lr, N - TPL);
    // A row of this lane (rows past the block's last repeat it: their outputs are never stored)
    // and the D rows it holds
    const int8_t* xrow = kStageX ? nullptr : xq + (size_t)(m0 + min(lr, Mb - 1)) * K + 16 * lg;
    int drow[E];
#pragma unroll
    for (int e = 0; e < E; ++e) drow[e] = m0 + min(4 * lg + e, Mb - 1);
    // lane byte offset inside a pair of packed rows: rows 2 lg, 2 lg + 1 of the k-step's eight
    const uint32_t lane_off = ((uint32_t)(2 * lg) * (uint32_t)N + (uint32_t)cbase) * 4u;

    float yacc[TPL][E];
#pragma unroll
    for (int t = 0; t < TPL; ++t)
#pragma unroll
        for (int e = 0; e < E; ++e) yacc[t][e] = 0.0f;

    for (int p0 = 0; p0 < G; p0 += kR16Waves * kR16Gpp) {
        int gj[kR16Gpp];
        float live[kR16Gpp];
#pragma unroll
        for (int j = 0; j < kR16Gpp; ++j) {
            const int g = p0 + wave + kR16Waves * j;
            live[j] = g < G ? 1.0f : 0.0f;  // a clamped duplicate group contributes nothing
            gj[j] = min(g, G - 1);
        }
        // all loads of the pass, in the order they are used
        i32x4_t xa[kR16Gpp][2];
        uint2 sf[kR16Gpp], mf[kR16Gpp];
        float xs[kR16Gpp][E];
        u32x4_t w[kR16Gpp][2][2];  // [group][k-step][packed row of the pair], 4 columns each
        // fused: this lane's activations of the pass and, in the first pass, each thread's first
        // 16-byte chunk of the row, requested ahead of the weights so that the max |x| and the
        // quantization below wait for these loads only (a clamped duplicate chunk does not change
        // a maximum)
        uint4 xm[kFused ? MR : 1];
        uint2 xv = make_uint2(0u, 0u);  // fused: this lane's 4 activations of its group (lane / 32)
        if constexpr (kFused) {
            xv = *reinterpret_cast<const uint2*>(x + gj[lane >> 5] * 128 + 4 * (lane & 31));
            if (p0 == 0) {
                const int c0 = min((int)threadIdx.x, (K >> 3) - 1);
#pragma unroll
                for (int m = 0; m < MR; ++m) xm[m] = *reinterpret_cast<const uint4*>(x + (size_t)min(m, M - 1) * K + 8 * c0);
            }
        }
        uint32_t x1 = 0;
        if constexpr (MR == 1 && !kFused) {
            static_assert(kR16Gpp * 32 == 64, "one dword of activations per lane");
            x1 = *reinterpret_cast<const uint32_t*>(xq + gj[lane >> 5] * 128 + 4 * (lane & 31));
        }
#pragma unroll
        for (int j = 0; j < kR16Gpp; ++j) {
            if constexpr (!kStageX) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    xa[j][ks] = *reinterpret_cast<const i32x4_t*>(xrow + gj[j] * 128 + 64 * ks);
            }
            sf[j] = *reinterpret_cast<const uint2*>(scales + (size_t)gj[j] * N + cbase);
            mf[j] = *reinterpret_cast<const uint2*>(mins + (size_t)gj[j] * N + cbase);
            if constexpr (!kFused) {
#pragma unroll
                for (int e = 0; e < E; ++e) xs[j][e] = xsum[(size_t)gj[j] * M + drow[e]];
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const char* row = reinterpret_cast<const char*>(codes + (size_t)(16 * gj[j] + 8 * ks + h) * N);
                    w[j][ks][h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(row + lane_off));
                }
        }
        // keep every load of the pass ahead of the math (the scheduler would otherwise sink half of
        // them between the MFMAs, leaving fewer bytes in flight)
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kFused) {
            if (p0 == 0) {  // the rows' max |x|, with this pass's weight loads in flight
                float amx[MR];
#pragma unroll
                for (int m = 0; m < MR; ++m) amx[m] = absmax8(xm[m], 0.0f);
                for (int c = threadIdx.x + 64 * kR16Waves; c < (K >> 3); c += 64 * kR16Waves)
#pragma unroll
                    for (int m = 0; m < MR; ++m)
                        amx[m] = absmax8(*reinterpret_cast<const uint4*>(x + (size_t)min(m, M - 1) * K + 8 * c), amx[m]);
#pragma unroll
                for (int m = 0; m < MR; ++m) {
#pragma unroll
                    for (int off = 32; off >= 1; off >>= 1) amx[m] = fmaxf(amx[m], __shfl_xor(amx[m], off));
                }
                if (lane == 0) {
#pragma unroll
                    for (int m = 0; m < MR; ++m) red[wave][m] = amx[m];
                }
                lds_barrier();
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    float mx = 0.0f;
#pragma unroll
                    for (int v = 0; v < kR16Waves; ++v) mx = fmaxf(mx, red[v][m]);
                    const float a = mx / 127.0f;  // correctly rounded division, as in the quantizer
                    arow[m] = a == 0.0f ? 1.0f : a;
                }
            }
            // this wave's groups: codes into LDS, and X_g of each row
            {  // lane: group lane / 32, 4 activations
                const uint2 v = xv;
                const int q0 = quant_i8(v.x & 0xFFFFu, arow[0]), q1 = quant_i8(v.x >> 16, arow[0]);
                const int q2 = quant_i8(v.y & 0xFFFFu, arow[0]), q3 = quant_i8(v.y >> 16, arow[0]);
                xw[wave][0][lane] = ((uint32_t)q0 & 0xFFu) | (((uint32_t)q1 & 0xFFu) << 8) |
                                    (((uint32_t)q2 & 0xFFu) << 16) | ((uint32_t)q3 << 24);
                int sum = q0 + q1 + q2 + q3;
#pragma unroll
                for (int off = 16; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
                xs[0][0] = (float)__shfl(sum, 0);  // |X| <= 127 * 128: exact
                xs[1][0] = (float)__shfl(sum, 32);
            }
        } else if constexpr (MR == 1) {
            xw[wave][0][lane] = x1;  // read back by this wave only, after its own write
        }
        if constexpr (kStageX) {
            wave_lds_sync();  // the codes just written by this wave's lanes are read across lanes
            const int ar = min(lr, MR - 1);  // A rows past the staged ones repeat one: never stored
#pragma unroll
            for (int j = 0; j < kR16Gpp; ++j)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    xa[j][ks] = *reinterpret_cast<const i32x4_t*>(&xw[wave][ar][32 * j + 16 * ks + 4 * lg]);
        }
#pragma unroll
        for (int j = 0; j < kR16Gpp; ++j) {
            i32x4_t acc[TPL];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int t = 0; t < TPL; ++t) {
                    const uint32_t w0 = w[j][ks][0][t], w1 = w[j][ks][1][t];
                    const uint32_t lo0 = w0 & 0x0F0F0F0Fu, hi0 = (w0 >> 4) & 0x0F0F0F0Fu;
                    const uint32_t lo1 = w1 & 0x0F0F0F0Fu, hi1 = (w1 >> 4) & 0x0F0F0F0Fu;
                    const i32x4_t b = {(int)__builtin_amdgcn_perm(hi0, lo0, 0x05010400u),
                                       (int)__builtin_amdgcn_perm(hi0, lo0, 0x07030602u),
                                       (int)__builtin_amdgcn_perm(hi1, lo1, 0x05010400u),
                                       (int)__builtin_amdgcn_perm(hi1, lo1, 0x07030602u)};
                    acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa[j][ks], b, ks == 0 ? i32x4_t{} : acc[t], 0, 0, 0);
                }
            const uint32_t sv[TPL] = {sf[j].x & 0xFFFFu, sf[j].x >> 16, sf[j].y & 0xFFFFu, sf[j].y >> 16};
            const uint32_t mv[TPL] = {mf[j].x & 0xFFFFu, mf[j].x >> 16, mf[j].y & 0xFFFFu, mf[j].y >> 16};
#pragma unroll
            for (int t = 0; t < TPL; ++t) {
                const float sc = bf16_bits_to_f32(sv[t]) * live[j], mn = bf16_bits_to_f32(mv[t]) * live[j];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    yacc[t][e] = __builtin_fmaf(sc, (float)acc[t][e], yacc[t][e]);  // |sum| < 2^18: exact in fp32
                    yacc[t][e] = __builtin_fmaf(mn, xs[j][e], yacc[t][e]);
                }
            }
        }
        if constexpr (kStageX) wave_lds_sync();  // this pass's reads precede the next pass's writes
    }

    // the waves' sums through LDS, added in wave order; y = bf16(a_m * sum)
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int row = 4 * lg + e;
        if (row < Mb) {
#pragma unroll
            for (int t = 0; t < TPL; ++t) part[wave][row][TPL * lr + t] = yacc[t][e];
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < Mb * COLS; idx += 64 * kR16Waves) {
        const int row = idx / COLS, c = idx % COLS, n = n0 + c;
        if (n < N) {
            float sum = 0.0f;
#pragma unroll
            for (int v = 0; v < kR16Waves; ++v) sum += part[v][row][c];
            float a = 0.0f;
            if constexpr (kFused) {
                a = arow[0];
#pragma unroll
                for (int m = 1; m < MR; ++m) a = row == m ? arow[m] : a;
            } else {
                a = ascale[m0 + row];
            }
            y[(size_t)(m0 + row) * N + n] = f32_to_bf16_bits(a * sum);
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
    // up to 64 rows, blocks of 16 rows that stream the weights again for each 16 rows (from the
    // Infinity Cache after the first): at K = 4096, N = 14336 that is 15-16 us at 17-32 rows and
    // 30 us at 64, against 35 us for the 128-row tiles, which win from ~96 rows on
    if (M <= kW4A8Rows16Max) {
        const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 15) / 16)), block(64 * kR16Waves);
        const uint16_t* nox = nullptr;
        if (M == 1)
            hipLaunchKernelGGL((w4a8_rows16_kernel<1, false>), grid, block, 0, stream, nox, xq, ascale, xsum, codes,
                               scales, mins, y, (int)M, (int)N, (int)K);
        else if (M <= 4)
            hipLaunchKernelGGL((w4a8_rows16_kernel<4, false>), grid, block, 0, stream, nox, xq, ascale, xsum, codes,
                               scales, mins, y, (int)M, (int)N, (int)K);
        else
            hipLaunchKernelGGL((w4a8_rows16_kernel<16, false>), grid, block, 0, stream, nox, xq, ascale, xsum, codes,
                               scales, mins, y, (int)M, (int)N, (int)K);
        return hipGetLastError();
    }
    const int64_t mt = (M + kBM - 1) / kBM;
    // 128 x 256 tiles (8 waves, one block per CU) when they still give half the CUs a block
    if ((N + 255) / 256 * mt >= 128) {
        const dim3 grid((unsigned)((N + 255) / 256), (unsigned)mt);
        hipLaunchKernelGGL((w4a8_gemm_kernel<8>), grid, dim3(512), 0, stream, xq, ascale, xsum, codes, scales, mins,
                           y, (int)M, (int)N, (int)K);
    } else {
        const dim3 grid((unsigned)((N + 127) / 128), (unsigned)mt);
        hipLaunchKernelGGL((w4a8_gemm_kernel<4>), grid, dim3(256), 0, stream, xq, ascale, xsum, codes, scales, mins,
                           y, (int)M, (int)N, (int)K);
    }
    return hipGetLastError();
}

hipError_t launch_matmul_w4a8_fused(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                                    const uint16_t* mins, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
    if (M != 1) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((N + 63) / 64)), block(64 * kR16Waves);
    const int8_t* noq = nullptr;
    const float* nof = nullptr;
    hipLaunchKernelGGL((w4a8_rows16_kernel<1, true>), grid, block, 0, stream, x, noq, nof, nof, codes, scales, mins, y,
                       (int)M, (int)N, (int)K);
    return hipGetLastError();
}

}  // namespace w4a16
