// mid.hip -- mid-M W4A16 paths (17 <= M <= 64) for the [K/8][N] G128 format, on bf16 MFMA.
//
// The large-M kernel amortizes one dequant of a weight over 256 rows and needs 256 output
// tiles of 256 x 224 to fill the chip; at a few dozen rows it has neither, and the skinny
// kernel's trick (all of K's activations resident in LDS) stops fitting past 16 rows.  The
// kernels here stream the weights once, like a GEMV, with one block per 64 columns.
//
// 17..32 rows (mid_rows32_kernel): the factored form of vidyal.ai "Low-Precision Kernels" ("How
// the measurements were taken": per group s * sum(x*q) + min * sum(x)), as in the skinny kernel,
// with no LDS for the operands:
//  * 8 waves; wave w owns the groups g = w (mod 8) and all 32 rows and 64 columns of the block;
//  * per group a lane loads 16 packed words (4 k-steps x 4 adjacent columns, 16-byte loads),
//    its bf16 scale/minimum pairs, and its own A fragments straight from global memory (2 row
//    tiles x 4 k-steps, 16 bytes each; x is small and stays in L2), two groups ahead;
//  * each word is one lane's B fragment of v_mfma_f32_16x16x32_bf16 after one v_and_or_b32 per
//    bf16 pair (128 + q_j, 128 + q_{j+4}); the A fragment is put in the same k order by four
//    v_perm_b32; a fifth MFMA against ones gives sum(x), and the group epilogue is
//    s * acc + (min - 128 s) * sum(x);
//  * the 8 waves' sums are added through LDS in wave order (bitwise reproducible).
// Most of its time is the loads: each block reads all 256 KB of a 32-row x from L2 besides its
// 128 KB of weights, and a CU's loads complete at ~30 GB/s.
//
// 17..32 and 33..64 rows where N % 4 == 0 and K is a multiple of 512 or 256 (midr_kernel<R> with
// R = 32 or 64 rows per block): the same factored form on v_mfma_f32_32x32x16, with every operand
// brought in by direct-to-LDS copies:
//  * 8 waves in sets (R = 64: two sets of 4, R = 32: four sets of 2); set s runs the groups
//    g = s (mod sets), and within a set a wave owns a 32 x 32 output tile of the block's R x 64,
//    over all of K, so a lane's word is its own B fragment and no wave unpacks a word twice;
//  * a stage holds one group per set: x (R rows x 128 k per group, rows XOR-swizzled in 16-byte
//    chunks so the fragment reads are conflict-free, each copy 1 KB of x), the groups' packed rows
//    and parameters; three stages, the copies two stages ahead, one barrier per stage;
//  * each wave reads its group's 8 A fragments and 8 words at once, then 8 k-steps of two MFMAs
//    (the second against ones gives sum(x)) and the group epilogue s * acc + (min - 128 s) * sum(x);
//  * the sets' sums are added through LDS in set order (bitwise reproducible).
// The same kernel reads the zero-point format's prepared copy (fp16 operands, fp32 parameters).
//
// 17..32 rows otherwise: mid_rows32_kernel above.  33..64 rows otherwise (mid_g128_kernel): dequantizes as vidyal.ai Step 2 builds its B tile (w_hat =
// bf16_rne(fmaf(q, s, min)), the reference value) straight into MFMA B fragments:
//  * block = 64 columns x MR rows x all of K; 2*KP waves: wave (h, p) owns the 32 columns of
//    half h and the groups g = p (mod KP).  With N = 14336 that is 224 blocks per row slice;
//  * per step the block's threads stage MR rows x KP groups of activations in LDS (two
//    stages, 16-byte chunks XOR-swizzled by row so the fragment reads are conflict-free) and
//    each wave runs its group: lane l holds the packed word of column l % 32, k-half l / 32 of a
//    16-k step -- exactly its B fragment of v_mfma_f32_32x32x16_bf16 -- dequantized by 22 VALU
//    instructions and used for all MR / 32 row blocks;
//  * the packed words, scales and minimums of the next step are loaded while this step runs; a
//    wave whose group lies past K skips the step;
//  * the KP partial sums of each output are added through LDS in a fixed order.
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "lds_dma.h"

namespace w4a16 {

namespace {

constexpr int kMidCols = 64;

// f(std::integral_constant<int, i>) for i = I .. N-1, so that i can select template arguments.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// ---- 17..32 rows ------------------------------------------------------------------------------

constexpr int kR32Waves = 8;
constexpr int kR32Ahead = 2;  // groups in flight per wave (the register budget of 2 waves/SIMD)

// (w >> 4j) & 0x000F000F | 0x43004300 = bf16 pair (128 + q_j, 128 + q_{j+4}), j = 0..3
__device__ __forceinline__ bf16x8_t r32_unpack(uint32_t w, uint32_t mask, uint32_t magic) {
    const u32x4_t p = {(w & mask) | magic, ((w >> 4) & mask) | magic, ((w >> 8) & mask) | magic,
                       ((w >> 12) & mask) | magic};
    return __builtin_bit_cast(bf16x8_t, p);
}

// A fragment (x0..x7) as dwords (x0,x1) (x2,x3) (x4,x5) (x6,x7) -> (x0,x4) (x1,x5) (x2,x6) (x3,x7)
__device__ __forceinline__ bf16x8_t r32_pair_up(uint4 v) {
    const uint4 p = make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u), __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                               __builtin_amdgcn_perm(v.w, v.y, 0x05040100u), __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
    return __builtin_bit_cast(bf16x8_t, p);
}

// One group's operands in a lane: packed words [k-step][column], scale/minimum pairs (bf16 pairs,
// or fp32 for the zero-point format's prepared copy), and the A fragments [k-step][row tile] in
// natural k order.
template <bool kP32>
struct R32Group {
    uint32_t w[4][4];
    uint32_t s[2], m[2];
    uint4 a[4][2];
};
template <>
struct R32Group<true> {
    uint32_t w[4][4];
    float s[4], m[4];
    uint4 a[4][2];
};

// kF16: fp16 activations and output on the fp16 matrix cores, codes as 1024 + q (the prepared
// zero-point copy), else bf16 and 128 + q.  kP32: fp32 scales and minimums [K/128][N].
template <bool kVec, bool kF16 = false, bool kP32 = false>
__global__ __launch_bounds__(64 * kR32Waves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mid_rows32_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ codes,
                       const void* __restrict__ scales_v, const void* __restrict__ mins_v,
                       uint16_t* __restrict__ y, int M, int N, int K, uint32_t mask, uint32_t magic) {
    const uint16_t* __restrict__ scales = static_cast<const uint16_t*>(scales_v);
    const uint16_t* __restrict__ mins = static_cast<const uint16_t*>(mins_v);
    const float* __restrict__ scales32 = static_cast<const float*>(scales_v);
    const float* __restrict__ mins32 = static_cast<const float*>(mins_v);
    using Group = R32Group<kP32>;
    constexpr float kOffset = kF16 ? 1024.0f : 128.0f;  // the magic number's value at q = 0
    auto mfma = [](bf16x8_t a, bf16x8_t b, f32x4_t c) {
        if constexpr (kF16) {
            typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
            return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                          0, 0, 0);
        } else {
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
        }
    };
    __shared__ float part[kR32Waves][32][64];
    const int lane = lane_id(), wave = wave_id();
    const int lr = lane & 15, lg = lane >> 4;
    const int G = K >> 7;
    const int J = G > wave ? (G - wave + kR32Waves - 1) / kR32Waves : 0;  // this wave's groups
    const int n0 = blockIdx.x * kMidCols;
    // this lane's 4 adjacent columns; past N they re-read in-range columns and are never stored
    int cbase = n0 + 4 * lr;
    if (kVec) cbase = min(cbase, N - 4);
    const uint32_t lane_off = ((uint32_t)lg * (uint32_t)N + (uint32_t)cbase) * 4u;
    // this lane's A rows lr and 16 + lr (clamped: rows past M feed only outputs never stored),
    // k chunk lg of each 32-k step
    const uint16_t* xrow0 = x + (size_t)min(lr, M - 1) * K + 8 * lg;
    const uint16_t* xrow1 = x + (size_t)min(16 + lr, M - 1) * K + 8 * lg;

    auto load = [&](int j, Group& o) {
        const int g = wave + kR32Waves * j;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t* row = codes + (size_t)(16 * g + 4 * s) * N;  // packed rows 16g + 4s + lg
            if (kVec) {
                const u32x4_t v = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(row) + lane_off));
#pragma unroll
                for (int c = 0; c < 4; ++c) o.w[s][c] = v[c];
            } else {
                const uint32_t* r = row + (size_t)lg * N;
#pragma unroll
                for (int c = 0; c < 4; ++c) o.w[s][c] = r[min(cbase + c, N - 1)];
            }
            o.a[s][0] = *reinterpret_cast<const uint4*>(xrow0 + g * 128 + 32 * s);
            o.a[s][1] = *reinterpret_cast<const uint4*>(xrow1 + g * 128 + 32 * s);
        }
        if constexpr (kP32) {
            const float* sp = scales32 + (size_t)g * N;
            const float* mp = mins32 + (size_t)g * N;
            if (kVec) {
                const float4 a = *reinterpret_cast<const float4*>(sp + cbase), b = *reinterpret_cast<const float4*>(mp + cbase);
                o.s[0] = a.x, o.s[1] = a.y, o.s[2] = a.z, o.s[3] = a.w;
                o.m[0] = b.x, o.m[1] = b.y, o.m[2] = b.z, o.m[3] = b.w;
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    o.s[c] = sp[min(cbase + c, N - 1)];
                    o.m[c] = mp[min(cbase + c, N - 1)];
                }
            }
            return;
        }
        const uint16_t* sp = scales + (size_t)g * N;
        const uint16_t* mp = mins + (size_t)g * N;
        if (kVec) {
            const uint2 a = *reinterpret_cast<const uint2*>(sp + cbase), b = *reinterpret_cast<const uint2*>(mp + cbase);
            o.s[0] = a.x, o.s[1] = a.y, o.m[0] = b.x, o.m[1] = b.y;
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c0 = min(cbase + 2 * h, N - 1), c1 = min(cbase + 2 * h + 1, N - 1);
                o.s[h] = (uint32_t)sp[c0] | ((uint32_t)sp[c1] << 16);
                o.m[h] = (uint32_t)mp[c0] | ((uint32_t)mp[c1] << 16);
            }
        }
    };

    // the magic exponent in a VGPR (the mask stays in an SGPR): one v_and_or_b32 per pair
    uint32_t magic_v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(magic_v) : "s"(magic));
    constexpr uint32_t kOne = kF16 ? 0x3C003C00u : 0x3F803F80u;  // 1.0 in both halves
    const u32x4_t ones_u = {kOne, kOne, kOne, kOne};
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, ones_u);

    // accumulator element e of lane l in a 16x16 tile: row 4 (l / 16) + e, column l % 16; tile c
    // of a row block holds the columns cbase + c
    float yacc[4][2][4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) yacc[c][rt][e] = 0.0f;

    auto compute = [&](const Group& o) {
        f32x4_t acc[4][2], accs[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            accs[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c][rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8_t b[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) b[c] = r32_unpack(o.w[s][c], mask, magic_v);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const bf16x8_t a = r32_pair_up(o.a[s][rt]);
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    acc[c][rt] = mfma(a, b[c], acc[c][rt]);
                accs[rt] = mfma(a, ones, accs[rt]);
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float sv, mv;
            if constexpr (kP32) {
                sv = o.s[c], mv = o.m[c];
            } else {
                const uint32_t sb = (c & 1) ? (o.s[c >> 1] >> 16) : (o.s[c >> 1] & 0xFFFFu);
                const uint32_t mb = (c & 1) ? (o.m[c >> 1] >> 16) : (o.m[c >> 1] & 0xFFFFu);
                sv = bf16_bits_to_f32(sb), mv = bf16_bits_to_f32(mb);
            }
            const float cc = __builtin_fmaf(-kOffset, sv, mv);  // min - 128 s (or - 1024 s)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    yacc[c][rt][e] = __builtin_fmaf(sv, acc[c][rt][e], yacc[c][rt][e]);
                    yacc[c][rt][e] = __builtin_fmaf(cc, accs[rt][e], yacc[c][rt][e]);
                }
        }
    };

    // groups j, j + 1 in flight while j is used; slot j % 2 is reloaded right after its use
    Group sl[kR32Ahead];
#pragma unroll
    for (int d = 0; d < kR32Ahead; ++d)
        if (d < J) load(d, sl[d]);
    for (int j0 = 0; j0 < J; j0 += kR32Ahead) {
#pragma unroll
        for (int d = 0; d < kR32Ahead; ++d) {
            if (j0 + d < J) compute(sl[d]);
            if (j0 + d + kR32Ahead < J) load(j0 + d + kR32Ahead, sl[d]);
        }
    }

#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            *reinterpret_cast<float4*>(&part[wave][16 * rt + 4 * lg + e][4 * lr]) =
                make_float4(yacc[0][rt][e], yacc[1][rt][e], yacc[2][rt][e], yacc[3][rt][e]);
    __syncthreads();
    for (int idx = threadIdx.x; idx < 32 * kMidCols; idx += 64 * kR32Waves) {
        const int row = idx / kMidCols, col = idx % kMidCols, n = n0 + col;
        if (row >= M || n >= N) continue;
        float sum = 0.0f;
#pragma unroll
        for (int v = 0; v < kR32Waves; ++v) sum += part[v][row][col];
        y[(size_t)row * N + n] = kF16 ? f32_to_f16_bits(sum) : f32_to_bf16_bits(sum);
    }
}

// ---- 33..64 rows ------------------------------------------------------------------------------

// 16-byte chunk c of activation row r sits at chunk c ^ (r & 15) of the row: the 16 rows of a
// fragment read then hit 16 different 4-bank groups.
__device__ __forceinline__ int mid_swizzle(int r, int c) { return c ^ (r & 15); }

// w_hat = bf16_rne(fmaf(q, s, m)) for the 8 codes of one word, in k order: one MFMA B fragment.
__device__ __forceinline__ bf16x8_t dequant_fragment(uint32_t w, uint32_t mlo, uint32_t mhi, float s, float s16,
                                                     float m) {
    const uint32_t ev = w & mlo, od = w & mhi;  // codes 0 2 4 6 / 16 x codes 1 3 5 7
    const float v0 = __builtin_fmaf((float)(ev & 0xFF), s, m);
    const float v2 = __builtin_fmaf((float)((ev >> 8) & 0xFF), s, m);
    const float v4 = __builtin_fmaf((float)((ev >> 16) & 0xFF), s, m);
    const float v6 = __builtin_fmaf((float)(ev >> 24), s, m);
    const float v1 = __builtin_fmaf((float)(od & 0xFF), s16, m);
    const float v3 = __builtin_fmaf((float)((od >> 8) & 0xFF), s16, m);
    const float v5 = __builtin_fmaf((float)((od >> 16) & 0xFF), s16, m);
    const float v7 = __builtin_fmaf((float)(od >> 24), s16, m);
    const uint4 u = make_uint4(pack2_bf16(v0, v1), pack2_bf16(v2, v3), pack2_bf16(v4, v5), pack2_bf16(v6, v7));
    return __builtin_bit_cast(bf16x8_t, u);
}

template <int MR, int KP>
__global__ __launch_bounds__(128 * KP) void mid_g128_kernel(const uint16_t* __restrict__ x,
                                                            const uint32_t* __restrict__ codes,
                                                            const uint16_t* __restrict__ scales,
                                                            const uint16_t* __restrict__ mins,
                                                            uint16_t* __restrict__ y, int M, int N, int K,
                                                            uint32_t mask_lo, uint32_t mask_hi) {
    constexpr int kThreads = 128 * KP;
    constexpr int kRB = MR / 32;           // 32-row MFMA blocks
    constexpr int kRowChunks = KP * 16;    // 16-byte chunks per staged row (KP groups of 128 k)
    constexpr int kStage = MR * kRowChunks;  // chunks per stage
    constexpr int kPerThread = kStage / kThreads;  // = MR / 8
    static_assert(kStage % kThreads == 0, "staging split");
    __shared__ u32x4_t xs[2][kStage];

    const int lane = lane_id(), wave = wave_id();
    const int l32 = lane & 31, lh = lane >> 5;
    const int half = wave & 1, phase = wave >> 1;
    const int n0 = blockIdx.x * kMidCols, m0 = blockIdx.y * MR;
    const int col = n0 + 32 * half + l32;
    const int ccol = min(col, N - 1);  // columns past N re-read the last one and are never stored
    const int G = K / 128;

    // staging: thread t moves chunks q = t + kThreads * j: row q / kRowChunks, chunk q % kRowChunks
    auto load_x = [&](int st, u32x4_t (&r)[kPerThread]) {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int q = (int)threadIdx.x + kThreads * j;
            const int row = q / kRowChunks, c = q % kRowChunks;
            const int gm = min(m0 + row, M - 1);
            const int k = min(st * KP * 128 + 8 * c, K - 8);  // chunks past K: any valid data (unused)
            r[j] = *reinterpret_cast<const u32x4_t*>(x + (size_t)gm * K + k);
        }
    };
    auto store_x = [&](int buf, const u32x4_t (&r)[kPerThread]) {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int q = (int)threadIdx.x + kThreads * j;
            const int row = q / kRowChunks, c = q % kRowChunks;
            xs[buf][row * kRowChunks + mid_swizzle(row, c)] = r[j];
        }
    };
    // this wave's group of step st: packed words of its 8 k-steps, scale and minimum
    struct BSet {
        uint32_t w[8], sb, mb;
        bool live;  // the group lies inside K (wave-uniform)
    };
    auto load_b = [&](int st, BSet& b) {
        const int g = st * KP + phase;
        b.live = g < G;
        const int gc = min(g, G - 1);
#pragma unroll
        for (int s = 0; s < 8; ++s) b.w[s] = codes[(size_t)(16 * gc + 2 * s + lh) * N + ccol];
        b.sb = scales[(size_t)gc * N + ccol];
        b.mb = mins[(size_t)gc * N + ccol];
    };

    f32x16_t acc[kRB];
#pragma unroll
    for (int i = 0; i < kRB; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;

    auto mma = [&](int buf, const BSet& b) {
        if (!b.live) return;  // wave-uniform: a group past K is skipped
        const float s = bf16_bits_to_f32(b.sb), m = bf16_bits_to_f32(b.mb);
        const float s16 = s * 0.0625f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const bf16x8_t bf = dequant_fragment(b.w[ks], mask_lo, mask_hi, s, s16, m);
            const int c = phase * 16 + 2 * ks + lh;  // chunk of this lane's 8 k in the staged row
#pragma unroll
            for (int i = 0; i < kRB; ++i) {
                const int r = 32 * i + l32;
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, xs[buf][r * kRowChunks + mid_swizzle(r, c)]);
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bf, acc[i], 0, 0, 0);
            }
        }
    };

    // Software pipeline, four steps per trip (steps is a multiple of 4; the surplus steps are
    // skipped groups).  Step s: the activations of s+2 are requested into one register set while
    // those of s+1 (requested during s-1) go to the other LDS buffer at the end of the step;
    // every second step requests the weights of the two steps after next.  Each load thus has
    // at least one whole step to arrive before anything waits for it, and no loaded register is
    // ever copied (a copy would wait for its load).  Loads past the end are clamped and unused.
    const int steps = ((G + KP - 1) / KP + 3) & ~3;
    auto clampst = [&](int st) { return min(st, steps - 1); };
    u32x4_t xa[kPerThread], xb[kPerThread];
    BSet p0, p1, q0, q1;
    load_x(0, xa);
    load_x(clampst(1), xb);
    load_b(0, p0);
    load_b(clampst(1), p1);
    store_x(0, xa);
    __syncthreads();
    for (int st = 0; st < steps; st += 4) {
        load_b(clampst(st + 2), q0);
        load_b(clampst(st + 3), q1);
        load_x(clampst(st + 2), xa);
        mma(0, p0);
        store_x(1, xb);  // activations of st + 1
        __syncthreads();

        load_x(clampst(st + 3), xb);
        mma(1, p1);
        store_x(0, xa);  // st + 2
        __syncthreads();

        load_b(clampst(st + 4), p0);
        load_b(clampst(st + 5), p1);
        load_x(clampst(st + 4), xa);
        mma(0, q0);
        store_x(1, xb);  // st + 3
        __syncthreads();

        load_x(clampst(st + 5), xb);
        mma(1, q1);
        store_x(0, xa);  // st + 4
        __syncthreads();
    }

    // Sum the KP phases in phase order: each wave writes its tile to LDS (the staging buffers
    // are free now), then phase 0 adds the others to its registers.  D element e of lane l is
    // row 8 (e / 4) + 4 (l / 32) + e % 4 of the 32-row block, column l % 32.
    float* part = reinterpret_cast<float*>(&xs[0][0]);
    constexpr int kTile = MR * 32;  // fp32 per (half, phase) tile
    static_assert(2 * KP * kTile * 4 <= (int)sizeof(xs), "partials fit in the staging buffers");
    if (phase > 0) {
#pragma unroll
        for (int i = 0; i < kRB; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = 32 * i + 8 * (e / 4) + 4 * lh + (e % 4);
                part[((phase * 2 + half) * MR + r) * 32 + l32] = acc[i][e];
            }
    }
    __syncthreads();
    if (phase == 0) {
#pragma unroll
        for (int i = 0; i < kRB; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = 32 * i + 8 * (e / 4) + 4 * lh + (e % 4);
                float v = acc[i][e];
#pragma unroll
                for (int p = 1; p < KP; ++p) v += part[((p * 2 + half) * MR + r) * 32 + l32];
                if (m0 + r < M && col < N) y[(size_t)(m0 + r) * N + col] = f32_to_bf16_bits(v);
            }
    }
}


// ---- 17..64 rows, factored, every operand by direct-to-LDS copies ----------------------------

// R rows per block (64 or 32).  The 8 waves form kGS sets of 8 / kGS waves (R = 64: 2 sets of 4;
// R = 32: 4 sets of 2); set s runs the groups g = s (mod kGS), and within a set wave j owns output
// rows 32 (j % (R / 32)) .. +31 and columns 32 (j / (R / 32)) .. +31 of the block's 64, over all of
// K.  A stage holds kGS consecutive groups: x (R rows x kGS * 128 k, each row's 16-byte chunks
// XOR-swizzled by row so the fragment reads are conflict-free; each copy is 1 KB of x: 2 rows x
// 512 B, or 1 KB of one row), their 16 kGS packed rows and parameters; three stages, the copies two
// stages ahead, one barrier per stage.
template <int R>
struct MidR {
    static constexpr int kGS = R == 64 ? 2 : 4;        // groups per stage
    static constexpr int kWPG = 8 / kGS;               // waves per group
    static constexpr int kRB = kGS * 256;              // bytes of one x row in a stage
    static constexpr int kX = R * kRB;                 // 32 KB
    static constexpr int kW = kGS * 16 * 256;          // packed words
    static constexpr int kP = kGS * 512;               // per group: scales (256 B slot), minimums (256 B slot)
    static constexpr int kS = kX + kW + kP;            // one stage
    static constexpr int kRPI = 1024 / kRB;            // x rows per copy instruction
    static constexpr int kWI = kGS / 2;                // word copies per wave and stage
    static constexpr int kCopies = 4 + kWI + 1;        // copies per wave and stage
    static constexpr int kStages = 3;
    static_assert(kStages * kS <= 160 * 1024, "LDS");
};

// kF16: fp16 activations and output on the fp16 matrix cores, codes as 1024 + q, else bf16 and
// 128 + q.  kP32: fp32 scales and minimums [K/128][N] (the prepared zero-point copy), else bf16.
// N % 4 == 0, K / 128 a multiple of kGS, 1 <= M <= R.
template <int R, bool kF16, bool kP32>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void midr_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ codes, const void* __restrict__ scales_v,
                 const void* __restrict__ mins_v, uint16_t* __restrict__ y, int M, int N, int K, uint32_t mask,
                 uint32_t magic, float* __restrict__ ws, int gps) {
    using L = MidR<R>;
    constexpr int kGS = L::kGS, kWPG = L::kWPG, kRB = L::kRB, kRPI = L::kRPI;
    __shared__ __attribute__((aligned(16))) uint8_t smem[L::kStages * L::kS];
    constexpr float kOffset = kF16 ? 1024.0f : 128.0f;  // the magic number's value at q = 0
    constexpr uint32_t kOne = kF16 ? 0x3C003C00u : 0x3F803F80u;
    const int lane = lane_id(), wave = wave_id();
    const int set = wave / kWPG, wj = wave % kWPG;
    const int wm = wj % (R / 32), wn = wj / (R / 32);
    const int l32 = lane & 31, lh = lane >> 5;
    const int n0 = blockIdx.x * kMidCols;
    const int G = K >> 7;
    // K split over blockIdx.y (gps groups each, a multiple of kGS): this block's groups gs ..
    const int gs = blockIdx.y * gps;
    const int P = (min(G, gs + gps) - gs) / kGS;  // stages' worth of groups
    const uint32_t sm = lds_addr(smem);

    // Copy offsets (constant over the stages).  x: copy i of wave w fills the kRPI rows from
    // (4 w + i) kRPI; lane l lands on 16-byte position p = l % (64 / kRPI) of row
    // r = (4 w + i) kRPI + l / (64 / kRPI) and reads the chunk p ^ (r % 16) of that row's kGS * 128 k
    // (rows past M repeat row M - 1; they feed only outputs that are never stored).
    uint32_t xoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (4 * wave + i) * kRPI + lane / (64 / kRPI);
        const int p = lane % (64 / kRPI);
        xoff[i] = (uint32_t)(((size_t)min(r, M - 1) * K + 8 * (p ^ (r & 15))) * 2);
    }
    // words: wave w copies the stage's packed rows 2 kGS w .. +2 kGS - 1, four per copy; lane l the
    // 4 columns at 4 (l % 16) of the copy's row l / 16 (the last block's columns past N repeat the
    // last 4)
    const uint32_t woff = (uint32_t)(((size_t)(lane >> 4) * N + min(n0 + 4 * (lane & 15), N - 4)) * 4);
    // parameters: wave w copies the scales (w even) or minimums (w odd) of the stage's group
    // (w / 2) % kGS: bf16, lane l the dword of columns n0 + 2 l, +1 (lanes past 31 repeat dword 31),
    // or fp32, lane l column n0 + l
    const uint32_t poff = kP32 ? (uint32_t)(min(n0 + lane, N - 1) * 4) : (uint32_t)(min(n0 / 2 + min(lane, 31), N / 2 - 1) * 4);
    const char* const parr = static_cast<const char*>((wave & 1) ? mins_v : scales_v);
    constexpr size_t kPBytes = kP32 ? 4 : 2;
    const int pgi = (wave >> 1) % kGS;

    // this wave's copies of stage p into LDS stage st (a stage past the last repeats it)
    auto issue = [&](int p, int st) {
        const int g0 = gs + min(p, P - 1) * kGS;  // first group of the stage
        const uint32_t base = sm + (uint32_t)(st * L::kS);
        const char* xs = reinterpret_cast<const char*>(x + (size_t)g0 * 128);
        dma16<0>(xoff[0], xs, base + 4096u * wave);
        dma16<1024>(xoff[1], xs, base + 4096u * wave);
        dma16<2048>(xoff[2], xs, base + 4096u * wave);
        dma16<3072>(xoff[3], xs, base + 4096u * wave);
        static_for<0, L::kWI>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            dma16<L::kX + 1024 * j>(woff, codes + (size_t)(16 * g0 + 2 * kGS * wave + 4 * j) * N,
                                    base + (uint32_t)(2 * kGS * 256) * wave);
        });
        dma4<L::kX + L::kW>(poff, parr + (size_t)(g0 + pgi) * N * kPBytes, base + 512u * pgi + 256u * (wave & 1));
    };

    uint32_t magic_v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(magic_v) : "s"(magic));
    const u32x4_t ones_u = {kOne, kOne, kOne, kOne};
    const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, ones_u);
    auto mfma = [](bf16x8_t a, bf16x8_t b, f32x16_t c) {
        if constexpr (kF16) {
            typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
            return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                          0, 0, 0);
        } else {
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
        }
    };
    const int col = 32 * wn + l32;   // this lane's column of the block
    const int arow = 32 * wm + l32;  // this lane's A row
    float yacc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) yacc[e] = 0.0f;

    issue(0, 0);
    issue(1, 1);
    int cur = 0;  // the LDS stage of stage p
    for (int p = 0; p < P; ++p) {
        wait_vm<L::kCopies>();  // this wave's copies of stage p have landed (those of p + 1 may not have)
        __syncthreads();        // ... and every wave's; all are done with stage p - 1, which is refilled next
        issue(p + 2, cur == 0 ? L::kStages - 1 : cur - 1);
        const uint8_t* sx = smem + cur * L::kS;
        const uint8_t* sw = sx + L::kX + set * 4096;
        const uint8_t* sp = sx + L::kX + L::kW + set * 512;
        cur = cur + 1 == L::kStages ? 0 : cur + 1;
        // the group's 8 A fragments and 8 words, read from LDS at once
        uint4 av[8];
        uint32_t wv[8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int ch = 2 * ks + lh;  // 16-byte chunk of the group's 128 k (the word row of the k-step)
            av[ks] = *reinterpret_cast<const uint4*>(sx + arow * kRB + (((16 * set + ch) ^ (arow & 15)) * 16));
            wv[ks] = *reinterpret_cast<const uint32_t*>(sw + ch * 256 + col * 4);
        }
        float s, mn;
        if constexpr (kP32) {
            s = *reinterpret_cast<const float*>(sp + 4 * col);
            mn = *reinterpret_cast<const float*>(sp + 256 + 4 * col);
        } else {
            s = bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(sp + 2 * col));
            mn = bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(sp + 256 + 2 * col));
        }
        f32x16_t acc, accs;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = accs[e] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const bf16x8_t a = r32_pair_up(av[ks]);
            acc = mfma(a, r32_unpack(wv[ks], mask, magic_v), acc);
            accs = mfma(a, ones, accs);
        }
        const float c = __builtin_fmaf(-kOffset, s, mn);  // min - 128 s (or - 1024 s)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            yacc[e] = __builtin_fmaf(s, acc[e], yacc[e]);
            yacc[e] = __builtin_fmaf(c, accs[e], yacc[e]);
        }
    }
    wait_vm<0>();     // no copy may still be writing this block's LDS
    __syncthreads();  // every wave is done reading the stages, which now take the other sets' sums
    float* part = reinterpret_cast<float*>(smem);
    if (set > 0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) part[(wave * 16 + e) * 64 + lane] = yacc[e];
    }
    __syncthreads();
    if (set == 0) {
        // element e of lane l: row 8 (e / 4) + 4 (l / 32) + e % 4 of the wave's 32, column l % 32
        const int n = n0 + col;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            float v = yacc[e];
#pragma unroll
            for (int t = 1; t < kGS; ++t) v += part[((t * kWPG + wj) * 16 + e) * 64 + lane];  // sets in order
            const int m = 32 * wm + 8 * (e / 4) + 4 * lh + (e % 4);
            if (m < M && n < N) {
                if (ws != nullptr)  // a K split's fp32 partial sums, [split][M][N]
                    ws[((size_t)blockIdx.y * M + m) * N + n] = v;
                else
                    y[(size_t)m * N + n] = kF16 ? f32_to_f16_bits(v) : f32_to_bf16_bits(v);
            }
        }
    }
}

// splits > 1: K split over gridDim.y, gps groups per split (a multiple of the stage's groups),
// fp32 partial sums to ws [splits][M][N] (y untouched).
template <int R, bool kF16, bool kP32>
void launch_midr(const uint16_t* x, int64_t M, const uint32_t* codes, const void* scales, const void* mins, int64_t N,
                 int64_t K, uint16_t* y, hipStream_t stream, float* ws = nullptr, int splits = 1, int gps = 0) {
    if (splits <= 1) gps = (int)(K / 128);
    hipLaunchKernelGGL((midr_kernel<R, kF16, kP32>), dim3((unsigned)((N + kMidCols - 1) / kMidCols), (unsigned)splits),
                       dim3(512), 0, stream, x, codes, scales, mins, y, (int)M, (int)N, (int)K, 0x000F000Fu,
                       kF16 ? 0x64006400u : 0x43004300u, ws, gps);
}

}  // namespace

hipError_t launch_rows32_prepared_zp(const uint16_t* x, int64_t M, bool act_f16, const uint32_t* codes,
                                     const float* scales, const float* mins, int64_t N, int64_t K, uint16_t* y,
                                     hipStream_t stream) {
    const unsigned gx = (unsigned)((N + kMidCols - 1) / kMidCols);
    const uint32_t magic = act_f16 ? 0x64006400u : 0x43004300u;  // 1024 (fp16) or 128 (bf16), both halves
    auto go = [&](auto vec, auto f16) {
        hipLaunchKernelGGL((mid_rows32_kernel<decltype(vec)::value, decltype(f16)::value, true>), dim3(gx),
                           dim3(64 * kR32Waves), 0, stream, x, codes, scales, mins, y, (int)M, (int)N, (int)K,
                           0x000F000Fu, magic);
    };
    using T = std::true_type;
    using F = std::false_type;
    if (midr_fits(32, N, K)) {
        if (act_f16) launch_midr<32, true, true>(x, M, codes, scales, mins, N, K, y, stream);
        else launch_midr<32, false, true>(x, M, codes, scales, mins, N, K, y, stream);
    } else if (N % 4 == 0) {
        if (act_f16) go(T{}, T{}); else go(T{}, F{});
    } else {
        if (act_f16) go(F{}, T{}); else go(F{}, F{});
    }
    return hipGetLastError();
}

hipError_t launch_rows64_prepared_zp(const uint16_t* x, int64_t M, bool act_f16, const uint32_t* codes,
                                     const float* scales, const float* mins, int64_t N, int64_t K, uint16_t* y,
                                     hipStream_t stream) {
    if (act_f16) launch_midr<64, true, true>(x, M, codes, scales, mins, N, K, y, stream);
    else launch_midr<64, false, true>(x, M, codes, scales, mins, N, K, y, stream);
    return hipGetLastError();
}

hipError_t launch_mid_g128_split(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                                 const uint16_t* mins, int64_t N, int64_t K, uint16_t* y, float* ws, hipStream_t stream) {
    const MidSplit sp = mid_split(M, N, K);
    if (sp.rows == 32)
        launch_midr<32, false, false>(x, M, codes, scales, mins, N, K, y, stream, ws, sp.splits, sp.gps);
    else
        launch_midr<64, false, false>(x, M, codes, scales, mins, N, K, y, stream, ws, sp.splits, sp.gps);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_splitk_reduce(ws, M * N, sp.splits, y, stream);
}

hipError_t launch_mid_g128(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                           const uint16_t* mins, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
    const unsigned gx = (unsigned)((N + kMidCols - 1) / kMidCols);
    if (M <= 32 && midr_fits(32, N, K)) {
        launch_midr<32, false, false>(x, M, codes, scales, mins, N, K, y, stream);
    } else if (M <= 32) {
        if (N % 4 == 0)
            hipLaunchKernelGGL((mid_rows32_kernel<true>), dim3(gx), dim3(64 * kR32Waves), 0, stream, x, codes, scales, mins,
                               y, (int)M, (int)N, (int)K, 0x000F000Fu, 0x43004300u);
        else
            hipLaunchKernelGGL((mid_rows32_kernel<false>), dim3(gx), dim3(64 * kR32Waves), 0, stream, x, codes, scales,
                               mins, y, (int)M, (int)N, (int)K, 0x000F000Fu, 0x43004300u);
    } else if (midr_fits(64, N, K)) {
        launch_midr<64, false, false>(x, M, codes, scales, mins, N, K, y, stream);
    } else {
        const unsigned gy = (unsigned)((M + 63) / 64);
        hipLaunchKernelGGL((mid_g128_kernel<64, 4>), dim3(gx, gy), dim3(128 * 4), 0, stream, x, codes, scales, mins, y,
                           (int)M, (int)N, (int)K, 0x0F0F0F0Fu, 0xF0F0F0F0u);
    }
    return hipGetLastError();
}

}  // namespace w4a16
