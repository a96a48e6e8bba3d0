// mid.hip -- mid-M W4A16 path (17 <= M <= 64) for the [K/8][N] G128 format, on bf16 MFMA.
//
// The large-M kernel amortizes one dequant of a weight over 256 rows and needs 256 output
// tiles of 256 x 224 to fill the chip; at a few dozen rows it has neither, and the skinny
// kernel's trick (all of K's activations resident in LDS) stops fitting past 16 rows.  This
// kernel streams the weights once per 64-row slice of M, like a GEMV, and does the dequant of
// vidyal.ai "Low-Precision Kernels", Step 2 (w_hat = bf16_rne(fmaf(q, s, min)), the reference
// value) straight into MFMA B fragments, with no LDS for the weights:
//
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
#include "device_common.h"
#include "launch.h"

namespace w4a16 {

namespace {

constexpr int kMidCols = 64;

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

}  // namespace

hipError_t launch_mid_g128(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                           const uint16_t* mins, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
    const unsigned gx = (unsigned)((N + kMidCols - 1) / kMidCols);
    if (M <= 32) {
        hipLaunchKernelGGL((mid_g128_kernel<32, 4>), dim3(gx, 1), dim3(128 * 4), 0, stream, x, codes, scales, mins, y,
                           (int)M, (int)N, (int)K, 0x0F0F0F0Fu, 0xF0F0F0F0u);
    } else {
        const unsigned gy = (unsigned)((M + 63) / 64);
        hipLaunchKernelGGL((mid_g128_kernel<64, 4>), dim3(gx, gy), dim3(128 * 4), 0, stream, x, codes, scales, mins, y,
                           (int)M, (int)N, (int)K, 0x0F0F0F0Fu, 0xF0F0F0F0u);
    }
    return hipGetLastError();
}

}  // namespace w4a16
