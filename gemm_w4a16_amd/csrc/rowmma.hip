// rowmma.hip -- the row-major weight formats (Q4 block-32, the integer-zero-point format, W8 per
// row) against fp16 activations on the fp16 matrix cores, 16 activation rows per pass over the
// weights.
//
// The pages' GEMV for these formats takes one activation row (thuongvuho.com "Why My 4-Bit CUDA
// Kernel Wasn't Faster"; anrans.github.io "Quantization and GEMV", "W4A16: dequantizing in
// registers" and "Exercises", 1); a batch of rows reuses every weight once per row, so here the
// dequantized weights of a 16-row tile feed v_mfma_f32_16x16x32_f16 against 16-row tiles of x:
//
//  * A lane's 16-byte load is one code block of one weight row: 32 k of Q4 or of the zero-point
//    format (both lay a row's codes out as 16 bytes per 32 k, k = 2j in the low nibble of byte j),
//    16 k of W8.  Lane (j, g) of a wave loads block 4u + g of weight row j of its 16-row tile, so
//    one unit u of 4 blocks covers 128 k (64 for W8) of 16 rows.
//  * The MFMA sums over 32 k, which here are 8 k from each of the 4 lane groups: the k order only
//    has to agree between A and B.  The 8 k of chunk c of lane group g's block are
//    k = 32(4u + g) + 8c + 0..7, so each lane's B fragment for MFMA c is chunk c of its own block,
//    and its A fragment is the same 8 k of its activation row.  No data crosses lanes.
//  * Q4 dequant is exact up to one rounding: the nibble pair (q_t, q_{t+4}) of a code dword becomes
//    the fp16 pair (1024 + q) with one AND-OR (the magic-number trick of both pages); subtracting
//    1032 (the offset and the bias 8) is exact, and one packed multiply by the scale rounds
//    (q - 8) s to fp16.  W8 bytes become 1024 + u, u = q + 128, and then q exactly; the row's fp32
//    scale multiplies the row's total once (the exercise's scale after accumulation).  Packed fp16
//    arithmetic, no packed fp32.  The zero-point format is factored per group instead (its scale
//    and zero point change only every 128 k): the MFMAs run on 1024 + q itself, a chain against
//    ones gives sum(x), and each group adds s acc - (1024 + z) s sum(x) in fp32 -- a quarter of the
//    exact dequant's VALU work per code word.
//  * Per wave, the activations of its units stay in registers while it walks the block's row
//    tiles; waves split K, and their partial tiles are added through LDS in a fixed order, so
//    results are bitwise reproducible run to run.
//  * The block's scales (and zero points) are contiguous in their [N][K/32] or [N][K/128] arrays:
//    each thread requests 16-byte pieces of them before its weight loads, writes them to LDS once
//    they arrive (an LDS-only barrier, the weight loads stay in flight), and the math reads them
//    there.  Two-byte loads per lane and use cost more than the weights did.
//  * Every load is unconditional (clamped addresses; what lies past the data meets a zero
//    activation): a load under a divergent branch, or one feeding a conditional store, makes the
//    wave wait for every load issued before it.
//  * 16 activation rows per launch; more rows take more launches, each a pass over the weights.
#include "device_common.h"
#include "launch.h"

namespace w4a16 {

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;

constexpr int kRmWaves = 16;
constexpr int kRmRows = 64;              // weight rows per block: four 16-row tiles
constexpr int kRmTiles = kRmRows / 16;

enum RmFmt { kRmQ4 = 0, kRmZP = 1, kRmW8 = 2 };

__device__ __forceinline__ h2_t as_h2(uint32_t v) { return __builtin_bit_cast(h2_t, v); }
__device__ __forceinline__ uint32_t as_u32(h2_t v) { return __builtin_bit_cast(uint32_t, v); }

// (x0..x7) as dwords (x0,x1) (x2,x3) (x4,x5) (x6,x7) -> (x0,x4) (x1,x5) (x2,x6) (x3,x7): the order of
// the nibble pairs (q_t, q_{t+4}) of a code dword.
__device__ __forceinline__ u32x4_t pair_nibble_order(u32x4_t v) {
    return u32x4_t{(v[0] & 0xFFFFu) | (v[2] << 16), (v[0] >> 16) | (v[2] & 0xFFFF0000u),
                   (v[1] & 0xFFFFu) | (v[3] << 16), (v[1] >> 16) | (v[3] & 0xFFFF0000u)};
}
// -> (x0,x2) (x1,x3) (x4,x6) (x5,x7): the order of the byte pairs (bytes 0 and 2, 1 and 3) of W8.
__device__ __forceinline__ u32x4_t pair_byte_order(u32x4_t v) {
    return u32x4_t{(v[0] & 0xFFFFu) | (v[1] << 16), (v[0] >> 16) | (v[1] & 0xFFFF0000u),
                   (v[2] & 0xFFFFu) | (v[3] << 16), (v[2] >> 16) | (v[3] & 0xFFFF0000u)};
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Scale (and zero-point) elements a block stages in LDS: 64 rows x K/32 fp16 scales (Q4), or
// 64 rows x K/128 scales and as many zero points; with more, they are loaded per use.
constexpr int kParamElems = 32768;

// One pass of one wave: UP units, each the code blocks of its row tiles and the activations of
// its k, in the k order of the dequantized pairs.
template <int kTiles, int MT, int kChunks, int UP>
struct RmPass {
    u32x4_t w[UP][kTiles];
    u32x4_t xa[UP][MT][kChunks];               // as loaded; paired (or zeroed) at use
    uint32_t sc[UP][kTiles], zc[UP][kTiles];  // per-use scale / zero point when not staged
    int u[UP], b[UP];
    bool live[UP][MT];                         // activation row and block exist
};

// kFmt: the format.  MT: 16-row activation tiles (M <= 16 MT; the launchers use MT = 1).  kR: row-tile groups; the 16
// waves are kS = 16 / kR K-slices times kR groups, each wave walking 4 / kR of the block's row
// tiles.  UP: units per pass.  kStage: 16-byte pieces of the block's scales (and zero points)
// each thread stages in LDS (0: loaded per use).  kVecP: those arrays' rows are whole pieces.
// kDB: two passes in flight per wave (the next pass's loads are issued before this pass's math).
template <int kFmt, int MT, int kR, int UP, int kStage, bool kVecP, bool kDB>
__global__ __launch_bounds__(1024) void rowmma_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ codes,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint16_t* __restrict__ zeros, uint16_t* __restrict__ y,
                                                      int M, int N, int K) {
    constexpr bool kW8 = kFmt == kRmW8, kZP = kFmt == kRmZP;
    constexpr int kBlockK = kW8 ? 16 : 32;        // k per 16-byte code block
    constexpr int kChunks = kBlockK / 8;          // MFMAs per unit and A tile
    constexpr int kS = kRmWaves / kR;             // K-slices
    constexpr int kMyTiles = kRmTiles / kR;       // row tiles per wave
    static_assert(!(kW8 && kStage), "W8 has one scale per row, applied to the row's total");
    static_assert(kStage * 8 * 1024 <= (kFmt == kRmZP ? kParamElems / 2 : kParamElems), "staged parameters fit");
    __shared__ float part[kS][kRmRows][16 * MT];
    __shared__ uint16_t prm[kStage > 0 ? kParamElems : 1];
    const int lane = lane_id(), wave = wave_id();
    const int j = lane & 15, g = lane >> 4;
    const int slice = wave % kS, rg = wave / kS;
    const int B = K / kBlockK;                    // code blocks per weight row
    const int U = (B + 3) >> 2;                   // units of 4 blocks (a group of 128 k for ZP)
    const int n0 = blockIdx.x * kRmRows;
    const int rows = min(kRmRows, N - n0);        // weight rows of this block
    const char* cbase = reinterpret_cast<const char*>(codes) + (size_t)n0 * B * 16;
    const int PB = kZP ? U : B;                   // parameters per weight row
    // mask and exponent opaque to the compiler, so each pair is one v_and_or_b32
    uint32_t mask, magic;
    asm volatile("s_mov_b32 %0, %1" : "=s"(mask) : "i"(kW8 ? 0x00FF00FFu : 0x000F000Fu));
    asm volatile("v_mov_b32 %0, %1" : "=v"(magic) : "i"(0x64006400u));  // fp16 1024.0 in both halves
    const h2_t off = {(_Float16)(kW8 ? -1152.0f : (kZP ? -1024.0f : -1032.0f)),
                      (_Float16)(kW8 ? -1152.0f : (kZP ? -1024.0f : -1032.0f))};

    // 0) staged parameters: the block's rows are contiguous in the [N][PB] arrays, so every
    //    thread requests kStage whole 16-byte pieces of them first (element by element when rows
    //    are not whole pieces), with no branch, so that the wait before they are written to LDS,
    //    after this wave's first units are requested, counts exactly these loads
    constexpr int kPieces = kStage > 0 ? kStage : 1;
    const int pcount = rows * PB;                 // elements per staged array
    u32x4_t pv[kZP ? 2 : 1][kPieces];
    if constexpr (kStage > 0) {
#pragma unroll
        for (int a = 0; a < (kZP ? 2 : 1); ++a) {
            const uint16_t* src = (a ? zeros : scales) + (size_t)n0 * PB;
#pragma unroll
            for (int i = 0; i < kPieces; ++i) {
                const int e = 8 * ((int)threadIdx.x + 1024 * i);
                if constexpr (kVecP) {
                    pv[a][i] = *reinterpret_cast<const u32x4_t*>(src + min(e, pcount - 8));
                } else {
                    uint32_t h[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q) h[q] = src[min(e + q, pcount - 1)];
                    pv[a][i] = u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
                }
            }
        }
    }

    // this wave's units: a contiguous range, so its loads of a row's 128 bytes are adjacent; all
    // waves make the same number of passes (dead units past the last one meet zero activations)
    const int upw = (U + kS - 1) / kS;
    const int ubeg = slice * upw;
    const int npass = (upw + UP - 1) / UP;
    using Pass = RmPass<kMyTiles, MT, kChunks, UP>;

    // 1) loads of pass `ps` of this wave, every one unconditional (indices clamped), in the order
    //    they are used
    auto load = [&](int ps, Pass& R) {
#pragma unroll
        for (int p = 0; p < UP; ++p) {
            const int i = UP * ps + p;
            const int uu = ubeg + i;
            const bool unit_live = uu < U && i < upw;
            R.u[p] = min(uu, U - 1);
            R.b[p] = min(4 * R.u[p] + g, B - 1);
#pragma unroll
            for (int r = 0; r < kMyTiles; ++r) {
                const int row = min(16 * (rg + kR * r) + j, rows - 1);
                const uint32_t o = (uint32_t)row * (uint32_t)B + (uint32_t)R.b[p];
                R.w[p][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(cbase + (size_t)o * 16u));
                if constexpr (!kW8 && kStage == 0) {
                    const size_t q = (size_t)(n0 + row) * PB + (kZP ? R.u[p] : R.b[p]);
                    R.sc[p][r] = scales[q];
                    R.zc[p][r] = kZP ? zeros[q] : 0u;
                }
            }
            // activations: loaded unconditionally from clamped addresses (a load under a
            // divergent branch would wait for every load before it); dead ones are zeroed at use
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const int m = 16 * t + j;
                R.live[p][t] = m < M && unit_live && 4 * R.u[p] + g < B;
                const u32x4_t* src =
                    reinterpret_cast<const u32x4_t*>(x + (size_t)min(m, M - 1) * K + (size_t)R.b[p] * kBlockK);
#pragma unroll
                for (int c = 0; c < kChunks; ++c) R.xa[p][t][c] = src[c];
            }
        }
    };

    f32x4_t acc[kMyTiles][MT];
#pragma unroll
    for (int r = 0; r < kMyTiles; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // 2) per unit and row tile: dequantize each chunk into a B fragment and multiply it with every
    //    activation tile
    // The zero-point format, factored per unit (one group of 128 k) as the small-M kernel does:
    // the B fragments are the exact fp16 1024 + q (one AND-OR per pair), a fifth MFMA chain
    // against ones gives sum(x) per activation row, and the group's epilogue adds
    // s acc + c sum(x) with c = -(1024 + z) s.  An all-zero weight row still gives exact zeros:
    // acc is 1024 sum(x) from the same MFMA order.
    auto compute_zp = [&](const Pass& R) {
        const u32x4_t ones_u = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};  // fp16 1.0 pairs
        const f16x8_t ones = __builtin_bit_cast(f16x8_t, ones_u);
#pragma unroll
        for (int p = 0; p < UP; ++p) {
            f32x4_t au[kMyTiles][MT], sx[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                sx[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < kMyTiles; ++r) au[r][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int c = 0; c < kChunks; ++c) {
                f16x8_t a[MT];
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    const u32x4_t xv = pair_nibble_order(R.xa[p][t][c]);
                    a[t] = __builtin_bit_cast(f16x8_t, R.live[p][t] ? xv : u32x4_t{0u, 0u, 0u, 0u});
                    sx[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], ones, sx[t], 0, 0, 0);
                }
#pragma unroll
                for (int r = 0; r < kMyTiles; ++r) {
                    const uint32_t wd = R.w[p][r][c];
                    const u32x4_t bf = {(wd & mask) | magic, ((wd >> 4) & mask) | magic, ((wd >> 8) & mask) | magic,
                                        ((wd >> 12) & mask) | magic};
#pragma unroll
                    for (int t = 0; t < MT; ++t)
                        au[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], __builtin_bit_cast(f16x8_t, bf),
                                                                          au[r][t], 0, 0, 0);
                }
            }
#pragma unroll
            for (int r = 0; r < kMyTiles; ++r) {
                const int rowl = min(16 * (rg + kR * r) + j, rows - 1);
                uint32_t sv, zv;
                if constexpr (kStage > 0) {
                    sv = prm[rowl * PB + R.u[p]];
                    zv = prm[kParamElems / 2 + rowl * PB + R.u[p]];
                } else {
                    sv = R.sc[p][r];
                    zv = R.zc[p][r];
                }
                const float sf = (float)__builtin_bit_cast(_Float16, (uint16_t)sv);
                const float cf = -(1024.0f + (float)__builtin_bit_cast(_Float16, (uint16_t)zv)) * sf;
#pragma unroll
                for (int t = 0; t < MT; ++t)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        acc[r][t][e] = __builtin_fmaf(sf, au[r][t][e], acc[r][t][e]);
                        acc[r][t][e] = __builtin_fmaf(cf, sx[t][e], acc[r][t][e]);
                    }
            }
        }
    };

    auto compute = [&](const Pass& R) {
        if constexpr (kZP) {
            compute_zp(R);
            return;
        }
#pragma unroll
        for (int p = 0; p < UP; ++p)
#pragma unroll
            for (int r = 0; r < kMyTiles; ++r) {
                const int rowl = min(16 * (rg + kR * r) + j, rows - 1);
                uint32_t sv = 0u, zv = 0u;
                if constexpr (kStage > 0) {
                    sv = prm[rowl * PB + (kZP ? R.u[p] : R.b[p])];
                    if constexpr (kZP) zv = prm[kParamElems / 2 + rowl * PB + R.u[p]];
                } else if constexpr (!kW8) {
                    sv = R.sc[p][r];
                    zv = R.zc[p][r];
                }
                const h2_t s2 = kW8 ? h2_t{(_Float16)1.0f, (_Float16)1.0f} : as_h2(sv | (sv << 16));
                const h2_t z2 = as_h2(zv | (zv << 16));
#pragma unroll
                for (int c = 0; c < kChunks; ++c) {
                    u32x4_t bf;
                    if constexpr (kW8) {
                        // bytes of dwords 2c, 2c + 1: u = q + 128, pairs (0,2) and (1,3) of each
#pragma unroll
                        for (int d = 0; d < 2; ++d) {
                            const uint32_t uu = R.w[p][r][2 * c + d] ^ 0x80808080u;
                            bf[2 * d + 0] = as_u32(as_h2((uu & mask) | magic) + off);
                            bf[2 * d + 1] = as_u32(as_h2(((uu >> 8) & mask) | magic) + off);
                        }
                    } else {
                        const uint32_t wd = R.w[p][r][c];
#pragma unroll
                        for (int tt = 0; tt < 4; ++tt) {
                            h2_t v = as_h2(((wd >> (4 * tt)) & mask) | magic) + off;  // q - 8, or q
                            if constexpr (kZP) v = v - z2;                             // q - z
                            bf[tt] = as_u32(v * s2);
                        }
                    }
                    const f16x8_t bfrag = __builtin_bit_cast(f16x8_t, bf);
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        const u32x4_t xv = kW8 ? pair_byte_order(R.xa[p][t][c]) : pair_nibble_order(R.xa[p][t][c]);
                        const u32x4_t a = R.live[p][t] ? xv : u32x4_t{0u, 0u, 0u, 0u};
                        acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), bfrag,
                                                                           acc[r][t], 0, 0, 0);
                    }
                }
            }
    };

    Pass pa, pb;
    load(0, pa);
    if constexpr (kDB) load(1, pb);
    if constexpr (kStage > 0) {
        __builtin_amdgcn_sched_barrier(0);  // the staged parameters reach LDS after those requests
        const int pe = kZP ? kParamElems / 2 : 0;
#pragma unroll
        for (int a = 0; a < (kZP ? 2 : 1); ++a)
#pragma unroll
            for (int i = 0; i < kPieces; ++i) {
                // unconditional: a thread past the end rewrites, at the clamped place, the very
                // piece it loaded from there (a conditional store would draw the loads after it)
                const int e = 8 * ((int)threadIdx.x + 1024 * i);
                if constexpr (kVecP) {
                    *reinterpret_cast<u32x4_t*>(&prm[a * pe + min(e, pcount - 8)]) = pv[a][i];
                } else {
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        prm[a * pe + min(e + q, pcount - 1)] = (uint16_t)(pv[a][i][q >> 1] >> (16 * (q & 1)));
                }
            }
        lds_barrier();  // an LDS-only barrier: the weight loads stay in flight
    }
    if constexpr (kDB) {
        // two passes in flight; the loads at the end of each iteration are unconditional (a dead
        // pass past the last one reads clamped blocks and meets zero activations), so the
        // compiler's wait counts stay exact
        for (int ps = 0; ps + 2 < npass; ps += 2) {
            compute(pa);
            load(ps + 2, pa);
            compute(pb);
            load(ps + 3, pb);
        }
        compute(pa);
        compute(pb);
    } else {
        compute(pa);
        for (int ps = 1; ps < npass; ++ps) {
            load(ps, pa);
            compute(pa);
        }
    }

    // 3) partial tiles through LDS: element (row 4g + e of A tile t, column j of row tile r)
#pragma unroll
    for (int r = 0; r < kMyTiles; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) part[slice][16 * (rg + kR * r) + j][16 * t + 4 * g + e] = acc[r][t][e];
    __syncthreads();
    for (int idx = threadIdx.x; idx < kRmRows * 16 * MT; idx += 1024) {
        const int nl = idx / (16 * MT), m = idx % (16 * MT);
        const int n = n0 + nl;
        if (n < N && m < M) {
            float sum = 0.0f;
#pragma unroll
            for (int s = 0; s < kS; ++s) sum += part[s][nl][m];
            if constexpr (kW8) sum *= reinterpret_cast<const float*>(scales)[n];
            y[(size_t)m * N + n] = f32_to_f16_bits(sum);
        }
    }
}

template <int kFmt, int MT, int kR, int UP, int kStage, bool kVecP, bool kDB>
void launch_rm(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales, const uint16_t* zeros,
               int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
    const dim3 grid((unsigned)((N + kRmRows - 1) / kRmRows)), block(1024);
    hipLaunchKernelGGL((rowmma_kernel<kFmt, MT, kR, UP, kStage, kVecP, kDB>), grid, block, 0, stream, x, codes, scales,
                       zeros, y, (int)M, (int)N, (int)K);
}

template <int kFmt, int MT, int kR, int UP, bool kDB>
void launch_rm_stage(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales, const uint16_t* zeros,
                     int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
    // staged parameters per block: 64 rows x K/32 scales (Q4), 64 rows x K/128 scales and zero
    // points (zero-point format), in 16-byte pieces per thread: 1, 2 or 4 of them
    if constexpr (kFmt != kRmW8) {
        const int64_t pb = kFmt == kRmQ4 ? K / 32 : K / 128;
        const int64_t pieces = (64 * pb + 8 * 1024 - 1) / (8 * 1024);
        const bool vec = pb % 8 == 0;
#define W4A16_RM_STAGE(P)                                                                            \
    if (vec)                                                                                         \
        launch_rm<kFmt, MT, kR, UP, P, true, kDB>(x, M, codes, scales, zeros, N, K, y, stream);    \
    else                                                                                             \
        launch_rm<kFmt, MT, kR, UP, P, false, kDB>(x, M, codes, scales, zeros, N, K, y, stream);   \
    return;
        if (pieces <= 1) { W4A16_RM_STAGE(1) }
        if (pieces <= 2) { W4A16_RM_STAGE(2) }
        if constexpr (kFmt == kRmQ4) {
            if (pieces <= 4) { W4A16_RM_STAGE(4) }
        }
#undef W4A16_RM_STAGE
    }
    launch_rm<kFmt, MT, kR, UP, 0, true, kDB>(x, M, codes, scales, zeros, N, K, y, stream);
}

template <int kFmt>
hipError_t launch_rowmma(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                         const uint16_t* zeros, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
    // 16 activation rows per launch, each a pass over the weights (from the 256 MB Infinity Cache
    // after the first, where they fit); one unit per pass of a wave, two in flight
    for (int64_t m0 = 0; m0 < M; m0 += 16) {
        const int64_t Mc = M - m0 < 16 ? M - m0 : 16;
        launch_rm_stage<kFmt, 1, 1, 1, true>(x + m0 * K, Mc, codes, scales, zeros, N, K, y + m0 * N, stream);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_rowmma_q4b32(const uint16_t* x, int64_t M, const uint8_t* codes, const uint16_t* scales, int64_t N,
                               int64_t K, uint16_t* y, hipStream_t stream) {
    return launch_rowmma<kRmQ4>(x, M, reinterpret_cast<const uint32_t*>(codes), scales, nullptr, N, K, y, stream);
}

hipError_t launch_rowmma_g128zp(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                                const uint16_t* zeros, int64_t N, int64_t K, uint16_t* y, hipStream_t stream) {
    return launch_rowmma<kRmZP>(x, M, codes, scales, zeros, N, K, y, stream);
}

hipError_t launch_rowmma_w8row(const uint16_t* x, int64_t M, const int8_t* codes, const float* scales, int64_t N,
                               int64_t K, uint16_t* y, hipStream_t stream) {
    return launch_rowmma<kRmW8>(x, M, reinterpret_cast<const uint32_t*>(codes), reinterpret_cast<const uint16_t*>(scales),
                                nullptr, N, K, y, stream);
}

}  // namespace w4a16
