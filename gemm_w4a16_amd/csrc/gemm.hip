// gemm.hip -- large-M W4A16 GEMM on bf16 MFMA (the compute-bound path).
//
// vidyal.ai "Low-Precision Kernels", Step 2 builds the B tile of a tiled matmul from packed
// integers (shift/mask, then q * scale + min in fp32 rounded to bf16) and feeds it to the
// tensor-core dot with fp32 accumulation; BF16 weights never reach memory.  Here that becomes:
//
//  * block tile BM x 224 (N) x 64 (K).  N = 224 = 7 x 32 so that the Llama up-projection width
//    14336 = 64 x 224 splits into exactly 64 column tiles and M = 1024 into 4 x 256: 256 blocks
//    for the 256 CUs (a power-of-two N tile would leave 1/8 of the chip idle);
//  * 256 threads = 4 waves stacked along M; a wave owns (BM/4) x 224 outputs as (BM/128) x 7
//    v_mfma_f32_32x32x16_bf16 accumulators (on gfx950 this shape runs at twice the rate of
//    16x16x32 -- measured ~2.4 vs ~1.3 PFLOP/s over the whole chip);
//  * LDS double buffer: while the MFMAs of k-tile t run from one buffer, the load unit copies the
//    A tile of t+1 straight into the other buffer (global_load_lds_dwordx4, XOR-swizzled rows)
//    and the threads hold the packed B words of t+1 in registers, dequantizing them into the
//    other buffer after their MFMAs; one barrier per k-tile;
//  * the packed B tile (8 packed rows x 224 columns) is dequantized by threads 0..223, one column
//    each: w_hat = bf16_rne(fmaf(q, s, min)) -- the same value as the reference dequant -- and
//    each 32-bit word becomes one 16-byte row segment of an [n][k] LDS tile, which is exactly an
//    MFMA B fragment; LDS rows are padded to 144 B so fragment reads are conflict-free;
//  * when the tile grid alone cannot fill the chip, K is split in whole groups; fp32 partials go
//    to the caller's workspace and a second kernel adds them in split order, so the result does
//    not depend on scheduling.
#include "device_common.h"
#include "launch.h"

namespace w4a16 {

namespace {

constexpr int BN = 224, BK = 64;
constexpr int LDT = BK + 8;  // B tile LDS row pitch in bf16 (144 B)
constexpr int kThreads = 256;
constexpr int kCUs = 256;
constexpr int kNT = BN / 32;  // 32-column MFMA tiles per wave (each wave spans all 224 columns)

// A tiles are copied global -> LDS by the load unit (global_load_lds_dwordx4), rows of 64 bf16
// (128 B) unpadded; the 16-byte chunk c of row r sits at chunk c ^ ((r >> 1) & 7), which keeps
// the 16 rows of a fragment read on 16 distinct 4-bank groups.
__device__ __forceinline__ int a_swizzle(int r, int c) { return c ^ ((r >> 1) & 7); }

// B rows 224..255 are scratch: threads 224..255 dequantize a duplicate column into them, which
// keeps the k-loop free of branches.
constexpr int kBRows = kThreads;

// Direct-to-LDS copies of the A tile (rows m0.., k0..k0+63) into `As`: wave w copies rows
// [w * BM/4, (w+1) * BM/4), 8 rows (1 KB) per instruction; lane l lands on chunk l % 8 of row
// l / 8 and so fetches the global chunk that the swizzle maps there.  Rows past M repeat row
// M-1: they only feed output rows that are never stored.  The per-lane byte offsets from x do
// not depend on k0 and are computed once; the k0 part is a wave-uniform base.
template <int BM>
struct ACopy {
    uint32_t off[BM / 32];
    __device__ __forceinline__ void init(int M, int K, int m0) {
        const int lane = lane_id(), wave = wave_id();
#pragma unroll
        for (int i = 0; i < BM / 32; ++i) {
            const int r = wave * (BM / 4) + 8 * i + (lane >> 3);
            const int gm = min(m0 + r, M - 1);
            off[i] = (uint32_t)(((size_t)gm * K + 8 * a_swizzle(r, lane & 7)) * 2);
        }
    }
    __device__ __forceinline__ void issue(const uint16_t* __restrict__ x, uint16_t* As, int k0) const {
        const int wave = wave_id();
        const char* base = reinterpret_cast<const char*>(x + k0);
#pragma unroll
        for (int i = 0; i < BM / 32; ++i)
            __builtin_amdgcn_global_load_lds(base + off[i], As + (wave * (BM / 4) + 8 * i) * BK, 16, 0, 0);
    }
};

// B: thread t < 224 owns column n0 + t of the tile: the 8 packed words of the k-tile.  `off` is
// the column's byte offset; each packed row start is wave-uniform.
__device__ __forceinline__ void load_b(uint32_t (&w)[BK / 8], const uint32_t* __restrict__ codes, int N, uint32_t off,
                                       int k0) {
#pragma unroll
    for (int r = 0; r < BK / 8; ++r) {
        const char* row = reinterpret_cast<const char*>(codes + (size_t)(k0 / 8 + r) * N);
        w[r] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(row + off));
    }
}

// w_hat = bf16_rne(fmaf(q, s, min)) for 8 k of this thread's column (packed row r of the tile),
// as one 16-byte row segment of the [n][k] tile (threads past column 223 write their duplicate
// into the scratch rows).
__device__ __forceinline__ void dequant_word(uint32_t w, int r, uint16_t* Bs, float s, float m) {
    const int t = threadIdx.x;
    {
        const uint32_t ev = w & 0x0F0F0F0Fu, od = (w >> 4) & 0x0F0F0F0Fu;  // q0 q2 q4 q6 / q1 q3 q5 q7
        const float v0 = __builtin_fmaf((float)(ev & 0xFF), s, m);
        const float v2 = __builtin_fmaf((float)((ev >> 8) & 0xFF), s, m);
        const float v4 = __builtin_fmaf((float)((ev >> 16) & 0xFF), s, m);
        const float v6 = __builtin_fmaf((float)(ev >> 24), s, m);
        const float v1 = __builtin_fmaf((float)(od & 0xFF), s, m);
        const float v3 = __builtin_fmaf((float)((od >> 8) & 0xFF), s, m);
        const float v5 = __builtin_fmaf((float)((od >> 16) & 0xFF), s, m);
        const float v7 = __builtin_fmaf((float)(od >> 24), s, m);
        *reinterpret_cast<uint4*>(Bs + t * LDT + r * 8) =
            make_uint4(pack2_bf16(v0, v1), pack2_bf16(v2, v3), pack2_bf16(v4, v5), pack2_bf16(v6, v7));
    }
}

__device__ __forceinline__ void dequant_b(const uint32_t (&w)[BK / 8], uint16_t* Bs, float s, float m) {
#pragma unroll
    for (int r = 0; r < BK / 8; ++r) dequant_word(w[r], r, Bs, s, m);
}

// Instruction interleaving inside one k-step region: each MFMA is followed by one LDS read (the
// next step's fragments) and a few VALU instructions (the dequant), so neither waits in a clump.
#ifndef W4A16_GEMM_VALU_PER_MFMA
#define W4A16_GEMM_VALU_PER_MFMA 3
#endif
template <int kMT>
__device__ __forceinline__ void gemm_step_schedule() {
#ifndef W4A16_GEMM_NO_SCHEDULE
#pragma unroll
    for (int i = 0; i < kMT * (BN / 32); ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x002, W4A16_GEMM_VALU_PER_MFMA, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
    }
#endif
}

__device__ __forceinline__ void wait_vm_all() {
    // s_waitcnt vmcnt(0): the direct-to-LDS copies of this wave have landed
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

// One k-tile: MFMAs on (As, Bs) while the next tile is prepared in (As_n, Bs_n) -- A by the
// load unit (issued here), B by dequantizing the words `wb` fetched one iteration earlier -- and
// the words of the tile after are requested into `wn`.  The four LDS buffers are distinct
// objects, so the compiler can see that the direct-to-LDS copy into As_n does not touch Bs_n or
// As and only the barrier at the end waits for it.
template <int BM>
struct KTile {
    static constexpr int kMT = BM / 128;  // 32-row MFMA tiles per wave (a wave owns BM/4 rows)
    f32x16_t acc[kMT][kNT];
    // two sets of B words (and their raw bf16 scale / min) used alternately: one being
    // dequantized, the other being fetched
    uint32_t w0[BK / 8], w1[BK / 8];
    uint32_t sb0, mb0, sb1, mb1;
    ACopy<BM> acopy;
    uint32_t boff;
    int bcol;

    __device__ __forceinline__ void run(const uint16_t* __restrict__ x, const uint32_t* __restrict__ codes,
                                        const uint16_t* __restrict__ scales, const uint16_t* __restrict__ mins,
                                        int N, int kn, int kn2, const uint16_t* As, const uint16_t* Bs, uint16_t* As_n,
                                        uint16_t* Bs_n, const uint32_t (&wb)[BK / 8], uint32_t sb, uint32_t mb,
                                        uint32_t (&wn)[BK / 8], uint32_t& sbn, uint32_t& mbn) {
        const int lane = lane_id(), wave = wave_id();
        const int l32 = lane & 31, lh = lane >> 5;
        load_b(wn, codes, N, boff, kn2);
        sbn = scales[(size_t)(kn2 / 128) * N + bcol];
        mbn = mins[(size_t)(kn2 / 128) * N + bcol];
        acopy.issue(x, As_n, kn);
        const float s = bf16_bits_to_f32(sb), m = bf16_bits_to_f32(mb);
        // v_mfma_f32_32x32x16_bf16: lane holds A[row l%32][k 8*(l/32)..+7] and B[k same][col l%32].
        // Fragments are double-buffered in registers: the reads for k-step ks+1 are issued in the
        // scheduling region of k-step ks, so no MFMA waits on an LDS read.
        bf16x8_t af[2][kMT], bfr[2][kNT];
        auto read_frags = [&](int ks, int slot) {
#pragma unroll
            for (int i = 0; i < kMT; ++i) {
                const int r = wave * (BM / 4) + i * 32 + l32;
                af[slot][i] = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const uint4*>(As + r * BK + 8 * a_swizzle(r, 2 * ks + lh)));
            }
#pragma unroll
            for (int j = 0; j < kNT; ++j)
                bfr[slot][j] = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const uint4*>(Bs + (j * 32 + l32) * LDT + 16 * ks + 8 * lh));
        };
        // One scheduling region per k-step (sched_barrier): the fragment reads of step ks+1, a
        // quarter of the next B tile's dequant and the 7 * kMT independent MFMAs of step ks.
        read_frags(0, 0);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            __builtin_amdgcn_sched_barrier(0);
            if (ks + 1 < BK / 16) read_frags(ks + 1, (ks + 1) & 1);
#pragma unroll
            for (int r = 2 * ks; r < 2 * ks + 2; ++r) dequant_word(wb[r], r, Bs_n, s, m);
#pragma unroll
            for (int j = 0; j < kNT; ++j)
#pragma unroll
                for (int i = 0; i < kMT; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][i], bfr[ks & 1][j], acc[i][j], 0,
                                                                        0, 0);
            gemm_step_schedule<kMT>();
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_all();
        __syncthreads();
    }
};

template <int BM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_g128_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ codes,
                      const uint16_t* __restrict__ scales, const uint16_t* __restrict__ mins,
                      uint16_t* __restrict__ y, float* __restrict__ ws, int M, int N, int K, int k_per_split,
                      int splits) {
    constexpr int kMT = KTile<BM>::kMT;
    __shared__ __attribute__((aligned(16))) uint16_t sa0[BM * BK], sa1[BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t sb0[kBRows * LDT], sb1[kBRows * LDT];
    // XCD-aware tile order: block b runs on XCD b % 8, so XCD x takes the x-th contiguous eighth
    // of the (split, m, n) tile sequence, n fastest -- its blocks share A rows in its own L2.
    const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
    const int total = tiles_n * tiles_m * splits;  // gridDim.x == 8 * per_xcd >= total
    const int per_xcd = (int)gridDim.x / 8;
    const int t = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (t >= total) return;
    const int split_id = t / (tiles_n * tiles_m);
    const int m0 = (t / tiles_n % tiles_m) * BM, n0 = (t % tiles_n) * BN;
    const int kbeg = split_id * k_per_split;
    const int kend = min(K, kbeg + k_per_split);  // kend - kbeg: a multiple of 128 = 2 k-tiles
    const int lane = lane_id(), wave = wave_id();
    const int l32 = lane & 31, lh = lane >> 5;

    KTile<BM> kt;
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) kt.acc[i][j][e] = 0.0f;
    // B column of this thread; threads >= 224 and columns past N repeat a valid column, never store
    kt.bcol = min(n0 + min((int)threadIdx.x, BN - 1), N - 1);
    kt.boff = (uint32_t)kt.bcol * 4u;
    kt.acopy.init(M, K, m0);

    // prologue: tile kbeg into (sa0, sb0); the words of kbeg+64 into w0
    kt.acopy.issue(x, sa0, kbeg);
    load_b(kt.w0, codes, N, kt.boff, kbeg);
    dequant_b(kt.w0, sb0, bf16_bits_to_f32(scales[(size_t)(kbeg / 128) * N + kt.bcol]),
              bf16_bits_to_f32(mins[(size_t)(kbeg / 128) * N + kt.bcol]));
    load_b(kt.w0, codes, N, kt.boff, kbeg + BK);
    kt.sb0 = scales[(size_t)(kbeg / 128) * N + kt.bcol];  // kbeg + 64 is in the same group
    kt.mb0 = mins[(size_t)(kbeg / 128) * N + kt.bcol];
    wait_vm_all();
    __syncthreads();

    // two k-tiles per trip so every buffer and register set is fixed; the last trip's look-ahead
    // loads are clamped to the last tile and their results unused
    for (int k0 = kbeg; k0 < kend; k0 += 2 * BK) {
        kt.run(x, codes, scales, mins, N, min(k0 + BK, kend - BK), min(k0 + 2 * BK, kend - BK), sa0, sb0, sa1, sb1,
               kt.w0, kt.sb0, kt.mb0, kt.w1, kt.sb1, kt.mb1);
        kt.run(x, codes, scales, mins, N, min(k0 + 2 * BK, kend - BK), min(k0 + 3 * BK, kend - BK), sa1, sb1, sa0,
               sb0, kt.w1, kt.sb1, kt.mb1, kt.w0, kt.sb0, kt.mb0);
    }

    // D fragment of a 32 x 32 tile: element e of lane l is row 8*(e/4) + 4*(l/32) + e%4, column l%32.
    const bool split = splits > 1;
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
            const int col = n0 + j * 32 + l32;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + wave * (BM / 4) + i * 32 + 8 * (e / 4) + 4 * lh + (e % 4);
                if (row < M && col < N) {
                    if (split)
                        ws[((size_t)split_id * M + row) * N + col] = kt.acc[i][j][e];
                    else
                        y[(size_t)row * N + col] = f32_to_bf16_bits(kt.acc[i][j][e]);
                }
            }
        }
}

// y = bf16(sum over splits, in split order) of the fp32 partials.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, uint16_t* __restrict__ y,
                                                            int64_t MN, int splits) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= MN) return;
    float s = ws[i];
    for (int z = 1; z < splits; ++z) s += ws[(size_t)z * MN + i];
    y[i] = f32_to_bf16_bits(s);
}

struct Plan {
    int bm, tiles_m, tiles_n, splits, k_per_split;
};

Plan plan_gemm(int64_t M, int64_t N, int64_t K) {
    Plan p;
    p.bm = M > 128 ? 256 : 128;  // 128: a wave owns one 32-row tile
    p.tiles_m = (int)((M + p.bm - 1) / p.bm);
    p.tiles_n = (int)((N + BN - 1) / BN);
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    const int groups = (int)(K / 128);
    int splits = 1;
    if (tiles < kCUs) splits = (int)std::min<int64_t>(groups, (kCUs + tiles - 1) / tiles);
    // k per split in whole groups; recompute the split count so no split is empty
    const int groups_per_split = (groups + splits - 1) / splits;
    p.k_per_split = groups_per_split * 128;
    p.splits = (groups + groups_per_split - 1) / groups_per_split;
    return p;
}

template <int BM>
void launch_bm(const Plan& p, const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
               const uint16_t* mins, int64_t N, int64_t K, uint16_t* y, float* workspace, hipStream_t stream) {
    // a 1-D grid of 8 x ceil(tiles / 8) blocks over (split, m, n); the surplus exit at once
    const int64_t tiles = (int64_t)p.tiles_n * p.tiles_m * p.splits;
    const dim3 grid((unsigned)(8 * ((tiles + 7) / 8)));
    hipLaunchKernelGGL((gemm_g128_kernel<BM>), grid, dim3(kThreads), 0, stream, x, codes, scales, mins, y, workspace,
                       (int)M, (int)N, (int)K, p.k_per_split, p.splits);
}

}  // namespace

size_t gemm_g128_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const Plan p = plan_gemm(M, N, K);
    return p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemm_g128(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                            const uint16_t* mins, int64_t N, int64_t K, uint16_t* y, float* workspace,
                            hipStream_t stream) {
    const Plan p = plan_gemm(M, N, K);
    if (p.bm == 256)
        launch_bm<256>(p, x, M, codes, scales, mins, N, K, y, workspace, stream);
    else
        launch_bm<128>(p, x, M, codes, scales, mins, N, K, y, workspace, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    const int64_t MN = M * N;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, stream, workspace, y,
                       MN, p.splits);
    return hipGetLastError();
}

}  // namespace w4a16
