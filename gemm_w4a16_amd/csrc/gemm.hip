// gemm.hip -- large-M W4A16 GEMM on bf16 MFMA (the compute-bound path).
//
// vidyal.ai "Low-Precision Kernels", Step 2 builds the B tile of a tiled matmul from packed
// integers (shift/mask, then q * scale + min in fp32 rounded to bf16) and feeds it to the
// tensor-core dot with fp32 accumulation; BF16 weights never reach memory.  Here that becomes:
//
//  * block tile BM x BN x 64 (K), 256 threads = 4 waves in a WM x (4/WM) grid; a wave owns
//    (BM/WM) x (BN/(4/WM)) outputs as 32x32 v_mfma_f32_32x32x16_bf16 accumulators (on gfx950
//    this shape runs at twice the rate of 16x16x32).  The tile is chosen so that the grid fills
//    the 256 CUs without splitting K where it can: 256 x 224 (waves stacked along M) at
//    M = 1024, since 14336 = 64 x 224 and 1024 = 4 x 256 give exactly 256 tiles -- a
//    power-of-two N tile would leave 1/8 of the chip idle; 128 x 256 and 128 x 128 (2 x 2 waves)
//    for 512 and 256 rows, and 128 x 64 (waves along M) up to 128 rows, where one M-tile means
//    each weight is dequantized once (224 tiles);
//  * every global read in the k-loop is a direct-to-LDS copy by the load unit (global_load_lds)
//    issued ahead of its use: the A tile one k-tile ahead (two LDS stages, XOR-swizzled rows),
//    the packed B words three k-tiles ahead (three stages) and each group's scales and minimums
//    with its first k-tile.  The copies are issued in an order that lets one `s_waitcnt vmcnt(n)`
//    before each k-tile's barrier wait only for what the next k-tile needs, so no wave waits on
//    HBM latency inside the loop;
//  * while the MFMAs of k-tile t read one dequantized B stage, the threads turn the 8 packed words
//    of each column of k-tile t+1 into the other (one column per thread, or two or four threads
//    per column when BN < 256): w_hat = bf16_rne(fmaf(q, s, min)), the same value as the
//    reference dequant.  Two codes at a time become exact fp32 through the fp8 (e4m3)
//    conversion, in which the bytes 0..15 are exactly the integers times 2^-9: 19 VALU
//    instructions per word, interleaved with the MFMAs.  Each word becomes one 16-byte row
//    segment of an [n][k] tile, which is exactly an MFMA B fragment; rows are padded to 144 B,
//    so fragment reads and dequant writes are free of bank conflicts;
//  * the MFMA steps run one step behind the fragment reads and across the k-tile boundary: the
//    first MFMAs after each barrier use fragments read before it, so no k-tile starts with a
//    wait for LDS.  The copies' sources and LDS stages are kept in scalar cursors advanced
//    once per k-tile (a handful of scalar instructions instead of per-tile address arithmetic,
//    since the scalar unit is shared by the CU's waves);
//  * the output tile leaves through LDS as whole rows (16 bytes per lane, a wave writing 1 KB of
//    consecutive bytes per instruction): with every block finishing at the same moment, one
//    16-byte write request per row and instruction left the epilogue bound by write requests;
//  * when the tile grid alone cannot fill the chip, K is split in whole groups; fp32 partials go
//    to the caller's workspace and a second kernel adds them in split order, so the result does
//    not depend on scheduling.
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "lds_dma.h"

namespace w4a16 {

namespace {

constexpr int BK = 64;
constexpr int LDT = BK + 8;  // dequantized B tile row pitch in bf16 (144 B)
constexpr int kCUs = 256;
// M-tiles per group of the tile order (see the kernel): 2 measured best (M = 512: 68.6 us against
// 70.4 us with 1 and 69.1 us with 4; M = 1024: 100.9-101.1 against 101.4 and 101.3)
constexpr int kMGroup = 2;

// Copy distances: at k-tile t the A tile of t+DA and the packed words of t+DB are requested.
// A then needs DA+1 LDS stages, the packed words DB, the scales/minimums (one stage per group of
// two k-tiles) DB/2 + 1; the dequantized B has two (k-tiles t and t+1).  Short k-tiles (small
// tiles) need longer distances to cover the latency.
template <int BM, int BN, int DA, int DB, int KS>
struct Smem {
    static_assert(DA >= 1 && DB >= DA + 2, "the words of t+2 must be requested before A(t+1)");
    static constexpr int kAS = DA + 1, kBS = DB, kSS = DB / 2 + 1;
    static constexpr int kThr = 256 * KS;
    // 16-byte chunks (vector copies) or dwords (dword copies) of a packed stage, padded to whole
    // rounds of the block's lanes
    static constexpr int kBpChunks = (2 * BN + kThr - 1) / kThr * kThr;
    static constexpr int kBpDwords = (8 * BN + kThr - 1) / kThr * kThr;
    static constexpr int kA = BM * BK * 2;     // A stage: BM rows x 64 bf16
    static constexpr int kBdq = BN * LDT * 2;  // dequantized B stage: BN rows x 144 B
    static constexpr int kBp = (kBpChunks * 16 > kBpDwords * 4 ? kBpChunks * 16 : kBpDwords * 4);  // [8][BN] u32 + pad
    static constexpr int kSc = 512 * 4;        // 256 scale slots + 256 minimum slots, a dword each
    static constexpr int oA = 0;
    static constexpr int oBdq = oA + kAS * kA;
    // written by the threads past column BN-1 when a column has one thread: thread BN + u
    // stores its row segment r at 16 (u + r), so (threads - BN + 7) x 16 B, rounded up
    static constexpr int kSink = BN < kThr && 2 * BN > kThr ? ((kThr - BN + 7) * 16 + 127) / 128 * 128 : 0;
    static constexpr int oSink = oBdq + 2 * kBdq;
    static constexpr int oBp = oSink + kSink;
    static constexpr int oSc = oBp + kBS * kBp;
    static constexpr int kTotal = oSc + kSS * kSc;
};


// A tiles: rows of 64 bf16 (128 B), unpadded; the 16-byte chunk c of row r sits at chunk
// c ^ ((r >> 1) & 7), which keeps the 16 rows of a fragment read on 16 distinct 4-bank groups.
__device__ __forceinline__ int a_swizzle(int r, int c) { return c ^ ((r >> 1) & 7); }

// f(std::integral_constant<int, i>) for i = I .. N-1, so that i can select template arguments.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// The byte offset of the stage after the one at `off`, for n stages of `size` bytes.
template <int size, int n>
__device__ __forceinline__ uint32_t next_stage(uint32_t off) {
    if constexpr (n == 1) {
        return 0;
    } else {
        off += size;
        return off == (uint32_t)(size * n) ? 0u : off;
    }
}

// Instruction interleaving inside one k-step region: MFMAs alternate with the LDS reads of the
// next step's fragments and with the dequant; the first `lead` MFMAs carry no dequant (its words
// are still on their way from LDS).
template <int kMFMA, int kValu>
__device__ __forceinline__ void step_schedule(int lead) {
#pragma unroll
    for (int i = 0; i < kMFMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        if (i >= lead) {
            __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);  // VALU
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);      // DS write
        }
    }
}

template <int BM, int BN, int WM, int DA, int DB, bool kVec, int KS>
struct Gemm {
    // KS groups of 4 waves split each k-tile's four k-steps (KS = 2: two waves per SIMD, so one
    // hides the other's latencies on short k-tiles); each group holds the whole output tile and
    // the groups' sums are added at the end.  Within a group the waves form a WM x WN grid.
    static_assert(KS == 1 || KS == 2, "k groups");
    static constexpr int kThr = 256 * KS, kWaves = 4 * KS, kOwnSteps = (BK / 16) / KS;
    static constexpr int WN = 4 / WM;
    static constexpr int kWRows = BM / WM, kWCols = BN / WN;  // a wave's output tile
    static constexpr int kMT = kWRows / 32, kNT = kWCols / 32;  // its 32 x 32 MFMA tiles
    static_assert(kMT >= 1 && kNT >= 1 && kWRows % 32 == 0 && kWCols % 32 == 0, "wave tile");
    using S = Smem<BM, BN, DA, DB, KS>;
    static constexpr int kAInst = BM / (32 * KS);  // A copies per wave per k-tile (8 rows, 1 KB each)
    static_assert(kAInst >= 1, "A rows per wave");
    static constexpr int kBInst = kVec ? S::kBpChunks / kThr : S::kBpDwords / kThr;  // packed-word copies
    static constexpr int kScInst = 2 / KS;  // scale + minimum copies per wave, when a group starts
    // dequant: kTPC threads per column, each converting kWPT of its 8 packed words per k-tile
    static constexpr int kTPC = 2 * BN <= kThr ? kThr / BN : 1;
    static constexpr int kWPT = 8 / kTPC;
    static_assert(BN <= kThr && (2 * BN > kThr || kThr % BN == 0) && kWPT >= 1, "dequant split");
    static_assert(S::kTotal <= 160 * 1024, "LDS budget");
    // schedule: kMFMA MFMAs per k-step; the first kLead of k-step 0 carry no dequant (its words
    // are still coming from LDS); kVPM VALU slots after each of the others
    static constexpr int kMFMA = kMT * kNT;
    static constexpr int kLead = kMFMA >= 8 ? 2 : 0;
    static constexpr int kValuPerStep = 22 * kWPT / kOwnSteps + 2;
    static constexpr int kVPM = (kValuPerStep + kMFMA - kLead - 1) / (kMFMA - kLead);

    // Copies a wave may still have in flight at the end of k-tile t (parity p) once A(t+1) has
    // landed: the rest of k-tile t+1-DA (its words and scales) and all of k-tiles t+2-DA .. t.
    static constexpr int sc_copies(int u) { return ((u + DB) & 1) == 0 ? kScInst : 0; }  // scales at k-tile u
    static constexpr int after_a(int p) {
        int n = kBInst + sc_copies(p + 1 - DA);
        for (int u = p + 2 - DA; u <= p; ++u) n += kAInst + kBInst + sc_copies(u);
        return n;
    }

    const uint16_t* x;
    const uint32_t* codes;
    const uint16_t* scales;
    const uint16_t* mins;
    uint8_t* smem;
    uint32_t sm;  // LDS address of smem
    int M, N, K, m0, n0, kbeg, ntiles;
    uint32_t mlo;  // 0x0F0F0F0F (a kernel argument, so the compiler keeps it in a register)
    // per-lane byte offsets of the copies (constant over the k-loop)
    uint32_t a_off[kAInst];  // from the k-tile's A base
    uint32_t b_off[kBInst > 0 ? kBInst : 1];  // from the k-tile's first packed row
    uint32_t sc_off[2];      // scale/min dword for even / odd g*N (the same slot in both arrays)
    // this wave's copy destinations in stage 0 (wave-uniform LDS addresses) and the array each
    // of its scale copies reads
    uint32_t a_lds, b_lds, sc_lds[kScInst];
    const char* sc_arr[kScInst];
    // this thread's LDS byte offsets (from smem, without the stage)
    uint32_t a_rd[kMT][kOwnSteps];  // A fragment (i, own k-step j)
    uint32_t b_rd;                  // B fragment of column tile 0, own k-step 0
    uint32_t bq_wr[2];            // dequantized row segment, per destination stage
    uint32_t bp_rd;               // packed word of this thread's first row, this thread's column
    uint32_t sc_rd[2];            // scale of this thread's column, for even / odd g*N

    __device__ __forceinline__ void init() {
        const int lane = lane_id(), wave = wave_id(), tid = threadIdx.x;
        const int l32 = lane & 31, lh = lane >> 5;
        const int w4 = wave % 4, wm = w4 % WM, wn = w4 / WM;
        sm = lds_addr(smem);
        // A copies: instruction i of wave w fills rows w*BM/(4 KS) + 8i .. +7; lane l lands on
        // chunk l % 8 of row l / 8 and so reads the global chunk that the swizzle maps there.
        // Rows past M repeat row M-1; they only feed outputs that are never stored.
#pragma unroll
        for (int i = 0; i < kAInst; ++i) {
            const int r = wave * (BM / kWaves) + 8 * i + (lane >> 3);
            const int gr = min(m0 + r, M - 1) - m0;
            a_off[i] = (uint32_t)(((size_t)gr * K + 8 * a_swizzle(r, lane & 7)) * 2);
        }
        a_lds = sm + S::oA + wave * (BM / kWaves) * BK * 2;
        // Packed words, LDS layout [8 packed rows][BN columns] u32.  Vector copies (N % 4 == 0):
        // 16-byte chunk c = row * BN/4 + column / 4; lanes past the last chunk land in the stage's
        // pad.  Dword copies: dword d = row * BN + column.  Columns past N repeat a valid column.
#pragma unroll
        for (int i = 0; i < kBInst; ++i) {
            const int d = (i * kWaves + wave) * kWave + lane;
            int row, col;
            if (kVec) {
                const int c = min(d, 2 * BN - 1);
                row = c / (BN / 4);
                col = min(n0 + 4 * (c % (BN / 4)), N - 4);
            } else {
                const int dd = min(d, 8 * BN - 1);
                row = dd / BN;
                col = min(n0 + dd % BN, N - 1);
            }
            b_off[i] = (uint32_t)(((size_t)row * N + col) * 4);
        }
        b_lds = sm + S::oBp + wave * (kVec ? 1024 : 256);
        // Scales and minimums: copy i of wave w covers lanes (i*kWaves + w)*64 .. of 512, the first
        // 256 scales, the rest minimums; slot (w % 4)*64 + l receives the aligned dword that holds
        // the bf16 of column min(n0 + min(slot, BN-1), N-1) in the group's row.  Where the dword
        // starts depends on the parity of g*N, so both offsets are kept.
        {
            const int c = min(n0 + min(w4 * kWave + lane, BN - 1), N - 1);
            sc_off[0] = (uint32_t)((2 * c) & ~3);
            sc_off[1] = (uint32_t)((2 + 2 * c) & ~3);
        }
#pragma unroll
        for (int i = 0; i < kScInst; ++i) {
            const int arr = (i * kWaves + wave) / 4;  // 0: scales, 1: minimums (wave-uniform)
            sc_arr[i] = reinterpret_cast<const char*>(arr ? mins : scales);
            sc_lds[i] = sm + S::oSc + w4 * 256 + arr * 1024;
        }
        const int ks0 = (wave / 4) * kOwnSteps;  // this wave's first k-step of each k-tile
#pragma unroll
        for (int i = 0; i < kMT; ++i)
#pragma unroll
            for (int j = 0; j < kOwnSteps; ++j) {
                const int r = wm * kWRows + i * 32 + l32;
                a_rd[i][j] = S::oA + (uint32_t)(r * BK + 8 * a_swizzle(r, 2 * (ks0 + j) + lh)) * 2;
            }
        b_rd = S::oBdq + (uint32_t)((wn * kWCols + l32) * LDT + 8 * lh) * 2 + ks0 * 32;
        // dequant: thread tid converts words h*kWPT .. of column col (one column per thread when
        // BN > 128, the threads past column BN-1 writing to the sink; else kTPC per column)
        const int col = kTPC > 1 ? tid % BN : min(tid, BN - 1);
        const int h = kTPC > 1 ? tid / BN : 0;
#pragma unroll
        for (int st = 0; st < 2; ++st)
            bq_wr[st] = (kTPC > 1 || tid < BN) ? S::oBdq + st * S::kBdq + col * LDT * 2 + h * kWPT * 16
                                               : S::oSink + (tid - BN) * 16;  // (only when BN < threads)
        bp_rd = S::oBp + col * 4 + h * kWPT * BN * 4;
        // the bf16 of column c in group g is the (g*N + c) & 1 half of its slot
        const int c = min(n0 + col, N - 1);
        sc_rd[0] = S::oSc + col * 4 + 2 * (c & 1);
        sc_rd[1] = S::oSc + col * 4 + 2 * ((c + 1) & 1);
    }

    // A copies i0 .. i1-1 of this wave's share of one k-tile: src = the block's first row at the
    // k-tile's first column, stage = the LDS stage's byte offset.
    template <int i0, int i1>
    __device__ __forceinline__ void issue_a(const char* src, uint32_t stage) const {
        const uint32_t lds = a_lds + stage;
        static_for<i0, i1>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            dma16<i * 8 * BK * 2>(a_off[i], src, lds);
        });
    }

    // The packed words of one k-tile: src = its first packed row at column 0.
    __device__ __forceinline__ void issue_b(const char* src, uint32_t stage) const {
        const uint32_t lds = b_lds + stage;
        static_for<0, kBInst>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (kVec)
                dma16<i * kWaves * 1024>(b_off[i], src, lds);
            else
                dma4<i * kWaves * 256>(b_off[i], src, lds);
        });
    }

    // The scales and minimums of one group: rb = 2 g N, the byte offset of row g in either array.
    __device__ __forceinline__ void issue_sc(size_t rb, uint32_t stage) const {
        const uint32_t off = (rb & 2) ? sc_off[1] : sc_off[0];  // (no dynamic index: keeps it in a register)
        const size_t row = rb & ~(size_t)3;
#pragma unroll
        for (int i = 0; i < kScInst; ++i) dma4<0>(off, sc_arr[i] + row, sc_lds[i] + stage);
    }

    // This thread's kWPT packed words (words stage bstage) and the bf16 bits of its column's scale
    // and minimum (scale stage scstage; odd = the parity of g*N for the words' group).
    __device__ __forceinline__ void read_words(uint32_t bstage, uint32_t scstage, bool odd, uint32_t (&w)[kWPT],
                                               uint32_t& sb, uint32_t& mb) const {
        const uint8_t* bp = smem + bp_rd + bstage;
#pragma unroll
        for (int r = 0; r < kWPT; ++r) w[r] = *reinterpret_cast<const uint32_t*>(bp + r * BN * 4);
        const uint8_t* sc = smem + (odd ? sc_rd[1] : sc_rd[0]) + scstage;
        sb = *reinterpret_cast<const uint16_t*>(sc);
        mb = *reinterpret_cast<const uint16_t*>(sc + 1024);
    }

    __device__ __forceinline__ void dequant_all(int st, const uint32_t (&w)[kWPT], uint32_t sb, uint32_t mb) const {
        const float s = bf16_bits_to_f32(sb), m = bf16_bits_to_f32(mb);
        uint8_t* dst = smem + bq_wr[st];
#pragma unroll
        for (int r = 0; r < kWPT; ++r)
            *reinterpret_cast<uint4*>(dst + r * 16) = dequant_word(w[r], mlo, s, m);
    }

    // The LDS reads of the fragments of own k-step ks of a k-tile (A stage at byte offset astage,
    // dequantized B stage st) into register slot `slot`.
    __device__ __forceinline__ void read_frags(uint32_t astage, int st, int ks, bf16x8_t (&af)[kMT],
                                               bf16x8_t (&bfr)[kNT]) const {
#pragma unroll
        for (int i = 0; i < kMT; ++i)
            af[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(smem + astage + a_rd[i][ks]));
#pragma unroll
        for (int j = 0; j < kNT; ++j)
            bfr[j] = __builtin_bit_cast(
                bf16x8_t, *reinterpret_cast<const uint4*>(smem + b_rd + S::kBdq * st + j * 32 * LDT * 2 + ks * 32));
    }

    // One k-tile of MFMA steps, shifted by one step: own step j reads the fragments of step j of
    // this k-tile into register slot j & 1 and runs the MFMAs of the step before it, whose
    // fragments sit in the other slot -- for j = 0, the last step of the previous k-tile, read
    // before the barrier that ended it.  So the first MFMAs after a barrier never wait for LDS.
    // Meanwhile the words `w` (the next k-tile) are dequantized into the other B stage, spread
    // evenly over the steps, and issue(integral_constant j) runs at the top of step j: the
    // copies for later k-tiles are spread over the tile rather than issued in one burst, which
    // would hold up the wave's MFMAs behind the load unit.  The MFMA takes the B fragment as its
    // first operand, so a lane's accumulator holds four adjacent output columns of one row.
    template <int st, typename Issue>
    __device__ __forceinline__ void mma_tile(uint32_t astage, f32x16_t (&acc)[kMT][kNT], bf16x8_t (&af)[2][kMT],
                                             bf16x8_t (&bfr)[2][kNT], const uint32_t (&w)[kWPT], uint32_t sb,
                                             uint32_t mb, Issue&& issue) const {
        uint8_t* dst = smem + bq_wr[st ^ 1];
        float s, m;
        static_for<0, kOwnSteps>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            __builtin_amdgcn_sched_barrier(0);
            issue(jc);
            if constexpr (j == 0) {
                // converted inside the scheduled region, so the wait for them follows the first MFMAs
                s = bf16_bits_to_f32(sb);
                m = bf16_bits_to_f32(mb);
            }
            read_frags(astage, st, j, af[j & 1], bfr[j & 1]);
#pragma unroll
            for (int r = 0; r < kWPT; ++r)
                if (r * kOwnSteps / kWPT == j)
                    *reinterpret_cast<uint4*>(dst + r * 16) = dequant_word(w[r], mlo, s, m);
            mma_step(acc, af[(j + 1) & 1], bfr[(j + 1) & 1]);
            step_schedule<kMFMA, kVPM>(j == 0 ? kLead : 0);
        });
        __builtin_amdgcn_sched_barrier(0);
    }

    __device__ __forceinline__ static void mma_step(f32x16_t (&acc)[kMT][kNT], const bf16x8_t (&af)[kMT],
                                                    const bf16x8_t (&bfr)[kNT]) {
#pragma unroll
        for (int jj = 0; jj < kNT; ++jj)
#pragma unroll
            for (int i = 0; i < kMT; ++i)
                acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[jj], af[i], acc[i][jj], 0, 0, 0);
    }
};

template <int BM, int BN, int WM, int DA, int DB, bool kVec, int KS>
__global__ __launch_bounds__(256 * KS) __attribute__((amdgpu_waves_per_eu(KS, KS)))
void gemm_g128_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ codes,
                      const uint16_t* __restrict__ scales, const uint16_t* __restrict__ mins,
                      uint16_t* __restrict__ y, float* __restrict__ ws, int M, int N, int K, int k_per_split,
                      int splits, uint32_t mask_lo) {
    using G = Gemm<BM, BN, WM, DA, DB, kVec, KS>;
    using S = Smem<BM, BN, DA, DB, KS>;
    constexpr int kMT = G::kMT, kNT = G::kNT, kWPT = G::kWPT;
    __shared__ __attribute__((aligned(16))) uint8_t smem[S::kTotal];
    // XCD-aware tile order: block b runs on XCD b % 8, so XCD x takes the x-th contiguous eighth
    // of the tile sequence.  Within a split the sequence walks groups of kMGroup M-tiles, n-major
    // inside a group, so an XCD's blocks share both their A rows and their packed weights in its
    // own L2 (at M = 1024: 2 M-tiles x 16 column strips per XCD, 11.3 MB of distinct operands,
    // against 16.7 MB for 1 M-tile x 32 strips).
    const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
    const int total = tiles_n * tiles_m * splits;  // gridDim.x == 8 * per_xcd >= total
    const int per_xcd = (int)gridDim.x / 8;
    const int t = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (t >= total) return;
    const int split_id = t / (tiles_n * tiles_m);
    // within a split, tiles run in groups of kMGroup M-tiles, n-major inside a group, m fastest
    const int r = t % (tiles_n * tiles_m);
    const int mg = r / (kMGroup * tiles_n), rr = r % (kMGroup * tiles_n);
    const int gm = min(kMGroup, tiles_m - mg * kMGroup);  // M-tiles in this group
    const int tile_m = mg * kMGroup + rr % gm, tile_n = rr / gm;

    G g;
    g.x = x;
    g.codes = codes;
    g.scales = scales;
    g.mins = mins;
    g.smem = smem;
    g.M = M;
    g.N = N;
    g.K = K;
    g.m0 = tile_m * BM;
    g.n0 = tile_n * BN;
    g.kbeg = split_id * k_per_split;
    g.ntiles = (min(K, g.kbeg + k_per_split) - g.kbeg) / BK;  // even: splits are whole groups
    g.mlo = mask_lo;
    g.init();
    const int ntiles = g.ntiles;
    // the accumulators stay outside `g`: a local array is kept in registers across the copies'
    // inline assembly, whose memory clobber would otherwise force them out to scratch
    f32x16_t acc[kMT][kNT];
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // Copy sources, wave-uniform.  k-tile indices past the end fetch the last k-tile again: the
    // data is never used, and the stage it lands in is one no MFMA or dequant is reading.
    const char* const a_base = reinterpret_cast<const char*>(x + (size_t)g.m0 * K + g.kbeg);
    const uint32_t a_lim = (uint32_t)(ntiles - 1) * BK * 2;
    const size_t b_step = (size_t)8 * N * 4;  // one k-tile of packed rows
    const char* const b_base = reinterpret_cast<const char*>(codes + (size_t)(g.kbeg / 8) * N);
    const int glast = ntiles / 2 - 1;  // the split's last group, counted from its first
    const size_t sc_step = (size_t)2 * N;
    const size_t sc_base = (size_t)(g.kbeg / 128) * sc_step;

    // Prologue: A of k-tiles 0 .. DA-1, the words of 0 .. DB-1 and the scales of their groups;
    // k-tile 0 is then dequantized into B stage 0.
#pragma unroll
    for (int t0 = 0; t0 < DA; ++t0) g.template issue_a<0, G::kAInst>(a_base + min(t0, ntiles - 1) * BK * 2, t0 * S::kA);
#pragma unroll
    for (int t0 = 0; t0 < DB; ++t0) {
        g.issue_b(b_base + (size_t)min(t0, ntiles - 1) * b_step, t0 * S::kBp);
        if (t0 % 2 == 0) g.issue_sc(sc_base + (size_t)min(t0 / 2, glast) * sc_step, (t0 / 2) * S::kSc);
    }
    wait_vm<0>();
    __syncthreads();
    {
        uint32_t w[kWPT], sb, mb;
        g.read_words(0, 0, ((g.kbeg / 128) & N & 1) != 0, w, sb, mb);
        g.dequant_all(0, w, sb, mb);
    }
    __syncthreads();

    // Cursors of the copies still to come (scalar registers, advanced once per k-tile): the A
    // k-tile copied next (byte offset, clamped), the words of k-tile tb and the scales of group gb
    // (pointers, clamped).  Stages as byte offsets: A of k-tile t (a_cur) and of t-1 (a_prev,
    // which is also the stage of t+DA), the words of t (b_cur, also the stage of t+DB), the
    // scales of group p = t/2 (s_cur) and of p-1 (s_prev).
    uint32_t a_o = (uint32_t)min(DA, ntiles - 1) * BK * 2;
    int tb = DB;
    const char* b_src = b_base + (size_t)min(DB, ntiles - 1) * b_step;
    int gb = (DB + 1) / 2;  // the first group whose first k-tile is DB or later
    size_t sc_rb = sc_base + (size_t)min(gb, glast) * sc_step;
    uint32_t a_cur = 0, a_prev = (S::kAS - 1) * S::kA, b_cur = 0, s_cur = 0, s_prev = (S::kSS - 1) * S::kSc;
    const uint32_t nodd = (uint32_t)N & 1;
    uint32_t gpar = (uint32_t)(g.kbeg / 128) & 1;  // parity of group p

    // k-tile t: read the words of t+1; run the MFMAs of t while dequantizing t+1 and copying
    // A(t+DA) (spread over the k-steps) and then the words of t+DB (with their group's scales
    // when t+DB starts a group); then wait until A(t+1) and everything issued before it has
    // landed -- the words of t+2 and their scales were requested no later than A(t+1), since
    // DB >= DA + 2 -- and meet at the barrier.
    constexpr int kSteps = G::kOwnSteps;  // k-steps each wave runs per k-tile
    static_assert(kSteps % 2 == 0, "the last step's fragments sit in slot 1");
    // fragment registers, two slots; slot 1 starts as zeros, so the "previous step" MFMAs of the
    // first k-tile add nothing
    bf16x8_t af[2][kMT], bfr[2][kNT];
#pragma unroll
    for (int i = 0; i < kMT; ++i) af[1][i] = bf16x8_t{};
#pragma unroll
    for (int j = 0; j < kNT; ++j) bfr[1][j] = bf16x8_t{};
    constexpr int kWaitEven = G::after_a(0), kWaitOdd = G::after_a(1);
    auto advance = [&](bool sc_copied) {
        a_o = min(a_o + BK * 2, a_lim);
        ++tb;
        b_src += tb < ntiles ? b_step : 0;
        if (sc_copied) {
            ++gb;
            sc_rb += gb <= glast ? sc_step : 0;
        }
        if constexpr (S::kAS > 2) {
            a_prev = a_cur;
            a_cur = next_stage<S::kA, S::kAS>(a_cur);
        }
    };
    for (int tt = 0; tt < ntiles; tt += 2) {
        {
            const uint32_t b_next = next_stage<S::kBp, S::kBS>(b_cur);
            const uint32_t a_rd = S::kAS == 2 ? 0 : a_cur, a_wr = S::kAS == 2 ? S::kA : a_prev;
            uint32_t w[kWPT], sb, mb;
            g.read_words(b_next, s_cur, (gpar & nodd) != 0, w, sb, mb);
            const char* a_src = a_base + a_o;
            g.template mma_tile<0>(a_rd, acc, af, bfr, w, sb, mb, [&](auto ksc) {
                constexpr int ks = decltype(ksc)::value;
                static_for<0, G::kAInst>([&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    if constexpr (i * kSteps / G::kAInst == ks) g.template issue_a<i, i + 1>(a_src, a_wr);
                });
                if constexpr (ks == kSteps - 1) {
                    g.issue_b(b_src, b_cur);
                    if constexpr (DB % 2 == 0) g.issue_sc(sc_rb, s_prev);
                }
            });
            advance(DB % 2 == 0);
            b_cur = b_next;
            wait_vm<kWaitEven>();
            __syncthreads();
        }
        {
            const uint32_t b_next = next_stage<S::kBp, S::kBS>(b_cur);
            const uint32_t a_rd = S::kAS == 2 ? S::kA : a_cur, a_wr = S::kAS == 2 ? 0 : a_prev;
            const uint32_t s_next = next_stage<S::kSc, S::kSS>(s_cur);
            uint32_t w[kWPT], sb, mb;
            g.read_words(b_next, s_next, ((gpar ^ 1) & nodd) != 0, w, sb, mb);
            const char* a_src = a_base + a_o;
            g.template mma_tile<1>(a_rd, acc, af, bfr, w, sb, mb, [&](auto ksc) {
                constexpr int ks = decltype(ksc)::value;
                static_for<0, G::kAInst>([&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    if constexpr (i * kSteps / G::kAInst == ks) g.template issue_a<i, i + 1>(a_src, a_wr);
                });
                if constexpr (ks == kSteps - 1) {
                    g.issue_b(b_src, b_cur);
                    if constexpr (DB % 2 == 1) g.issue_sc(sc_rb, s_cur);
                }
            });
            advance(DB % 2 == 1);
            b_cur = b_next;
            s_prev = s_cur;
            s_cur = s_next;
            gpar ^= 1;
            wait_vm<kWaitOdd>();
            __syncthreads();
        }
    }
    G::mma_step(acc, af[1], bfr[1]);  // the last step of the last k-tile
    wait_vm<0>();  // no copy may still be writing this block's LDS when it exits

    // D fragment of the MFMA of B tile jj and A tile i: element e of lane l is output row l % 32
    // of A tile i and column 8 (e / 4) + 4 (l / 32) + e % 4 of B tile jj -- four adjacent columns
    // for each q = e / 4.
    const int lane = lane_id(), wave = wave_id();
    const int l32 = lane & 31, lh = lane >> 5;
    const int w4 = wave % 4, wm = w4 % WM, wn = w4 / WM;
    const int row0 = wm * G::kWRows + l32;     // + 32 i
    const int col0 = wn * G::kWCols + 4 * lh;  // + 32 jj + 8 q
    if constexpr (KS == 2) {
        // the second k group hands its sums to the first through LDS (all copies have landed:
        // every wave waited for its own above, and the barrier covers the others'); rows are
        // padded by 16 B so the 16-byte writes and reads of a wave are free of bank conflicts
        constexpr int kPitch = BN + 4;
        static_assert(BM * kPitch * 4 <= S::kTotal, "partials fit in LDS");
        float* part = reinterpret_cast<float*>(smem);
        __syncthreads();
        if (wave >= 4) {
#pragma unroll
            for (int i = 0; i < kMT; ++i)
#pragma unroll
                for (int j = 0; j < kNT; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x4_t v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                           acc[i][j][4 * q + 3]};
                        *reinterpret_cast<f32x4_t*>(part + (row0 + 32 * i) * kPitch + col0 + 32 * j + 8 * q) = v;
                    }
        }
        __syncthreads();
        if (wave < 4) {
#pragma unroll
            for (int i = 0; i < kMT; ++i)
#pragma unroll
                for (int j = 0; j < kNT; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(part + (row0 + 32 * i) * kPitch + col0 +
                                                                             32 * j + 8 * q);
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[i][j][4 * q + r] += v[r];
                    }
        }
    }
    const bool split = splits > 1;
    if (kVec && !split && N % 8 == 0) {
        // bf16 output through LDS: the first k group writes its tile as rows of bf16 (8 bytes per
        // lane and q), then every thread stores whole 16-byte chunks of rows, so a wave writes
        // 1 KB of consecutive row bytes per instruction -- full cache lines instead of one 16-byte
        // piece per row and instruction, which left the write path, not the kernel, the limit.
        // Rows are padded by 16 B to spread the banks.  The stores are non-temporal: the output is
        // not read again by this kernel, and lines left dirty in L2 are written back at its end.
        constexpr int kOP = 2 * BN + 16;  // staged row pitch, bytes
        static_assert(BM * kOP <= S::kTotal, "staged output fits in LDS");
        constexpr int kChunks = BN / 8;   // 16-byte chunks per row
        __syncthreads();  // (KS = 2: the second group has read its partials back)
        if (KS == 1 || wave < 4) {
#pragma unroll
            for (int i = 0; i < kMT; ++i)
#pragma unroll
                for (int j = 0; j < kNT; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<uint2*>(smem + (row0 + 32 * i) * kOP + (col0 + 32 * j + 8 * q) * 2) =
                            make_uint2(pack2_bf16(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                                       pack2_bf16(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
        }
        __syncthreads();
        for (int c = threadIdx.x; c < BM * kChunks; c += G::kThr) {
            const int r = c / kChunks, cc = c % kChunks;
            const int row = g.m0 + r, col = g.n0 + 8 * cc;
            if (row < M && col < N)
                __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(smem + r * kOP + cc * 16),
                                            reinterpret_cast<u32x4_t*>(y + (size_t)row * N + col));
        }
        return;
    }
    if (KS == 2 && wave >= 4) return;
    // Direct stores: with N % 4 == 0 each lane writes its four adjacent outputs at once (8 bytes
    // of bf16, or 16 of fp32 partials), unchecked when the whole tile lies inside the output.
    const bool interior = g.m0 + BM <= M && g.n0 + BN <= N;
#pragma unroll
    for (int i = 0; i < kMT; ++i) {
        const int row = g.m0 + row0 + 32 * i;
        const int col = g.n0 + col0;
        uint16_t* yr = y + (size_t)min(row, M - 1) * N + col;
        float* wr = ws + ((size_t)split_id * M + min(row, M - 1)) * N + col;
#pragma unroll
        for (int j = 0; j < kNT; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = 32 * j + 8 * q;
                const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1];
                const float v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
                if constexpr (kVec) {
                    if (interior || (row < M && col + c < N)) {
                        if (split)
                            *reinterpret_cast<f32x4_t*>(wr + c) = f32x4_t{v0, v1, v2, v3};
                        else
                            *reinterpret_cast<uint2*>(yr + c) = make_uint2(pack2_bf16(v0, v1), pack2_bf16(v2, v3));
                    }
                } else {
                    const float v[4] = {v0, v1, v2, v3};
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (row < M && col + c + r < N) {
                            if (split)
                                wr[c + r] = v[r];
                            else
                                yr[c + r] = f32_to_bf16_bits(v[r]);
                        }
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

// Tile shapes by M (see the header comment): each fills the 256 CUs at N = 14336 without a K
// split, from 65..128 rows (128 x 64 tiles, waves along M: each weight dequantized once) to 1024
// rows (256 x 224, waves along M).
enum TileCfg { kT128x64, kT128x128, kT128x256, kT256x224 };

struct GemmPlan {
    TileCfg cfg;
    int bm, bn, tiles_m, tiles_n, splits, k_per_split;
};

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K) {
    GemmPlan p;
    if (M <= 128) p.cfg = kT128x64, p.bm = 128, p.bn = 64;
    else if (M <= 256) p.cfg = kT128x128, p.bm = 128, p.bn = 128;
    else if (M <= 512) p.cfg = kT128x256, p.bm = 128, p.bn = 256;
    else p.cfg = kT256x224, p.bm = 256, p.bn = 224;
    p.tiles_m = (int)((M + p.bm - 1) / p.bm);
    p.tiles_n = (int)((N + p.bn - 1) / p.bn);
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    const int groups = (int)(K / 128);
    // split K only when the tiles would leave more than half the CUs idle, into as many splits as
    // still fit one wave of blocks (rounding up left a partial second wave: at N = 4096,
    // K = 14336, M = 1024, 76 tiles x 4 splits took 183.8 us against 128.5 us for x 3)
    int splits = 1;
    if (2 * tiles <= kCUs) splits = (int)std::min<int64_t>(groups, kCUs / tiles);
    // k per split in whole groups; recompute the split count so no split is empty
    const int groups_per_split = (groups + splits - 1) / splits;
    p.k_per_split = groups_per_split * 128;
    p.splits = (groups + groups_per_split - 1) / groups_per_split;
    return p;
}

template <int BM, int BN, int WM, int DA, int DB, int KS>
void launch_cfg(const GemmPlan& p, const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                const uint16_t* mins, int64_t N, int64_t K, uint16_t* y, float* workspace, hipStream_t stream) {
    // a 1-D grid of 8 x ceil(tiles / 8) blocks over (split, m, n); the surplus exit at once
    const int64_t tiles = (int64_t)p.tiles_n * p.tiles_m * p.splits;
    const dim3 grid((unsigned)(8 * ((tiles + 7) / 8)));
    if (N % 4 == 0)
        hipLaunchKernelGGL((gemm_g128_kernel<BM, BN, WM, DA, DB, true, KS>), grid, dim3(256 * KS), 0, stream, x, codes, scales,
                           mins, y, workspace, (int)M, (int)N, (int)K, p.k_per_split, p.splits, 0x0F0F0F0Fu);
    else
        hipLaunchKernelGGL((gemm_g128_kernel<BM, BN, WM, DA, DB, false, KS>), grid, dim3(256 * KS), 0, stream, x, codes, scales,
                           mins, y, workspace, (int)M, (int)N, (int)K, p.k_per_split, p.splits, 0x0F0F0F0Fu);
}

}  // namespace

size_t gemm_g128_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (M <= kMidMaxRows) return 0;
    const GemmPlan p = plan_gemm(M, N, K);
    return p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemm_g128(const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                            const uint16_t* mins, int64_t N, int64_t K, uint16_t* y, float* workspace,
                            hipStream_t stream) {
    if (M <= kMidMaxRows) return launch_mid_g128(x, M, codes, scales, mins, N, K, y, stream);
    const GemmPlan p = plan_gemm(M, N, K);
    switch (p.cfg) {
        case kT128x64: launch_cfg<128, 64, 4, 3, 6, 1>(p, x, M, codes, scales, mins, N, K, y, workspace, stream); break;
        case kT128x128: launch_cfg<128, 128, 2, 2, 5, 2>(p, x, M, codes, scales, mins, N, K, y, workspace, stream); break;
        case kT128x256: launch_cfg<128, 256, 2, 1, 4, 1>(p, x, M, codes, scales, mins, N, K, y, workspace, stream); break;
        case kT256x224: launch_cfg<256, 224, 4, 1, 3, 1>(p, x, M, codes, scales, mins, N, K, y, workspace, stream); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    return launch_splitk_reduce(workspace, M * N, p.splits, y, stream);
}

hipError_t launch_splitk_reduce(const float* ws, int64_t MN, int splits, uint16_t* y, hipStream_t stream) {
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, stream, ws, y, MN, splits);
    return hipGetLastError();
}

}  // namespace w4a16
