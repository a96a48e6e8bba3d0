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
//    power-of-two N tile would leave 1/8 of the chip idle; 128 x 256, 128 x 128 and 64 x 128
//    (2 x 2 waves) for 512, 256 and 128 rows (224 tiles);
//  * every global read in the k-loop is a direct-to-LDS copy by the load unit (global_load_lds)
//    issued ahead of its use: the A tile one k-tile ahead (two LDS stages, XOR-swizzled rows),
//    the packed B words three k-tiles ahead (three stages) and each group's scales and minimums
//    with its first k-tile.  The copies are issued in an order that lets one `s_waitcnt vmcnt(n)`
//    before each k-tile's barrier wait only for what the next k-tile needs, so no wave waits on
//    HBM latency inside the loop;
//  * while the MFMAs of k-tile t read one dequantized B stage, the threads turn the 8 packed words
//    of each column of k-tile t+1 into the other (one column per thread, or two or four threads
//    per column when BN < 256): w_hat = bf16_rne(fmaf(q, s, min)), the
//    same value as the reference dequant, 22 VALU instructions per word, interleaved with the
//    MFMAs (about four VALU instructions fit under one 32x32x16 MFMA).  Each word becomes one
//    16-byte row segment of an [n][k] tile, which is exactly an MFMA B fragment; rows are padded
//    to 144 B, so fragment reads and dequant writes are free of bank conflicts;
//  * when the tile grid alone cannot fill the chip, K is split in whole groups; fp32 partials go
//    to the caller's workspace and a second kernel adds them in split order, so the result does
//    not depend on scheduling.
#include "device_common.h"
#include "launch.h"

namespace w4a16 {

namespace {

constexpr int BK = 64;
constexpr int LDT = BK + 8;  // dequantized B tile row pitch in bf16 (144 B)
constexpr int kThreads = 256;
constexpr int kCUs = 256;

// Copy distances: at k-tile t the A tile of t+DA and the packed words of t+DB are requested.
// A then needs DA+1 LDS stages, the packed words DB, the scales/minimums (one stage per group of
// two k-tiles) DB/2 + 1; the dequantized B has two (k-tiles t and t+1).  Short k-tiles (small
// tiles) need longer distances to cover the latency.
template <int BM, int BN, int DA, int DB>
struct Smem {
    static_assert(DA >= 1 && DB >= DA + 2, "the words of t+2 must be requested before A(t+1)");
    static constexpr int kAS = DA + 1, kBS = DB, kSS = DB / 2 + 1;
    static constexpr int kBpChunks = (2 * BN + 255) / 256 * 256;  // 16-byte chunks of a packed stage
    static constexpr int kA = BM * BK * 2;     // A stage: BM rows x 64 bf16
    static constexpr int kBdq = BN * LDT * 2;  // dequantized B stage: BN rows x 144 B
    static constexpr int kBp = kBpChunks * 16;  // packed stage: [8 packed rows][BN columns] u32 + pad
    static constexpr int kSc = 512 * 4;        // 256 scale slots + 256 minimum slots, a dword each
    static constexpr int oA = 0;
    static constexpr int oBdq = oA + kAS * kA;
    // written by the threads past column BN-1 when a column has one thread: thread BN + u
    // stores its row segment r at 16 (u + r), so (256 - BN + 7) x 16 B, rounded up
    static constexpr int kSink = BN < 256 && BN > 128 ? ((256 - BN + 7) * 16 + 127) / 128 * 128 : 0;
    static constexpr int oSink = oBdq + 2 * kBdq;
    static constexpr int oBp = oSink + kSink;
    static constexpr int oSc = oBp + kBS * kBp;
    static constexpr int kTotal = oSc + kSS * kSc;
};


// A tiles: rows of 64 bf16 (128 B), unpadded; the 16-byte chunk c of row r sits at chunk
// c ^ ((r >> 1) & 7), which keeps the 16 rows of a fragment read on 16 distinct 4-bank groups.
__device__ __forceinline__ int a_swizzle(int r, int c) { return c ^ ((r >> 1) & 7); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Direct-to-LDS copies: lane l reads 16 (or 4) bytes at sbase + voff and the load unit writes
// them to LDS byte m0 + 16 l (or 4 l).  They are issued from inline assembly so that the
// compiler does not track them: the compiler cannot tell the LDS stages apart and would wait for
// every copy in flight before any LDS access.  The only waits for them are the explicit ones
// before the k-tile barriers.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(uint32_t voff, const void* sbase, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(n): at most n of this wave's copies are still in flight.
template <int n>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | 0x0F70 /* expcnt, lgkmcnt: no wait */);
}

// One dequantized word: 8 k of one column -> 16 bytes of bf16, w_hat = bf16_rne(fmaf(q, s, m)).
// Codes 0, 2, 4, 6 come from w & 0x0F0F0F0F and codes 1, 3, 5, 7 from w & 0xF0F0F0F0 as 16 q,
// multiplied by s/16: the product is the same exact value, so the fma rounds identically.  The
// masks arrive as kernel arguments so that each byte converts with one v_cvt_f32_ubyteN.
__device__ __forceinline__ uint4 dequant_word(uint32_t w, uint32_t mlo, uint32_t mhi, float s, float s16, float m) {
    const uint32_t ev = w & mlo, od = w & mhi;
    const float v0 = __builtin_fmaf((float)(ev & 0xFF), s, m);
    const float v2 = __builtin_fmaf((float)((ev >> 8) & 0xFF), s, m);
    const float v4 = __builtin_fmaf((float)((ev >> 16) & 0xFF), s, m);
    const float v6 = __builtin_fmaf((float)(ev >> 24), s, m);
    const float v1 = __builtin_fmaf((float)(od & 0xFF), s16, m);
    const float v3 = __builtin_fmaf((float)((od >> 8) & 0xFF), s16, m);
    const float v5 = __builtin_fmaf((float)((od >> 16) & 0xFF), s16, m);
    const float v7 = __builtin_fmaf((float)(od >> 24), s16, m);
    return make_uint4(pack2_bf16(v0, v1), pack2_bf16(v2, v3), pack2_bf16(v4, v5), pack2_bf16(v6, v7));
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

template <int BM, int BN, int WM, int DA, int DB, bool kVec>
struct Gemm {
    static constexpr int WN = 4 / WM;
    static constexpr int kWRows = BM / WM, kWCols = BN / WN;  // a wave's output tile
    static constexpr int kMT = kWRows / 32, kNT = kWCols / 32;  // its 32 x 32 MFMA tiles
    static_assert(kMT >= 1 && kNT >= 1 && kWRows % 32 == 0 && kWCols % 32 == 0, "wave tile");
    static constexpr int kAInst = BM / 32;  // A copies per wave per k-tile (1 KB each)
    static constexpr int kBInst = kVec ? Smem<BM, BN, DA, DB>::kBpChunks / 256 : 8 * BN / 256;  // packed-word copies
    // dequant: kTPC threads per column, each converting kWPT of its 8 packed words per k-tile
    static constexpr int kTPC = BN <= 128 ? 256 / BN : 1;
    static constexpr int kWPT = 8 / kTPC;
    static_assert(BN <= 256 && (BN > 128 || 256 % BN == 0), "dequant split");
    using S = Smem<BM, BN, DA, DB>;
    static_assert(S::kTotal <= 160 * 1024, "LDS budget");
    // schedule: kMFMA MFMAs per k-step; the first kLead of k-step 0 carry no dequant (its words
    // are still coming from LDS); kVPM VALU slots after each of the others
    static constexpr int kMFMA = kMT * kNT;
    static constexpr int kLead = kMFMA >= 8 ? 2 : 0;
    static constexpr int kValuPerStep = 22 * kWPT / (BK / 16) + 2;
    static constexpr int kVPM = (kValuPerStep + kMFMA - kLead - 1) / (kMFMA - kLead);

    // Copies a wave may still have in flight at the end of k-tile t (parity p) once A(t+1) has
    // landed: the rest of k-tile t+1-DA (its words and scales) and all of k-tiles t+2-DA .. t.
    static constexpr int sc_copies(int u) { return ((u + DB) & 1) == 0 ? 2 : 0; }  // scales at k-tile u
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
    uint32_t mlo, mhi;
    // per-lane byte offsets of the copies (constant over the k-loop)
    uint32_t a_off[kAInst];  // from the k-tile's A base
    uint32_t b_off[kBInst > 0 ? kBInst : 1];  // from the k-tile's first packed row
    uint32_t sc_off[2];      // scale/min dword for even / odd g*N
    // this thread's LDS byte offsets (from smem, without the stage)
    uint32_t a_rd[kMT][BK / 16];  // A fragment (i, k-step)
    uint32_t b_rd;                // B fragment of j = 0, k-step 0
    uint32_t bq_wr[2];            // dequantized row segment, per destination stage
    uint32_t bp_rd;               // packed word of this thread's first row, this thread's column
    uint32_t sc_rd[2];            // scale of this thread's column, for even / odd g*N

    __device__ __forceinline__ void init() {
        const int lane = lane_id(), wave = wave_id(), tid = threadIdx.x;
        const int l32 = lane & 31, lh = lane >> 5;
        const int wm = wave % WM, wn = wave / WM;
        sm = lds_addr(smem);
        // A copies: instruction i of wave w fills rows w*BM/4 + 8i .. +7; lane l lands on chunk
        // l % 8 of row l / 8 and so reads the global chunk that the swizzle maps there.  Rows past
        // M repeat row M-1; they only feed outputs that are never stored.
#pragma unroll
        for (int i = 0; i < kAInst; ++i) {
            const int r = wave * (BM / 4) + 8 * i + (lane >> 3);
            const int gr = min(m0 + r, M - 1) - m0;
            a_off[i] = (uint32_t)(((size_t)gr * K + 8 * a_swizzle(r, lane & 7)) * 2);
        }
        // Packed words, LDS layout [8 packed rows][BN columns] u32.  Vector copies (N % 4 == 0):
        // 16-byte chunk c = row * BN/4 + column / 4; lanes past the last chunk land in the stage's
        // pad.  Dword copies: dword d = row * BN + column.  Columns past N repeat a valid column.
#pragma unroll
        for (int i = 0; i < kBInst; ++i) {
            const int d = (i * 4 + wave) * kWave + lane;
            int row, col;
            if (kVec) {
                const int c = min(d, 2 * BN - 1);
                row = c / (BN / 4);
                col = min(n0 + 4 * (c % (BN / 4)), N - 4);
            } else {
                row = d / BN;
                col = min(n0 + d % BN, N - 1);
            }
            b_off[i] = (uint32_t)(((size_t)row * N + col) * 4);
        }
        // Scales (one copy) and minimums (another): slot w*64 + l receives the aligned dword that
        // holds the bf16 of column min(n0 + min(w*64 + l, BN-1), N-1) in the group's row; where
        // the dword starts depends on the parity of g*N, so both offsets are kept.
        {
            const int c = min(n0 + min(wave * kWave + lane, BN - 1), N - 1);
            sc_off[0] = (uint32_t)((2 * c) & ~3);
            sc_off[1] = (uint32_t)((2 + 2 * c) & ~3);
        }
#pragma unroll
        for (int i = 0; i < kMT; ++i)
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                const int r = wm * kWRows + i * 32 + l32;
                a_rd[i][ks] = S::oA + (uint32_t)(r * BK + 8 * a_swizzle(r, 2 * ks + lh)) * 2;
            }
        b_rd = S::oBdq + (uint32_t)((wn * kWCols + l32) * LDT + 8 * lh) * 2;
        // dequant: thread tid converts words h*kWPT .. of column col (one column per thread when
        // BN > 128, the threads past column BN-1 writing to the sink; else kTPC per column)
        const int col = kTPC > 1 ? tid % BN : min(tid, BN - 1);
        const int h = kTPC > 1 ? tid / BN : 0;
#pragma unroll
        for (int st = 0; st < 2; ++st)
            bq_wr[st] = (kTPC > 1 || tid < BN) ? S::oBdq + st * S::kBdq + col * LDT * 2 + h * kWPT * 16
                                               : S::oSink + (tid - BN) * 16;
        bp_rd = S::oBp + col * 4 + h * kWPT * BN * 4;
        // the bf16 of column c in group g is the (g*N + c) & 1 half of its slot
        const int c = min(n0 + col, N - 1);
        sc_rd[0] = S::oSc + col * 4 + 2 * (c & 1);
        sc_rd[1] = S::oSc + col * 4 + 2 * ((c + 1) & 1);
    }

    __device__ __forceinline__ int64_t group_n(int t) const {
        return (int64_t)((kbeg + min(t, ntiles - 1) * BK) / 128) * N;
    }

    // Copies i0 .. i1-1 of this wave's share of A of k-tile ta, into stage ta % kAS.  Indices past
    // the end fetch the last k-tile again (the data is never used; the stage is the one the index
    // names, which no MFMA is reading).
    __device__ __forceinline__ void issue_a(int ta, int i0 = 0, int i1 = kAInst) const {
        const int wave = wave_id();
        const char* base =
            reinterpret_cast<const char*>(x) + ((size_t)m0 * K + kbeg + (size_t)min(ta, ntiles - 1) * BK) * 2;
        const uint32_t dst = sm + S::oA + (ta % S::kAS) * S::kA + wave * (BM / 4) * BK * 2;
#pragma unroll
        for (int i = i0; i < i1; ++i) dma16(a_off[i], base, dst + i * 8 * BK * 2);
    }

    // The packed words of k-tile tb into stage tb % kBS and, if kSc, its group's scales and
    // minimums into stage (tb / 2) % kSS (tb is then the group's first k-tile).
    template <bool kSc>
    __device__ __forceinline__ void issue_b(int tb) const {
        const int wave = wave_id();
        const char* base =
            reinterpret_cast<const char*>(codes) + (size_t)((kbeg + min(tb, ntiles - 1) * BK) / 8) * N * 4;
        const uint32_t dst = sm + S::oBp + (tb % S::kBS) * S::kBp;
#pragma unroll
        for (int i = 0; i < kBInst; ++i) {
            if (kVec)
                dma16(b_off[i], base, dst + (i * 4 + wave) * 1024);
            else
                dma4(b_off[i], base, dst + (i * 4 + wave) * 256);
        }
        if (kSc) {
            const int64_t gN = group_n(tb);
            const uint32_t off = (gN & 1) ? sc_off[1] : sc_off[0];  // (no dynamic index: keeps it in a register)
            const uint32_t sdst = sm + S::oSc + ((tb / 2) % S::kSS) * S::kSc + wave * 256;
            const int64_t row = (2 * gN) & ~(int64_t)3;
            dma4(off, reinterpret_cast<const char*>(scales) + row, sdst);
            dma4(off, reinterpret_cast<const char*>(mins) + row, sdst + 1024);
        }
    }

    // This thread's kWPT packed words of k-tile tn and its group's scale and minimum.
    __device__ __forceinline__ void read_words(int tn, uint32_t (&w)[kWPT], float& s, float& s16, float& m) const {
        const uint8_t* bp = smem + bp_rd + (tn % S::kBS) * S::kBp;
#pragma unroll
        for (int r = 0; r < kWPT; ++r) w[r] = *reinterpret_cast<const uint32_t*>(bp + r * BN * 4);
        const uint8_t* sc = smem + ((group_n(tn) & 1) ? sc_rd[1] : sc_rd[0]) + ((tn / 2) % S::kSS) * S::kSc;
        s = bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(sc));
        m = bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(sc + 1024));
        s16 = s * 0.0625f;
    }

    __device__ __forceinline__ void dequant_all(int st, const uint32_t (&w)[kWPT], float s, float s16, float m) const {
        uint8_t* dst = smem + bq_wr[st];
#pragma unroll
        for (int r = 0; r < kWPT; ++r)
            *reinterpret_cast<uint4*>(dst + r * 16) = dequant_word(w[r], mlo, mhi, s, s16, m);
    }

    // One k-tile t: MFMAs on A stage t % kAS and dequantized B stage `st` = t & 1 while the words `w` (the next
    // k-tile) are dequantized into the other B stage, spread evenly over the k-steps.  issue(ks) runs at the
    // top of each k-step: the copies for later k-tiles are spread over the tile rather than issued
    // in one burst, which would hold up the wave's first MFMAs behind the load unit.
    template <int st, typename Issue>
    __device__ __forceinline__ void mma_tile(int t, f32x16_t (&acc)[kMT][kNT], const uint32_t (&w)[kWPT], float s,
                                             float s16, float m, Issue&& issue) const {
        const uint8_t* abase = smem + S::kA * (S::kAS == 2 ? st : t % S::kAS);
        const uint8_t* bbase = smem + b_rd + S::kBdq * st;
        uint8_t* dst = smem + bq_wr[st ^ 1];
        bf16x8_t af[2][kMT], bfr[2][kNT];
        auto read_frags = [&](int ks, int slot) {
#pragma unroll
            for (int i = 0; i < kMT; ++i)
                af[slot][i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(abase + a_rd[i][ks]));
#pragma unroll
            for (int j = 0; j < kNT; ++j)
                bfr[slot][j] =
                    __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(bbase + j * 32 * LDT * 2 + ks * 32));
        };
        read_frags(0, 0);
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            __builtin_amdgcn_sched_barrier(0);
            issue(ks);
            if (ks + 1 < BK / 16) read_frags(ks + 1, (ks + 1) & 1);
#pragma unroll
            for (int r = 0; r < kWPT; ++r)
                if (r * (BK / 16) / kWPT == ks)
                    *reinterpret_cast<uint4*>(dst + r * 16) = dequant_word(w[r], mlo, mhi, s, s16, m);
#pragma unroll
            for (int j = 0; j < kNT; ++j)
#pragma unroll
                for (int i = 0; i < kMT; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][i], bfr[ks & 1][j], acc[i][j], 0,
                                                                        0, 0);
            step_schedule<kMFMA, kVPM>(ks == 0 ? kLead : 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
};

template <int BM, int BN, int WM, int DA, int DB, bool kVec>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_g128_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ codes,
                      const uint16_t* __restrict__ scales, const uint16_t* __restrict__ mins,
                      uint16_t* __restrict__ y, float* __restrict__ ws, int M, int N, int K, int k_per_split,
                      int splits, uint32_t mask_lo, uint32_t mask_hi) {
    using G = Gemm<BM, BN, WM, DA, DB, kVec>;
    constexpr int kMT = G::kMT, kNT = G::kNT, kWPT = G::kWPT;
    __shared__ __attribute__((aligned(16))) uint8_t smem[Smem<BM, BN, DA, DB>::kTotal];
    // XCD-aware tile order: block b runs on XCD b % 8, so XCD x takes the x-th contiguous eighth
    // of the (split, m, n) tile sequence, n fastest -- its blocks share A rows in its own L2.
    const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
    const int total = tiles_n * tiles_m * splits;  // gridDim.x == 8 * per_xcd >= total
    const int per_xcd = (int)gridDim.x / 8;
    const int t = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (t >= total) return;
    const int split_id = t / (tiles_n * tiles_m);

    G g;
    g.x = x;
    g.codes = codes;
    g.scales = scales;
    g.mins = mins;
    g.smem = smem;
    g.M = M;
    g.N = N;
    g.K = K;
    g.m0 = (t / tiles_n % tiles_m) * BM;
    g.n0 = (t % tiles_n) * BN;
    g.kbeg = split_id * k_per_split;
    g.ntiles = (min(K, g.kbeg + k_per_split) - g.kbeg) / BK;  // even: splits are whole groups
    g.mlo = mask_lo;
    g.mhi = mask_hi;
    g.init();
    // the accumulators stay outside `g`: a local array is kept in registers across the copies'
    // inline assembly, whose memory clobber would otherwise force them out to scratch
    f32x16_t acc[kMT][kNT];
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // Prologue: A of k-tiles 0 .. DA-1, the words of 0 .. DB-1 and the scales of their groups;
    // k-tile 0 is then dequantized into B stage 0.
#pragma unroll
    for (int t0 = 0; t0 < DA; ++t0) g.issue_a(t0);
#pragma unroll
    for (int t0 = 0; t0 < DB; ++t0) {
        if (t0 % 2 == 0)
            g.template issue_b<true>(t0);
        else
            g.template issue_b<false>(t0);
    }
    wait_vm<0>();
    __syncthreads();
    {
        uint32_t w[kWPT];
        float s, s16, m;
        g.read_words(0, w, s, s16, m);
        g.dequant_all(0, w, s, s16, m);
    }
    __syncthreads();

    // k-tile t: read the words of t+1; run the MFMAs of t while dequantizing t+1 and copying
    // A(t+DA) (spread over the k-steps) and then the words of t+DB (with their group's scales
    // when t+DB starts a group); then wait until A(t+1) and everything issued before it has
    // landed -- the words of t+2 and their scales were requested no later than A(t+1), since
    // DB >= DA + 2 -- and meet at the barrier.
    constexpr int kSteps = BK / 16;
    constexpr int kWaitEven = G::after_a(0), kWaitOdd = G::after_a(1);
    auto issue_a_step = [&](int ta, int ks) {  // the A copies whose turn is k-step ks
#pragma unroll
        for (int i = 0; i < G::kAInst; ++i)
            if (i * kSteps / G::kAInst == ks) g.issue_a(ta, i, i + 1);
    };
    for (int tt = 0; tt < g.ntiles; tt += 2) {
        {
            uint32_t w[kWPT];
            float s, s16, m;
            g.read_words(tt + 1, w, s, s16, m);
            g.template mma_tile<0>(tt, acc, w, s, s16, m, [&](int ks) {
                issue_a_step(tt + DA, ks);
                if (ks == kSteps - 1) g.template issue_b<DB % 2 == 0>(tt + DB);
            });
            wait_vm<kWaitEven>();
            __syncthreads();
        }
        {
            uint32_t w[kWPT];
            float s, s16, m;
            g.read_words(tt + 2, w, s, s16, m);
            g.template mma_tile<1>(tt + 1, acc, w, s, s16, m, [&](int ks) {
                issue_a_step(tt + 1 + DA, ks);
                if (ks == kSteps - 1) g.template issue_b<DB % 2 == 1>(tt + 1 + DB);
            });
            wait_vm<kWaitOdd>();
            __syncthreads();
        }
    }
    wait_vm<0>();  // no copy may still be writing this block's LDS when it exits

    // D fragment of a 32 x 32 tile: element e of lane l is row 8*(e/4) + 4*(l/32) + e%4, column l%32.
    const int lane = lane_id(), wave = wave_id();
    const int l32 = lane & 31, lh = lane >> 5;
    const int wm = wave % WM, wn = wave / WM;
    const bool split = splits > 1;
#pragma unroll
    for (int i = 0; i < kMT; ++i)
#pragma unroll
        for (int j = 0; j < kNT; ++j) {
            const int col = g.n0 + wn * G::kWCols + j * 32 + l32;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = g.m0 + wm * G::kWRows + i * 32 + 8 * (e / 4) + 4 * lh + (e % 4);
                if (row < M && col < N) {
                    if (split)
                        ws[((size_t)split_id * M + row) * N + col] = acc[i][j][e];
                    else
                        y[(size_t)row * N + col] = f32_to_bf16_bits(acc[i][j][e]);
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
// split, from 128 rows (64 x 128 tiles, 2 x 2 waves) to 1024 rows (256 x 224, waves along M).
enum TileCfg { kT64x128, kT128x128, kT128x256, kT256x224 };

struct GemmPlan {
    TileCfg cfg;
    int bm, bn, tiles_m, tiles_n, splits, k_per_split;
};

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K) {
    GemmPlan p;
    if (M <= 128) p.cfg = kT64x128, p.bm = 64, p.bn = 128;
    else if (M <= 256) p.cfg = kT128x128, p.bm = 128, p.bn = 128;
    else if (M <= 512) p.cfg = kT128x256, p.bm = 128, p.bn = 256;
    else p.cfg = kT256x224, p.bm = 256, p.bn = 224;
    p.tiles_m = (int)((M + p.bm - 1) / p.bm);
    p.tiles_n = (int)((N + p.bn - 1) / p.bn);
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    const int groups = (int)(K / 128);
    int splits = 1;  // split K only when the tiles would leave more than half the CUs idle
    if (2 * tiles <= kCUs) splits = (int)std::min<int64_t>(groups, (kCUs + tiles - 1) / tiles);
    // k per split in whole groups; recompute the split count so no split is empty
    const int groups_per_split = (groups + splits - 1) / splits;
    p.k_per_split = groups_per_split * 128;
    p.splits = (groups + groups_per_split - 1) / groups_per_split;
    return p;
}

template <int BM, int BN, int WM, int DA, int DB>
void launch_cfg(const GemmPlan& p, const uint16_t* x, int64_t M, const uint32_t* codes, const uint16_t* scales,
                const uint16_t* mins, int64_t N, int64_t K, uint16_t* y, float* workspace, hipStream_t stream) {
    // a 1-D grid of 8 x ceil(tiles / 8) blocks over (split, m, n); the surplus exit at once
    const int64_t tiles = (int64_t)p.tiles_n * p.tiles_m * p.splits;
    const dim3 grid((unsigned)(8 * ((tiles + 7) / 8)));
    if (N % 4 == 0)
        hipLaunchKernelGGL((gemm_g128_kernel<BM, BN, WM, DA, DB, true>), grid, dim3(kThreads), 0, stream, x, codes, scales,
                           mins, y, workspace, (int)M, (int)N, (int)K, p.k_per_split, p.splits, 0x0F0F0F0Fu,
                           0xF0F0F0F0u);
    else
        hipLaunchKernelGGL((gemm_g128_kernel<BM, BN, WM, DA, DB, false>), grid, dim3(kThreads), 0, stream, x, codes, scales,
                           mins, y, workspace, (int)M, (int)N, (int)K, p.k_per_split, p.splits, 0x0F0F0F0Fu,
                           0xF0F0F0F0u);
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
        case kT64x128: launch_cfg<64, 128, 2, 3, 6>(p, x, M, codes, scales, mins, N, K, y, workspace, stream); break;
        case kT128x128: launch_cfg<128, 128, 2, 2, 5>(p, x, M, codes, scales, mins, N, K, y, workspace, stream); break;
        case kT128x256: launch_cfg<128, 256, 2, 1, 4>(p, x, M, codes, scales, mins, N, K, y, workspace, stream); break;
        case kT256x224: launch_cfg<256, 224, 4, 1, 3>(p, x, M, codes, scales, mins, N, K, y, workspace, stream); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    const int64_t MN = M * N;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, stream, workspace, y,
                       MN, p.splits);
    return hipGetLastError();
}

}  // namespace w4a16
