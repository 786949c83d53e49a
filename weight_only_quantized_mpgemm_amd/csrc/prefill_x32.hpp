// Large-M (prefill) W4A16 GEMM for gfx950 on the 32x32x16 matrix instruction.
//
// [TurboMind, technique (iii), Fig. 9 caption]: a software-pipelined main loop keeps the
// matrix cores busy on step k with already-dequantized fragments while the integer/float
// ALUs dequantize step k+1 and the memory pipeline fetches later tiles.  Source: "LMDeploy
// Accelerates Mixed-Precision LLM Inference with TurboMind" (arXiv 2508.15601).
//
// Why 32x32x16: one wave of a CDNA4 SIMD issues at most one instruction every four cycles,
// and a matrix instruction takes two of those slots.  v_mfma_f32_32x32x16 keeps the matrix
// core busy 32 cycles per issue (twice the 16x16x32 form for the same two slots), which
// leaves about six slots per matrix instruction for the dequantization, LDS reads and
// bookkeeping of the next step -- the 16x16x32 form leaves two, fewer than the fp16
// dequantization alone needs (13 vector operations per 8 weights, each weight feeding
// 128 rows).
//
// Design (K % 128 == 0), in two tile shapes of equal work per wave (NB column blocks x
// MB = 8 / NB row blocks of 32 x 32):
//   - NB = 2: workgroup tile 128 (m) x 256 (n), four waves side by side along n, each
//     owning a 128 x 64 block = 2 (n) x 4 (m) blocks;
//   - NB = 1: workgroup tile 256 (m) x 128 (n), each wave a 256 x 32 block = 1 (n) x 8 (m)
//     blocks.  Every dequantized weight then feeds 256 rows instead of 128, halving the
//     dequantization work (and the weight loads) per MFMA, for twice the LDS operand reads
//     (one ds_read_b128 per MFMA; gfx950's LDS sustains that beside full-rate MFMAs);
//   - either way 128 fp32 accumulators per lane in AGPRs, updated in place by inline-asm
//     MFMA;
//   - weights are the A operand (rows = n): lane l holds column n = l % 32 of a 32-column
//     block (two 16-column strips of the packed layout) at k = 16u + 8 (l / 32) .. +7 of a
//     32-deep step.  In the packed layout that is strip (l % 32) / 16, lane position
//     l % 16 + 16 (2u + l / 32), word = step within the 128-deep tile -- each lane simply
//     loads a different 16-byte slot of the same 1 KiB tiles, so the layout is shared with
//     the 16x16x32 kernels;
//   - weights: one 16-byte load per lane per (column block, k half) per 128-deep tile,
//     issued three tiles (six stages) ahead into four register sets used in rotation (one
//     tile ahead in two sets for g = 64) --
//     HBM latency under full load exceeds the one to two stages a two-set scheme gives;
//   - activations are the B operand (columns = m), read from a ring of four BM x 64 LDS
//     stages filled by buffer_load_dwordx4 ... lds three stages ahead (XOR-swizzled 16-byte
//     chunks, chunk ^ row % 8, so eight consecutive rows hit eight bank groups); a short
//     grid keeps only its live rows, in eight stages filled seven ahead;
//   - each 32-deep step runs 16 MFMAs; after MFMA i come 1/16 of the next step's work: its
//     LDS operand reads (2 MB per step) and dequantization operations (13 or 14 for each of
//     the next step's 2 NB weight words).  With four words the operations go round-robin
//     over them, so no operation directly follows the one it depends on; with two, word 0
//     is done first, since the next step's first MFMA needs it.  The dequantization is
//     inline asm too, so the compiler neither reorders it nor pads it with wait states
//     meant for the MFMAs.
//
// This header holds the kernel template and its launch helpers; the gemm_prefill_x32*.hip
// translation units instantiate it per code format (they compile in parallel).
#pragma once

#include <cstdlib>
#include <type_traits>
#include <utility>

#include "kernels.hpp"

namespace mpgemm {

namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kXThreads = 256;
constexpr int kXStages = 4;                  // 64-deep LDS stages in the ring (eight at small M)
// Workgroup tile shapes SH: 1 = 256 (m) x 128 (n), 2 = 128 x 256, 3 = 256 x 256.  Each of
// the four waves owns shape_nb(SH) 32-column blocks of shape_mb(SH) 32-row blocks.
constexpr int shape_nb(int sh) { return sh == 1 ? 1 : 2; }
constexpr int shape_mb(int sh) { return sh == 2 ? 4 : 8; }
constexpr int tile_m(int sh) { return 32 * shape_mb(sh); }    // workgroup tile rows (m)
constexpr int tile_n(int sh) { return 128 * shape_nb(sh); }   // workgroup tile columns (n)
// Workgroups of the split reduction per tile: four chunks of a lane's 4 NB MB each.
constexpr int x32_reduce_wgs(int sh) { return shape_nb(sh) * shape_mb(sh); }
// Weight register sets (loads run NWS - 1 tiles ahead): four for 4-bit codes with
// g = 128; two for g = 64, whose doubled scale/zero registers would not fit four sets
// without spilling, and two for 8-bit codes (twice the code registers per set).
template <int G, int CODE>
constexpr int kXWSets = (G == 128 && CODE == kU4) ? 4 : 2;

template <int N>
struct IC {
    static constexpr int value = N;
};

// Loads a stage's wait may leave in flight: every load the wave issued after the DMA of
// the stage after it.  That DMA went out in step 0 of stage st + 2 - XS (DMAs run XS - 1
// stages ahead); after it came the weight loads of that stage's step 1, and all loads of
// the XS - 3 stages in between: their DMAs (DMB each) and, in the even stages of a pass
// that loads weights (LW), kWLoads weight loads.  Only stages of the same pass of the
// stage loop are counted (KB: the stage's place in the pass): the pass may follow the
// prologue, whose weight loads the compiler moves past its barrier.
constexpr int stage_wait_loads(int xs, int dmb, int wloads, int kb, bool lw) {
    int n = (xs - 3) * dmb;
    for (int j = kb + 2 - xs; j <= kb - 1; ++j)
        if (lw && j >= 0 && j % 2 == 0) n += wloads;
    return n;
}

// Wait until at most NV vector-memory operations of this wave are outstanding, then meet
// the rest of the workgroup.  The memory clobber keeps LDS accesses on their side of it.
template <int NV>
__device__ __forceinline__ void wait_vm_barrier() {
    static_assert(NV >= 0 && NV < 64, "vmcnt range");
    constexpr int imm = (NV & 15) | ((NV >> 4) << 14) | (7 << 4) | (15 << 8);
    asm volatile("s_waitcnt %0\n\ts_barrier" ::"n"(imm) : "memory");
}

// acc += a * b on one 32 x 32 block, accumulator pinned in place in AGPRs.  Inline asm is
// invisible to the compiler's hazard tracking: the schedule keeps every VALU write of an
// operand at least three instructions ahead of the MFMA that reads it, and the main loop
// drains the matrix pipeline (mfma_drain) before any code the compiler places after it.
template <int ACT>
__device__ __forceinline__ void mfma32(f32x16_t &c, const u32x4_t &a, const u32x4_t &b);
template <>
__device__ __forceinline__ void mfma32<kF16>(f32x16_t &c, const u32x4_t &a, const u32x4_t &b) {
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
template <>
__device__ __forceinline__ void mfma32<kBF16>(f32x16_t &c, const u32x4_t &a, const u32x4_t &b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// Constants the dequantization keeps in registers for the whole kernel.  Produced by asm
// so the compiler cannot rematerialize them (an s_mov / v_mov per use) inside the loop.
struct DqConst {
    uint32_t m_lo, m_hi;     // SGPR masks 0x000F000F, 0x00F000F0
    uint32_t b_hi, b_lo;     // VGPR fp16x2 patterns 1024.0 (0x6400) and 64.0 (0x5400)
    uint32_t m_byte;         // VGPR 0x0F0F0F0F (bf16 nibble spread)
    uint32_t p_hi;           // VGPR bytes 0x64 (8-bit codes: the byte-permute pattern)
    uint32_t sel_lo, sel_hi; // SGPR permute selectors for codes (0, 1) and (2, 3) of a word
};
template <int CODE>
__device__ __forceinline__ DqConst make_dq_const() {
    DqConst c;
    if constexpr (CODE == kU4) {
        asm volatile("s_mov_b32 %0, 0x000F000F" : "=s"(c.m_lo));
        asm volatile("s_mov_b32 %0, 0x00F000F0" : "=s"(c.m_hi));
        asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(c.b_hi));
        asm volatile("v_mov_b32 %0, 0x54005400" : "=v"(c.b_lo));
        asm volatile("v_mov_b32 %0, 0x0F0F0F0F" : "=v"(c.m_byte));
    } else if constexpr (CODE == kU8) {
        asm volatile("v_mov_b32 %0, 0x64646464" : "=v"(c.p_hi));
        asm volatile("s_mov_b32 %0, 0x04010400" : "=s"(c.sel_lo));
        asm volatile("s_mov_b32 %0, 0x04030402" : "=s"(c.sel_hi));
    } else if constexpr (CODE == kE5M2) {
        // each code to the high byte of an fp16 half, low byte zero (selector 0x0C)
        asm volatile("s_mov_b32 %0, 0x010C000C" : "=s"(c.sel_lo));
        asm volatile("s_mov_b32 %0, 0x030C020C" : "=s"(c.sel_hi));
    }
    return c;
}

// Scratch values of one word's dequantization.
struct DqTmp {
    uint32_t sh, h[4];
    float f[8];
};

// Operation OP of the dequantization of word w into out (8 weights, k order), with the
// results of Dq<ACT>::word.  fp16 (13 operations): one shift, four isolate-and-combine
// (1024 + q / 64 + q as fp16 pairs), four exact packed adds of -(B + z), four packed
// multiplies by s (the one rounding).  bf16 (17 operations): the same shift and isolate-
// and-combine, eight mixed-precision fmas (B + q) s - (B + z) s that read each fp16 half
// directly and are exact in fp32 (11-bit integers times an 11-bit significand; the
// difference (q - z) s has at most 16 bits), four conversions to bf16 pairs (the one
// rounding).  Dq<kBF16>::word computes q s - z s instead: the same exact values.
template <int ACT>
struct DqOps;

template <>
struct DqOps<kF16> {
    static constexpr int kCount = 13;
    template <int OP>
    static __device__ __forceinline__ void run(uint32_t w, const DqF16 &d, const DqConst &c,
                                               DqTmp &t, u32x4_t &out) {
        if constexpr (OP == 0) {
            asm("v_lshrrev_b32 %0, 8, %1" : "=v"(t.sh) : "v"(w));
        } else if constexpr (OP >= 1 && OP <= 4) {
            constexpr int j = OP - 1;
            const uint32_t src = (j < 2) ? w : t.sh;
            if constexpr ((j & 1) == 0)
                asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(t.h[j]) : "v"(src), "s"(c.m_lo), "v"(c.b_hi));
            else
                asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(t.h[j]) : "v"(src), "s"(c.m_hi), "v"(c.b_lo));
        } else if constexpr (OP >= 5 && OP <= 8) {
            constexpr int j = OP - 5;
            const uint32_t nz = (j & 1) ? d.nz_lo2 : d.nz_hi2;
            asm("v_pk_add_f16 %0, %1, %2" : "=v"(t.h[j]) : "v"(t.h[j]), "v"(nz));
        } else {
            constexpr int j = OP - 9;
            uint32_t r;
            asm("v_pk_mul_f16 %0, %1, %2" : "=v"(r) : "v"(t.h[j]), "v"(d.s2));
            out[j] = r;
        }
    }
};

template <>
struct DqOps<kBF16> {
    static constexpr int kCount = 17;
    template <int OP>
    static __device__ __forceinline__ void run(uint32_t w, const DqBF16 &d, const DqConst &c,
                                               DqTmp &t, u32x4_t &out) {
        if constexpr (OP == 0) {
            asm("v_lshrrev_b32 %0, 8, %1" : "=v"(t.sh) : "v"(w));
        } else if constexpr (OP >= 1 && OP <= 4) {
            constexpr int j = OP - 1;
            const uint32_t src = (j < 2) ? w : t.sh;
            if constexpr ((j & 1) == 0)
                asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(t.h[j]) : "v"(src), "s"(c.m_lo), "v"(c.b_hi));
            else
                asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(t.h[j]) : "v"(src), "s"(c.m_hi), "v"(c.b_lo));
        } else if constexpr (OP >= 5 && OP <= 12) {
            constexpr int e = OP - 5, j = e / 2;
            const uint16_t bits = (uint16_t)((e & 1) ? t.h[j] >> 16 : t.h[j]);
            t.f[e] = __builtin_fmaf((float)bitcast<_Float16>(bits), d.s, (j & 1) ? d.nz_lo : d.nz_hi);
        } else {
            constexpr int j = OP - 13;
            out[j] = pack_bf16x2(t.f[2 * j], t.f[2 * j + 1]);
        }
    }
};

// The same for 8-bit codes: the words w0, w1 hold codes k0..k7 (k0 in the low byte), in the
// arithmetic of Dq8<ACT>::pair.  fp16 (12 operations): four byte permutes against 0x64
// (1024 + q pairs), four exact packed adds of -(1024 + z), four packed multiplies by s.
// bf16 (12 operations): eight convert-and-fma q * s - z * s, four conversions to bf16
// pairs.
template <int ACT>
struct DqOps8;

template <>
struct DqOps8<kF16> {
    static constexpr int kCount = 12;
    template <int OP>
    static __device__ __forceinline__ void run(uint32_t w0, uint32_t w1, const DqF16 &d,
                                               const DqConst &c, DqTmp &t, u32x4_t &out) {
        if constexpr (OP <= 3) {
            const uint32_t w = OP < 2 ? w0 : w1;
            if constexpr ((OP & 1) == 0)
                asm("v_perm_b32 %0, %1, %2, %3" : "=v"(t.h[OP]) : "v"(c.p_hi), "v"(w), "s"(c.sel_lo));
            else
                asm("v_perm_b32 %0, %1, %2, %3" : "=v"(t.h[OP]) : "v"(c.p_hi), "v"(w), "s"(c.sel_hi));
        } else if constexpr (OP <= 7) {
            constexpr int j = OP - 4;
            asm("v_pk_add_f16 %0, %1, %2" : "=v"(t.h[j]) : "v"(t.h[j]), "v"(d.nz_hi2));
        } else {
            constexpr int j = OP - 8;
            uint32_t r;
            asm("v_pk_mul_f16 %0, %1, %2" : "=v"(r) : "v"(t.h[j]), "v"(d.s2));
            out[j] = r;
        }
    }
};

template <>
struct DqOps8<kBF16> {
    static constexpr int kCount = 12;
    template <int OP>
    static __device__ __forceinline__ void run(uint32_t w0, uint32_t w1, const DqBF16 &d,
                                               const DqConst &c, DqTmp &t, u32x4_t &out) {
        (void)c;
        if constexpr (OP <= 7) {
            t.f[OP] = __builtin_fmaf(ubyte(OP < 4 ? w0 : w1, OP & 3), d.s, d.nzs);
        } else {
            constexpr int j = OP - 8;
            out[j] = pack_bf16x2(t.f[2 * j], t.f[2 * j + 1]);
        }
    }
};

// The same for FP8 codes, in the arithmetic of DqF8<ACT, CODE>::pair.  fp16 (8 operations):
// four exact conversions of code pairs to fp16 pairs (E4M3: scaled convert at scale 1.0;
// E5M2: byte permute to the high bytes), four packed multiplies by s.  bf16 (16
// operations): four exact conversions of code pairs to fp32 pairs, eight exact fp32
// multiplies by s, four conversions to bf16 pairs (the one rounding).
template <int ACT, int CODE>
struct DqOpsF8;

template <int CODE>
struct DqOpsF8<kF16, CODE> {
    static constexpr int kCount = 8;
    template <int OP>
    static __device__ __forceinline__ void run(uint32_t w0, uint32_t w1, const DqF16 &d,
                                               const DqConst &c, DqTmp &t, u32x4_t &out) {
        if constexpr (OP <= 3) {
            const uint32_t w = OP < 2 ? w0 : w1;
            if constexpr (CODE == kE4M3) {
                t.h[OP] = fp8_pair_f16<kE4M3, (OP & 1) != 0>(w);
            } else {
                const uint32_t sel = (OP & 1) ? c.sel_hi : c.sel_lo;
                asm("v_perm_b32 %0, %1, %1, %2" : "=v"(t.h[OP]) : "v"(w), "s"(sel));
            }
        } else {
            constexpr int j = OP - 4;
            uint32_t r;
            asm("v_pk_mul_f16 %0, %1, %2" : "=v"(r) : "v"(t.h[j]), "v"(d.s2));
            out[j] = r;
        }
    }
};

template <int CODE>
struct DqOpsF8<kBF16, CODE> {
    static constexpr int kCount = 16;
    template <int OP>
    static __device__ __forceinline__ void run(uint32_t w0, uint32_t w1, const DqBF16 &d,
                                               const DqConst &c, DqTmp &t, u32x4_t &out) {
        (void)c;
        if constexpr (OP <= 3) {
            const f32x2_t f = fp8_pair_f32<CODE, (OP & 1) != 0>(OP < 2 ? w0 : w1);
            t.f[2 * OP] = f.x;
            t.f[2 * OP + 1] = f.y;
        } else if constexpr (OP <= 11) {
            t.f[OP - 4] = t.f[OP - 4] * d.s;
        } else {
            constexpr int j = OP - 12;
            out[j] = pack_bf16x2(t.f[2 * j], t.f[2 * j + 1]);
        }
    }
};

template <int ACT, int CODE>
struct DqOpsSel {
    typedef DqOpsF8<ACT, CODE> type;
};
template <int ACT>
struct DqOpsSel<ACT, kU4> {
    typedef DqOps<ACT> type;
};
template <int ACT>
struct DqOpsSel<ACT, kU8> {
    typedef DqOps8<ACT> type;
};

// Tile of workgroup b.  Workgroups are dispatched round-robin over the eight XCDs
// (b % 8), each with its own L2; XCD x gets a contiguous range of tile indices, walked in
// groups of four M-tiles (all four rows of one N-tile, then the next N-tile), so the
// workgroups that run together on one XCD share four activation row-blocks and a few weight
// column-blocks instead of touching every row-block of X.
__host__ __device__ inline void tile_of(int b, int tm, int tn, int &mt, int &nt) {
    constexpr int kXcds = 8, kGroupM = 4;
    const int T = tm * tn, per = T / kXcds, extra = T % kXcds;
    const int x = b % kXcds;
    const int t = x * per + (x < extra ? x : extra) + b / kXcds;
    const int g = t / (kGroupM * tn);
    const int rest = tm - g * kGroupM;
    const int gm = rest < kGroupM ? rest : kGroupM;
    const int r = t - g * kGroupM * tn;
    mt = g * kGroupM + r % gm;
    nt = r / gm;
}

// Work of workgroup b in a launch whose first `full` workgroups run whole tiles and whose
// remaining tiles are each split into P consecutive workgroups over the K range: the tile
// (mt, nt), the part of its K range (0 .. parts-1) and the part count.  Split tile s (in
// launch order) is tile index full + s, the index the reduction kernel looks up.
struct X32Work {
    int mt, nt, part, parts, split_index;
};
__host__ __device__ inline X32Work x32_work_of(int b, int tm, int tn, int full, int P) {
    X32Work w{0, 0, 0, 1, -1};
    int t = b;
    if (b >= full && P > 1) {
        w.split_index = (b - full) / P;
        w.part = (b - full) % P;
        w.parts = P;
        t = full + w.split_index;
    }
    tile_of(t, tm, tn, w.mt, w.nt);
    return w;
}

// RAG: Kx < K; activation chunks at k >= Kx are loaded as zeros.  MA: row blocks of 32 that
// hold rows below M (MA < 8 / NB when M <= 32 MA): the MFMAs and activation operand reads
// of the others are skipped (their accumulators stay zero and are never stored); loads and
// DMAs are unchanged (rows past M read as zeros).
template <int ACT, bool SYM, int G, int NWS, int SH, int CODE, bool RAG, int MA>
__global__ __launch_bounds__(kXThreads) void prefill_x32_kernel(
    const uint16_t *__restrict__ X, const uint32_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros, int M, int N, int K,
    int Kw, int Kx, int Ny, int ldy, uint16_t *__restrict__ Y, int full, int P,
    float *__restrict__ part) {
    // N: the padded column count of the packed planes; Kw: their padded K (a multiple of
    // 128); K: the loop length, Kw rounded up to a multiple of 256 (the stage loop runs
    // blocks of four 64-deep stages; a 128-deep tile past Kw re-reads the last weight tile
    // against activations that read as zero, adding exact zeros); Kx: activation row length
    // (the user K); Ny: output columns (the user N); ldy: Y's row stride (Ny, or the full
    // row of a launch that covers a column range of Y).
    // full, P, part: workgroups past the first `full` take 1/P of the K range of one tile
    // each (P consecutive workgroups per tile; P = 1: no split) and store fp32 partials in
    // `part` instead of Y.
    typedef typename Dq<ACT>::type DqT;       // the same constants type for every code format
    typedef typename DqOpsSel<ACT, CODE>::type Ops;
    typedef DqFor<ACT, CODE> DqB;
    constexpr int BITS = kCodeBits<CODE>;
    // 128-bit pieces per lane, column block and k half per 128-deep step: one slot of a
    // 16 x 128 tile of 4-bit codes, one slot of each of two 16 x 64 tiles of 8-bit codes.
    constexpr int WV = BITS / 4;
    constexpr int GPT = kTileK / G;          // groups per 128-deep tile (1 or 2)
    constexpr int NB = shape_nb(SH);         // 32-column blocks per wave
    constexpr int MB = shape_mb(SH);         // 32-row blocks per wave
    constexpr int NMF = 2 * NB * MB;         // MFMAs per 32-deep step (16, or 32 at SH 3)
    constexpr int BM = tile_m(SH), BN = tile_n(SH);
    // One row of tiles whose live rows (MA row blocks) fill less than the tile, with four
    // weight sets: the ring holds only those rows, in eight stages instead of four, so its
    // DMAs run seven stages ahead and a weight tile has about six stages to land.  Few
    // rows make a short step (MA of MB row blocks), and with four stages the loads were not
    // covered.  (With two weight sets the compiler merged the eight-stage pass with the
    // tail and copied weight registers at the loop head, behind a full load wait.)
    constexpr bool DEEP = SH != 3 && MA < MB && NWS == 4;
    constexpr int XS = DEEP ? 8 : kXStages;  // ring stages
    constexpr int SR = DEEP ? 32 * MA : BM;  // rows per stage
    constexpr int DMB = SR / 32;             // DMA blocks of 8 rows per wave and stage
    constexpr int kChunks = SR * 8;          // 16-byte chunks per stage (8 per 64-deep row)
    // Loads each wave issues per weight tile: 2 NB WV 16-byte code slots (column blocks x
    // k halves x pieces), plus scales (and zeros) per column block and group.
    constexpr int kWLoads = 2 * NB * WV + NB * GPT * (SYM ? 1 : 2);
    static_assert(kWLoads <= 16, "weight loads are spread over one step's 16 MFMAs");
    __shared__ u32x4_t xs[XS][kChunks];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const X32Work work = x32_work_of(blockIdx.x, (M + BM - 1) / BM, (N + BN - 1) / BN, full, P);
    const int mt = work.mt, nt = work.nt, sp = work.part, parts = work.parts;
    const int sidx = work.split_index;       // split tile index (parts > 1)
    const int m_blk = mt * BM;
    const int KT = Kw >> 7;                  // 128-deep weight tiles in the packed planes
    const int S = (K >> 6) / parts;          // 64-deep stages of this part (a multiple of 4)
    const int t0 = sp * (S >> 1);            // its first weight tile (S = 2 tiles' stages)
    const int KTl = parts > 1 ? S >> 1 : KT; // weight tiles it may read (loads clamp to them)
    const int groups = Kw / G;
    const int strips = N >> 4;
    const int strip0 = nt * (BN / 16) + wave * 2 * NB;

    const rsrc_t xrs = make_rsrc(X, (uint32_t)((size_t)M * Kx * 2));
    const rsrc_t wrs = make_rsrc(codes, (uint32_t)((size_t)strips * KT * 1024 * WV));
    const rsrc_t srs = make_rsrc(scales, (uint32_t)((size_t)groups * N * 2));
    const rsrc_t zrs = make_rsrc(zeros, (uint32_t)((size_t)groups * N * BITS / 8));
    const DqConst dc = make_dq_const<CODE>();

    // DMA source offsets: wave w fills blocks b = DMB w + i of every stage; block b holds
    // rows 8b .. 8b+7, lane l writes LDS chunk 64b + l = (row 8b + l/8, physical chunk l%8),
    // which holds logical chunk (l%8) ^ (l/8).  Rows past M read zeros (one past the end).
    // (Offset arrays have fixed bounds, of which DMB / NB entries are used: with bounds
    // that depend on a template parameter, the host pass of this compiler silently emits
    // no launch stub for the kernel.)
    // The 256 x 256 tile keeps only block 0's offset and adds i times the 8-row stride at
    // each DMA (eight offsets would not fit its registers): rows past M then take offsets
    // past the plane, or wrap into it for the largest planes; either way their loads do
    // not fault, and those rows' results are never stored.
    uint32_t xoff[8];
#pragma unroll
    for (int i = 0; i < (SH == 3 ? 1 : DMB); ++i) {
        const int r = 8 * (wave * DMB + i) + (lane >> 3);
        const uint32_t row = SH == 3 ? (uint32_t)(m_blk + r) : (uint32_t)min(m_blk + r, M);
        xoff[i] = (row * Kx + (((lane & 7) ^ (lane >> 3)) * 8) + t0 * 128) * 2u;
    }
    const uint32_t xstep = 16u * (uint32_t)Kx;        // 8 rows of activations, in bytes
    // Ragged K: first k of the lane's chunk within a stage.
    const int k_chunk = ((lane & 7) ^ (lane >> 3)) * 8;
    // Weight slots: column block nb (strips strip0 + 2nb, +1), k half u.  Strips past N
    // read the last real strip; their results are never stored.
    const int my_strip_in_pair = (lane & 31) >> 4;
    constexpr int zrow = 16 * BITS / 8;                // zero bytes per (strip, group)
    uint32_t woff[2][2], soff[2], zoff[2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const uint32_t strip = (uint32_t)min(strip0 + 2 * nb + my_strip_in_pair, strips - 1);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint32_t pos = (lane & 15) + 16 * (2 * u + (lane >> 5));
            woff[nb][u] = (strip * KT + t0) * 1024u * WV + pos * 16u;
        }
        const uint32_t e = strip * groups * 16u + (lane & 15);
        soff[nb] = (e >> 1) * 4u + t0 * GPT * 32u;
        zoff[nb] = (BITS == 4 ? (e >> 3) * 4u : (e >> 2) * 4u) + t0 * GPT * zrow;
    }
    const uint32_t sshift = (lane & 1) * 16;
    // A lane's zero is nibble (lane & 7) of a dword (4-bit codes) or byte (lane & 3).
    const uint32_t zshift = BITS == 4 ? (lane & 7) * 4 : (lane & 3) * 8;
    constexpr uint32_t zmask = (1u << BITS) - 1;
    constexpr uint32_t zsym = 1u << (BITS - 1);        // symmetric zero: 8 or 128
    // B operand: row 32 mb + lane % 32, logical chunk 4s + 2u + lane / 32 of the stage;
    // physical chunk = logical ^ (lane % 8) = (4s + 2u) ^ cb.
    const int brow = (lane & 31) * 8;
    const int cb = (lane >> 5) ^ (lane & 7);

    f32x16_t acc[NB][MB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = f32x16_t{};

    struct WSet {
        u32x4_t w[NB][2][WV];                // [nb][u][piece]: the tile's four 32-deep steps
        uint32_t s[NB][GPT], z[NB][GPT];
    };
    static_assert(NWS == 2 || NWS == 4, "a pass of the stage loop holds whole weight-set rotations");
    static_assert(XS == 4 || XS == 8, "ring depth");
    WSet ws[NWS];
    DqT dq[NWS][NB][GPT];
    u32x4_t A[2][2][NB], B[2][2][MB];        // [set][u][nb] / [set][u][mb]

    // Block i (of DMB) of this wave's share of stage st's DMA.
    auto dma_part = [&](int st, auto buf, int i) __attribute__((always_inline)) {
        const int sc = min(st, S - 1);
        const uint32_t soff_k = (uint32_t)sc * 128u;
        uint32_t off;
        if constexpr (SH == 3) {
            uint32_t step = (uint32_t)i * xstep;
            asm volatile("" : "+s"(step));     // added here, not hoisted as 8 registers
            off = xoff[0] + step;
        } else {
            off = xoff[i];
        }
        if constexpr (RAG) off = sc * 64 + k_chunk < Kx ? off : 0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xrs, (__attribute__((address_space(3))) void *)&xs[decltype(buf)::value][(wave * DMB + i) * 64],
            16, off, soff_k, 0, 0);
    };
    auto dma = [&](int st, auto buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < DMB; ++i) dma_part(st, buf, i);
    };
    // Load j (of kWLoads) of weight tile t: the 2 NB code slots, then scales and zeros.
    auto load_w_part = [&](int t, WSet &w, auto J) __attribute__((always_inline)) {
        constexpr int j = decltype(J)::value;
        t = min(t, KTl - 1);
        if constexpr (j < 2 * NB * WV) {
            constexpr int nb = j / (2 * WV), u = (j / WV) % 2, v = j % WV;
            w.w[nb][u][v] = buf_load_b128(wrs, woff[nb][u], (t * WV + v) * 1024);
        } else {
            constexpr int m = j - 2 * NB * WV, per = SYM ? 1 : 2;
            constexpr int nb = m / (GPT * per), h = (m / per) % GPT, kind = m % per;
            if constexpr (kind == 0)
                w.s[nb][h] = buf_load_b32(srs, soff[nb], (t * GPT + h) * 32);
            else
                w.z[nb][h] = buf_load_b32(zrs, zoff[nb], (t * GPT + h) * zrow);
        }
    };
    auto load_w = [&](int t, WSet &w) __attribute__((always_inline)) {
        [&]<int... J>(std::integer_sequence<int, J...>) {
            (load_w_part(t, w, IC<J>()), ...);
        }(std::make_integer_sequence<int, kWLoads>{});
    };
    auto make_dq = [&](const WSet &w, DqT(&d)[NB][GPT]) __attribute__((always_inline)) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int h = 0; h < GPT; ++h)
                d[nb][h] = DqB::make((uint16_t)(w.s[nb][h] >> sshift),
                                     SYM ? zsym : ((w.z[nb][h] >> zshift) & zmask));
    };
    auto read_b = [&](auto buf, int s, u32x4_t(&b)[2][MB]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int mb = 0; mb < MA; ++mb)
                b[u][mb] = xs[decltype(buf)::value][mb * 256 + brow + ((4 * s + 2 * u) ^ cb)];
    };
    // The A operand of 32-deep step `word` of column block nb, k half u (compiler-scheduled
    // form, for the prologue).
    auto dq_word = [&](const WSet &w, int nb, int u, int word, const DqT &d) __attribute__((always_inline)) {
        if constexpr (BITS == 4)
            return DqB::word(w.w[nb][u][0][word], d);
        else
            return DqB::pair(w.w[nb][u][word / 2][2 * (word % 2)],
                                  w.w[nb][u][word / 2][2 * (word % 2) + 1], d);
    };
    auto dequant_a = [&](const WSet &w, const DqT(&d)[NB][GPT], int word, u32x4_t(&a)[2][NB]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                a[u][nb] = dq_word(w, nb, u, word, d[nb][(word * 32) / G]);
    };

    // Dequantization operations of the next step.  Four words (word q = (u, nb) = (q / 2,
    // q % 2)): operation o is step o / 4 of word o % 4.  Two words (q = u), and the four
    // words of the 256 x 256 tile (whose 32-MFMA steps put an MFMA between any two
    // operations anyway, and whose registers hold only one word's scratch values): word
    // 0's operations first, then word 1's, and so on.
    auto run_ops = [&](auto LO, auto HI, const WSet &wn, const DqT(&dn)[NB][GPT], int word_n,
                       DqTmp(&tmp)[2 * NB], u32x4_t(&an)[2][NB]) __attribute__((always_inline)) {
        constexpr int lo = decltype(LO)::value, hi = decltype(HI)::value;
        [&]<int... O>(std::integer_sequence<int, O...>) {
            (([&] {
                 constexpr int o = lo + O;
                 if constexpr (o < hi) {
                     constexpr bool rr = NB == 2 && SH != 3;     // round-robin
                     constexpr int q = rr ? o % 4 : o / Ops::kCount;
                     constexpr int op = rr ? o / 4 : o % Ops::kCount;
                     constexpr int u = q / NB, nb = q % NB;
                     if constexpr (BITS == 4)
                         Ops::template run<op>(wn.w[nb][u][0][word_n], dn[nb][(word_n * 32) / G],
                                               dc, tmp[q], an[u][nb]);
                     else
                         Ops::template run<op>(wn.w[nb][u][word_n / 2][2 * (word_n % 2)],
                                               wn.w[nb][u][word_n / 2][2 * (word_n % 2) + 1],
                                               dn[nb][(word_n * 32) / G], dc, tmp[q], an[u][nb]);
                 }
             }()),
             ...);
        }(std::make_integer_sequence<int, 8>{});
    };

    // One 32-deep step: MFMA i (u = i/8, nb = i/MB % NB, mb = i % MB) on the current
    // operands, then slice i of the next step's preparation.
    auto step = [&](const u32x4_t(&a)[2][NB], const u32x4_t(&b)[2][MB], u32x4_t(&an)[2][NB],
                    u32x4_t(&bn)[2][MB], const WSet &wn, const DqT(&dn)[NB][GPT], int word_n,
                    auto bufn, int s_n, auto hook) __attribute__((always_inline)) {
        DqTmp tmp[2 * NB];
        constexpr int kReadEvery = 8 / MB;   // 2 MB operand reads spread over 16 MFMAs
        [&]<int... I>(std::integer_sequence<int, I...>) {
            (([&] {
                 constexpr int u = I / 8, nb = (I / MB) % NB, mb = I % MB;
                 if constexpr (mb < MA) mfma32<ACT>(acc[nb][mb], a[u][nb], b[u][mb]);
                 if constexpr (I % kReadEvery == 0) {
                     constexpr int r = I / kReadEvery, ru = r / MB, rmb = r % MB;
                     if constexpr (rmb < MA)
                         bn[ru][rmb] = xs[decltype(bufn)::value][rmb * 256 + brow + ((4 * s_n + 2 * ru) ^ cb)];
                 }
                 constexpr int total = 2 * NB * Ops::kCount;
                 run_ops(IC<(total * I) / 16>(), IC<(total * (I + 1)) / 16>(), wn, dn, word_n, tmp, an);
                 hook(IC<I>());
                 __builtin_amdgcn_sched_barrier(0);
             }()),
             ...);
        }(std::make_integer_sequence<int, 16>{});
        // Keep this step's operands allocated to the end of the step, so no register of an
        // operand that an in-flight MFMA reads is handed to the next step's values.
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) asm volatile("" ::"v"(a[u][nb]));
#pragma unroll
            for (int mb = 0; mb < MA; ++mb) asm volatile("" ::"v"(b[u][mb]));
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // One 32-deep step of the 256 x 256 tile: 32 MFMAs, MFMA i on column block i % 2, row
    // block (i % 16) / 2 and k half i / 16, so each activation operand feeds two MFMAs in a
    // row.  Its activation operands are single-buffered (a second set would not fit beside
    // 256 accumulators): after MFMA 2r the step reads its own second-half operand of row
    // block r, whose register the previous step last read 15 MFMAs before, and after MFMA
    // 16 + 2r the next step's first-half operand of row block r, last read here 15 MFMAs
    // before.  The dequantization of the next step's four words is spread over the 32
    // MFMAs as in the other shapes.
    auto step_wide = [&](const u32x4_t(&a)[2][NB], u32x4_t(&b)[2][MB], u32x4_t(&an)[2][NB],
                         const WSet &wn, const DqT(&dn)[NB][GPT], int word_n, auto buf, int s,
                         auto bufn, int s_n, auto hook) __attribute__((always_inline)) {
        DqTmp tmp[2 * NB];
        constexpr int total = 2 * NB * Ops::kCount;
        [&]<int... I>(std::integer_sequence<int, I...>) {
            (([&] {
                 constexpr int u = I / 16, mb = (I % 16) / 2, nb = I % 2;
                 mfma32<ACT>(acc[nb][mb], a[u][nb], b[u][mb]);
                 if constexpr (I % 2 == 0) {
                     if constexpr (u == 0)
                         b[1][mb] = xs[decltype(buf)::value][mb * 256 + brow + ((4 * s + 2) ^ cb)];
                     else
                         b[0][mb] = xs[decltype(bufn)::value][mb * 256 + brow + ((4 * s_n) ^ cb)];
                 }
                 run_ops(IC<(total * I) / 32>(), IC<(total * (I + 1)) / 32>(), wn, dn, word_n,
                         tmp, an);
                 hook(IC<I>());
                 __builtin_amdgcn_sched_barrier(0);
             }()),
             ...);
        }(std::make_integer_sequence<int, 32>{});
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) asm volatile("" ::"v"(a[u][nb]));
        __builtin_amdgcn_sched_barrier(0);
    };

    // One 64-deep stage st (ring buffer BUF = st % XS, tile t = st / 2, half H = st % 2,
    // weight set TW = t % NWS): step 0 runs word 2H and prepares word 2H+1 from this
    // stage's buffer, and issues the DMA of stage st + XS - 1 into the buffer stage st - 1
    // read; step 1 runs word 2H+1 and prepares the next stage's first step (the next
    // tile's word 0 when H == 1).  Stage 2t loads tile t + NWS - 1 in step 1, except in the
    // final four stages (LAST), whose weight loads nothing would read.
    // The wait (WAITN, from stage_wait_loads): vmcnt counts a wave's loads in issue order,
    // so leaving in flight no more loads than the wave issued after its DMA of stage st+1
    // finds that stage in LDS.  DMAs write LDS, so the compiler neither moves them across
    // the barrier nor drops them; the weight loads it may move (their memory never
    // changes) or drop when dead, as in the final stages, which therefore issue none.  The
    // count takes weight loads only from the same pass of the stage loop, after the DMA in
    // program order; the build walks every launch path of the generated code and fails if
    // a wait could pass early.  Counting them lets a weight tile land up to XS - 2 stages
    // after it was requested instead of within the next step.
    auto stage = [&](int st, auto BUF, auto H, auto TW, auto LOADW, auto WAITN) __attribute__((always_inline)) {
        constexpr int buf = decltype(BUF)::value, h = decltype(H)::value, tw = decltype(TW)::value;
        constexpr int nbuf = (buf + 1) % XS, nw = (tw + 1) % NWS;
        constexpr bool loadw = decltype(LOADW)::value != 0;
        const int t = st >> 1;
        wait_vm_barrier<decltype(WAITN)::value>();
        // The DMA of stage st + XS - 1 (DMB blocks) and, in the first half of a tile, the
        // weight loads of tile t + NWS - 1 go out one at a time between MFMAs, instead of as
        // one burst per wave at the barrier.
        auto dma_hook = [&](auto I) __attribute__((always_inline)) {
            constexpr int i = decltype(I)::value;
            constexpr int every = NMF / DMB;
            if constexpr (i % every == 1) dma_part(st + XS - 1, IC<(buf + XS - 1) % XS>(), i / every);
        };
        auto w_hook = [&](auto I) __attribute__((always_inline)) {
            constexpr int i = decltype(I)::value;
            if constexpr (h == 0 && loadw) {
                if constexpr (kWLoads <= 8) {
                    if constexpr (i % 2 == 0 && i / 2 < kWLoads)
                        load_w_part(t + NWS - 1, ws[(tw + NWS - 1) % NWS], IC<i / 2>());
                } else {
                    if constexpr (i < kWLoads)
                        load_w_part(t + NWS - 1, ws[(tw + NWS - 1) % NWS], IC<i>());
                }
            }
        };
        if constexpr (SH == 3) {
            step_wide(A[0], B[0], A[1], ws[tw], dq[tw], 2 * h + 1, BUF, 0, BUF, 1, dma_hook);
            if (h == 1) {
                make_dq(ws[nw], dq[nw]);
                __builtin_amdgcn_sched_barrier(0);
                step_wide(A[1], B[0], A[0], ws[nw], dq[nw], 0, BUF, 1, IC<nbuf>(), 0, w_hook);
            } else {
                step_wide(A[1], B[0], A[0], ws[tw], dq[tw], 2, BUF, 1, IC<nbuf>(), 0, w_hook);
            }
        } else {
            step(A[0], B[0], A[1], B[1], ws[tw], dq[tw], 2 * h + 1, BUF, 1, dma_hook);
            if (h == 1) {
                make_dq(ws[nw], dq[nw]);
                __builtin_amdgcn_sched_barrier(0);
                step(A[1], B[1], A[0], B[0], ws[nw], dq[nw], 0, IC<nbuf>(), 0, w_hook);
            } else {
                step(A[1], B[1], A[0], B[0], ws[tw], dq[tw], 2, IC<nbuf>(), 0, w_hook);
            }
        }
    };
    // Stages st .. st+3 (tiles 2u, 2u+1 of a pass of the stage loop, u = 0 or 1); LAST: the
    // kernel's final four stages, a pass of their own.
    auto four = [&](int st, auto U, auto LAST) __attribute__((always_inline)) {
        constexpr int u = decltype(U)::value;
        constexpr bool last = decltype(LAST)::value != 0;
        constexpr int lw = last ? 0 : 1;
        constexpr int b = 4 * u;
        stage(st + 0, IC<(b + 0) % XS>(), IC<0>(), IC<(2 * u) % NWS>(), IC<lw>(),
              IC<stage_wait_loads(XS, DMB, kWLoads, b + 0, lw)>());
        stage(st + 1, IC<(b + 1) % XS>(), IC<1>(), IC<(2 * u) % NWS>(), IC<lw>(),
              IC<stage_wait_loads(XS, DMB, kWLoads, b + 1, lw)>());
        stage(st + 2, IC<(b + 2) % XS>(), IC<0>(), IC<(2 * u + 1) % NWS>(), IC<lw>(),
              IC<stage_wait_loads(XS, DMB, kWLoads, b + 2, lw)>());
        stage(st + 3, IC<(b + 3) % XS>(), IC<1>(), IC<(2 * u + 1) % NWS>(), IC<lw>(),
              IC<stage_wait_loads(XS, DMB, kWLoads, b + 3, lw)>());
    };

    // Prologue: stages 0 .. XS-2 in flight, tiles 0 .. NWS-2, then stage 0's first
    // operands.  The DMAs go first; the prologue's wait leaves at most their last XS - 2
    // stages in flight, so stage 0 has landed whatever the compiler does with the weight
    // loads.
    [&]<int... J>(std::integer_sequence<int, J...>) {
        (dma(J, IC<J>()), ...);
    }(std::make_integer_sequence<int, XS - 1>{});
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < NWS - 1; ++t) load_w(t, ws[t]);
    wait_vm_barrier<(XS - 2) * DMB>();
    make_dq(ws[0], dq[0]);
    read_b(IC<0>(), 0, B[0]);
    dequant_a(ws[0], dq[0], 0, A[0]);
    // The zeroed accumulators and the first operands were written by VALU / LDS reads
    // that the compiler waits for; pad before the first (inline-asm) MFMA reads them.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 4" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // S is a multiple of 4: passes of PASS stages (whole rotations of the ring and of the
    // weight sets), then, for eight-stage passes, a four-stage tail (a pass's first four
    // stages, so ring buffers and weight sets line up).
    // Each pass ends with mfma_drain, so whatever the compiler places after the loop (it
    // may copy accumulators between registers right at the loop exit) finds the inline-asm
    // MFMAs' results written.
    constexpr int PASS = (NWS == 4 || XS == 8) ? 8 : 4;
    int st = 0;
    for (; st + PASS <= S; st += PASS) {
        four(st, IC<0>(), IC<0>());
        if constexpr (PASS == 8) four(st + 4, IC<1>(), IC<0>());
        mfma_drain();
    }
    if constexpr (PASS == 8) {
        if (st < S) {
            four(st, IC<0>(), IC<1>());
            mfma_drain();
        }
    }
    // The last stages prefetched (redundant) LDS data; let every DMA land before the wave
    // can retire.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // Split tile: store this part's fp32 accumulators in register order (chunk i of the
    // lane's 32 four-float chunks at i * 256 + thread, so every store instruction writes
    // 1 KiB in one piece) and stop; x32_split_reduce_kernel adds the P parts afterwards.
    if (parts > 1) {
        constexpr int kChunksPerPart = BM * BN / 4;
        f32x4_t *dst = reinterpret_cast<f32x4_t *>(part) + (size_t)(sidx * P + sp) * kChunksPerPart;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int mb = 0; mb < MA; ++mb)          // rows past M: never read back
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    dst[((nb * MB + mb) * 4 + q) * kXThreads + tid] =
                        f32x4_t{acc[nb][mb][4 * q], acc[nb][mb][4 * q + 1], acc[nb][mb][4 * q + 2],
                                acc[nb][mb][4 * q + 3]};
        return;
    }
    // Epilogue through LDS.  Result element j of block (nb, mb) in lane l is
    // n = 32 nb + 8 (j / 4) + 4 (l / 32) + j % 4 of the wave's 32 NB columns and
    // m = 32 mb + l % 32: written out directly, every store would put 8 bytes into each of
    // 32 rows, and the memory system then writes partly filled lines back.  Instead the
    // workgroup's BM x BN result tile (64 KiB, rounded to the output format) goes into the
    // activation ring, free once every wave has passed the barrier, and comes back as
    // whole rows: each 16-byte store of a wave covers complete lines.  16-byte chunk c of
    // tile row r sits at chunk c ^ (r % 16), so the 8-byte writes of 16 rows and the
    // 16-byte reads of a row each spread over all 64 banks.
    __syncthreads();
    if constexpr (SH == 3) {
        // The 256 x 256 tile: its 256 accumulators leave no registers to round them in bulk,
        // so they go to LDS in fp32 straight from the accumulator registers, one 128-row
        // half of the tile (128 KiB, the whole ring) at a time, and are rounded as they
        // come back as whole rows.  16-byte chunk c (of 64) of half-tile row r sits at
        // chunk c ^ (r % 16), so the writes of 16 rows spread over all 64 banks.
        constexpr int CPR = BN / 4;              // 16-byte fp32 chunks per tile row
        constexpr int HR = BM / 2;               // rows per half
        static_assert(HR * BN * 4 == (int)sizeof(xs), "a half tile fills the ring");
        f32x4_t *ot = reinterpret_cast<f32x4_t *>(&xs[0][0]);
        const int n_blk = nt * BN;
        const bool aligned = (ldy & 7) == 0;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            if (hf == 1) __syncthreads();        // every read of the first half is done
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = wave * 16 + 8 * nb + 2 * q + (lane >> 5);
#pragma unroll
                    for (int mb = 0; mb < MB / 2; ++mb) {
                        const int r = mb * 32 + (lane & 31), b = hf * (MB / 2) + mb;
                        ot[r * CPR + (c ^ (r & 15))] =
                            f32x4_t{acc[nb][b][4 * q], acc[nb][b][4 * q + 1], acc[nb][b][4 * q + 2],
                                    acc[nb][b][4 * q + 3]};
                    }
                }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < HR * (CPR / 2) / kXThreads; ++i) {
                const int idx = i * kXThreads + tid;
                const int r = idx / (CPR / 2), cp = idx % (CPR / 2);   // 8 outputs per thread
                const int m = m_blk + hf * HR + r, n = n_blk + 8 * cp;
                if (m >= M || n >= Ny) continue;
                const u32x2_t lo = round4<ACT>(ot[r * CPR + ((2 * cp) ^ (r & 15))]);
                const u32x2_t hi = round4<ACT>(ot[r * CPR + ((2 * cp + 1) ^ (r & 15))]);
                const u32x4_t v = {lo[0], lo[1], hi[0], hi[1]};
                uint16_t *p = Y + (size_t)m * ldy + n;
                if (aligned && n + 8 <= Ny) {
                    *reinterpret_cast<u32x4_t *>(p) = v;
                } else {
                    const int avail = min(8, Ny - n);
                    for (int e = 0; e < avail; ++e) p[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
                }
            }
        }
    } else {
        constexpr int CPR = BN / 8;              // 16-byte chunks per tile row
        static_assert(BM * BN * 2 <= (int)sizeof(xs), "the result tile fits the ring");
        u32x2_t *ot = reinterpret_cast<u32x2_t *>(&xs[0][0]);
        const int half = lane >> 5;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = wave * 4 * NB + 4 * nb + q;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) {
                    const int r = mb * 32 + (lane & 31);
                    const f32x4_t v = {acc[nb][mb][4 * q], acc[nb][mb][4 * q + 1],
                                       acc[nb][mb][4 * q + 2], acc[nb][mb][4 * q + 3]};
                    ot[2 * (r * CPR + (c ^ (r & 15))) + half] = round4<ACT>(v);
                }
            }
        __syncthreads();
        const u32x4_t *oc = &xs[0][0];
        const int n_blk = nt * BN;
        const bool aligned = (ldy & 7) == 0;
#pragma unroll
        for (int i = 0; i < BM * CPR / kXThreads; ++i) {
            const int idx = i * kXThreads + tid;
            const int r = idx / CPR, c = idx % CPR;
            const int m = m_blk + r, n = n_blk + 8 * c;
            if (m >= M || n >= Ny) continue;
            const u32x4_t v = oc[r * CPR + (c ^ (r & 15))];
            uint16_t *p = Y + (size_t)m * ldy + n;
            if (aligned && n + 8 <= Ny) {
                *reinterpret_cast<u32x4_t *>(p) = v;
            } else {
                const int avail = min(8, Ny - n);
                for (int e = 0; e < avail; ++e) p[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
            }
        }
    }
}

// Y of the split tiles: the sum of their P fp32 partials, in split order (so results do not
// depend on which part ran first), rounded once to the output format.  NB MB workgroups per
// tile (8, or 16 for the 256 x 256 tile), four of a lane's 4 NB MB register-order chunks
// each: thread `tid` reads the four floats that
// thread `tid` of the main kernel wrote for each of its chunks -- all 4 P loads issued
// before the first add, so one memory round trip covers them -- and knows their (m, n)
// the same way.
template <int ACT, int SH>
__global__ __launch_bounds__(kXThreads) void x32_split_reduce_kernel(
    const f32x4_t *__restrict__ part, int full, int P, int M, int N, int Ny, int ldy,
    uint16_t *__restrict__ Y) {
    constexpr int NB = shape_nb(SH), MB = shape_mb(SH), BM = tile_m(SH), BN = tile_n(SH);
    constexpr int kChunksPerPart = BM * BN / 4;
    constexpr int kMaxParts = 8, kCpt = 4;     // parts, chunks per thread
    constexpr int kWgs = x32_reduce_wgs(SH);
    const int sidx = blockIdx.x / kWgs, c0 = (blockIdx.x % kWgs) * kCpt;
    int mt, nt;
    tile_of(full + sidx, (M + BM - 1) / BM, (N + BN - 1) / BN, mt, nt);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const f32x4_t *src = part + (size_t)sidx * P * kChunksPerPart + c0 * kXThreads + tid;
    f32x4_t v[kMaxParts][kCpt];
#pragma unroll
    for (int o = 0; o < kMaxParts; ++o)
#pragma unroll
        for (int j = 0; j < kCpt; ++j)
            if (o < P) v[o][j] = src[(size_t)o * kChunksPerPart + j * kXThreads];
#pragma unroll
    for (int j = 0; j < kCpt; ++j) {
        f32x4_t s = v[0][j];
#pragma unroll
        for (int o = 1; o < kMaxParts; ++o)
            if (o < P) s += v[o][j];
        const int i = c0 + j, nb = i / (4 * MB), mb = (i / 4) % MB, q = i % 4;
        const int n = nt * BN + wave * 32 * NB + nb * 32 + 8 * q + 4 * (lane >> 5);
        const int m = mt * BM + mb * 32 + (lane & 31);
        if (m < M && n < Ny) store4<ACT>(Y + (size_t)m * ldy + n, Ny - n, s);
    }
}

// Stage-loop length of the kernel: the packed K rounded up to a multiple of 256.
inline int x32_loop_k(int Kp) { return (Kp + 255) / 256 * 256; }

// Compute units of the current device (cached per device).
inline int device_cus() {
    static int cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cus[dev] = n;
    }
    return cus[dev];
}

// Fewer tiles than compute units.  One workgroup fills a compute unit (its registers take
// the whole SIMD), so T < CUs tiles leave CUs - T units idle.  Splitting each tile's K
// range P ways (T P <= CUs, P <= 8) runs the tiles in about 1/P of the time, for one fp32
// partial of the tile per part, written to the workspace (past its counter region, which
// the small-M kernels use) and added up by a second, small kernel.  Parts keep at least
// 1024 of K (the pipeline's prologue and epilogue stay small against the loop) and whole
// 256-deep blocks of the stage loop (so K = 5120, twenty blocks, splits five ways).  A partial last round of a larger grid is left alone:
// under the chip's power limit the busy units of such a round run at a higher clock, and
// splitting it (measured at 2048 x 4096 x 6144: 384 tiles) saved less than the partials
// cost.  MPGEMM_X32_SPLIT=0 turns the split off.
struct X32Split {
    int full, p;                             // tiles run whole; parts per remaining tile
};
inline X32Split x32_split(int tiles, int loop_k, bool rag, int cus) {
    X32Split sp{tiles, 1};
    if (rag || cus <= 0) return sp;
    if (const char *env = getenv("MPGEMM_X32_SPLIT"))
        if (env[0] == '0') return sp;
    if (tiles >= cus) return sp;
    const int r = tiles;
    for (int p = 8; p >= 2; --p)
        if (r * p <= cus && loop_k % (256 * p) == 0 && loop_k / p >= 1024) {
            sp.full = tiles - r;
            sp.p = p;
            break;
        }
    return sp;
}
inline size_t x32_split_bytes(const X32Split &sp, int tiles, int sh) {
    if (sp.p == 1) return 0;
    return kSplitCounterBytes + (size_t)(tiles - sp.full) * sp.p * tile_m(sh) * tile_n(sh) * 4;
}

// One launch of tile shape SH over the whole of `a` (with the K split of small grids).
template <int ACT, bool SYM, int G, int SH, int CODE, bool RAG>
void launch_tiles(const GemmArgs &a, hipStream_t stream) {
    const int tiles = ((a.Np + tile_n(SH) - 1) / tile_n(SH)) * ((a.M + tile_m(SH) - 1) / tile_m(SH));
    const int loop_k = x32_loop_k(a.Kp);
    X32Split sp = x32_split(tiles, loop_k, RAG, device_cus());
    const size_t need = x32_split_bytes(sp, tiles, SH);
    if (need > a.workspace_bytes || a.workspace == nullptr ||
        ((uintptr_t)a.workspace & 15u) != 0)
        sp = X32Split{tiles, 1};
    float *part = sp.p > 1 ? reinterpret_cast<float *>(static_cast<char *>(a.workspace) +
                                                       kSplitCounterBytes)
                           : nullptr;
    const dim3 grid((unsigned)(sp.full + (tiles - sp.full) * sp.p));
    // Row blocks that can hold rows below M: one tile row of a 256-row tile needs a quarter
    // of them up to 64 rows, half up to 128; one of a 128-row tile half up to 64.  (The
    // 256 x 256 tile always runs all eight.)
    constexpr int MB = shape_mb(SH);
    auto run = [&](auto MA) __attribute__((always_inline)) {
        prefill_x32_kernel<ACT, SYM, G, kXWSets<G, CODE>, SH, CODE, RAG, decltype(MA)::value>
            <<<grid, dim3(kXThreads), 0, stream>>>(a.X, a.codes, a.scales, a.zeros, a.M, a.Np,
                                                   loop_k, a.Kp, a.K, a.N, a.ldy ? a.ldy : a.N,
                                                   a.Y, sp.full, sp.p,
                                                   part);
    };
    if constexpr (SH == 1) {
        if (a.M <= 8 * MB) run(IC<MB / 4>());
        else if (a.M <= 16 * MB) run(IC<MB / 2>());
        else run(IC<MB>());
    } else if constexpr (SH == 2) {
        if (a.M <= 16 * MB) run(IC<MB / 2>());
        else run(IC<MB>());
    } else {
        run(IC<MB>());
    }
    if (sp.p > 1)
        x32_split_reduce_kernel<ACT, SH>
            <<<dim3((unsigned)(tiles - sp.full) * x32_reduce_wgs(SH)), dim3(kXThreads), 0,
               stream>>>(reinterpret_cast<const f32x4_t *>(part), sp.full, sp.p, a.M, a.Np, a.N,
                         a.ldy ? a.ldy : a.N, a.Y);
}

// Columns [n0, n1) of `a` (n0 a multiple of 16; n1 a multiple of 16 or a.N) as a GEMM of
// its own: the packed planes are strip-major (a 16-column strip's codes, scales and zeros
// are contiguous), so the range is an offset view of them and of Y, with Y's row stride.
inline GemmArgs column_range(const GemmArgs &a, int n0, int n1, int group, int bits) {
    GemmArgs r = a;
    const size_t strips = (size_t)(n0 / 16), groups = (size_t)(a.Kp / group);
    r.codes = a.codes + strips * (a.Kp / 128) * (64 * bits);     // 256 bits bytes per tile
    r.scales = a.scales + strips * groups * 16;
    r.zeros = a.zeros ? a.zeros + strips * groups * (16 * bits / 8) : nullptr;
    r.Y = a.Y + n0;
    r.ldy = a.ldy ? a.ldy : a.N;
    r.N = (n1 < a.N ? n1 : a.N) - n0;
    r.Np = (n1 < a.N ? n1 : a.Np) - n0;
    return r;
}

// The 256 x 256 tile with a last round that would fill at most half of the compute units
// runs its whole rounds over the leading columns and the remaining columns as one round of
// 256 x 128 tiles (a second launch, no partials): the half-empty round of 256 x 256 tiles
// took nearly a full round's time (Llama-3-8B gate_up at M = 2048: 896 tiles, 3.5 rounds).
// The first column of the 256 x 128 launch (0: one launch), for M rows, Np padded columns
// and `cus` compute units.
inline int wide_split_column(int M, int Np, int cus) {
    const int tm = (M + 255) / 256, tn = (Np + 255) / 256;
    const int rounds = cus > 0 ? tm * tn / cus : 0, rest = tm * tn - rounds * cus;
    if (rounds > 0 && rest > 0 && 2 * rest <= cus && cus % tm == 0)
        return rounds * (cus / tm) * 256;
    return 0;
}

template <int ACT, bool SYM, int G, int SH, int CODE, bool RAG>
void launch_one(const GemmArgs &a, hipStream_t stream) {
    if constexpr (SH == 3) {
        if (const int n1 = wide_split_column(a.M, a.Np, device_cus())) {
            launch_tiles<ACT, SYM, G, 3, CODE, RAG>(column_range(a, 0, n1, G, kCodeBits<CODE>),
                                                    stream);
            launch_tiles<ACT, SYM, G, 1, CODE, RAG>(column_range(a, n1, a.N, G, kCodeBits<CODE>),
                                                    stream);
            return;
        }
    }
    launch_tiles<ACT, SYM, G, SH, CODE, RAG>(a, stream);
}

template <int ACT, int SH, int CODE, bool RAG>
void launch_act(const GemmArgs &a, hipStream_t stream) {
    if constexpr (kCodeFp8<CODE>) {         // FP8 codes carry no zero point
        a.group == 128 ? launch_one<ACT, true, 128, SH, CODE, RAG>(a, stream)
                       : launch_one<ACT, true, 64, SH, CODE, RAG>(a, stream);
    } else {
        const bool sym = a.zeros == nullptr;
        if (a.group == 128) {
            sym ? launch_one<ACT, true, 128, SH, CODE, RAG>(a, stream)
                : launch_one<ACT, false, 128, SH, CODE, RAG>(a, stream);
        } else {
            sym ? launch_one<ACT, true, 64, SH, CODE, RAG>(a, stream)
                : launch_one<ACT, false, 64, SH, CODE, RAG>(a, stream);
        }
    }
}

// Every variant of code format CODE in tile shape SH.
template <int SH, int CODE>
void launch_x32(const GemmArgs &a, hipStream_t stream) {
    const bool rag = a.K != x32_loop_k(a.Kp);
    if (a.act == kBF16)
        rag ? launch_act<kBF16, SH, CODE, true>(a, stream) : launch_act<kBF16, SH, CODE, false>(a, stream);
    else
        rag ? launch_act<kF16, SH, CODE, true>(a, stream) : launch_act<kF16, SH, CODE, false>(a, stream);
}

}  // namespace

}  // namespace mpgemm
