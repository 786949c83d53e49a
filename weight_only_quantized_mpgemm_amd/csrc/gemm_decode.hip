// Small-M (decode) GEMM for gfx950: 2-, 3-, 4- and 8-bit integer codes and FP8 codes.
//
// [TurboMind, GEMM pipeline; Fig. 6 and Fig. 9 captions]: the packed low-bit weights are
// loaded straight into registers, turned into 16-bit values by I2F conversion and scaling,
// and fed to the matrix cores while later tiles' loads are in flight.  Source: "LMDeploy
// Accelerates Mixed-Precision LLM Inference with TurboMind" (arXiv 2508.15601).
//
// At M <= 64 the GEMM is bound by HBM bandwidth: every weight byte is read once and used
// for at most M multiply-adds, so the kernel is built around keeping the weight loads in
// flight and everything else off the vector-memory path.  Design for MI355X:
//   - a workgroup owns S adjacent 16-column strips and a range of the K tiles; its NW waves
//     split that range into contiguous slices (split-K inside the workgroup), and the K
//     range may be split over P workgroups too (grid.y).  The host picks S, NW and P by
//     shape (pick_split below);
//   - the workgroup's activations (M rows of its K range, a few KiB to 32 KiB) are read
//     once into LDS at the start, with 16-byte loads issued before any weight load, and
//     every MFMA takes its activation operand from LDS (ds_read_b128).  The weight path then
//     issues one 128-bit load per lane and tile (a wave reads 1 KiB contiguously) plus the
//     scale and zero words: on this chip the cost of a memory-bound pass is the number of
//     vector-memory instructions in flight, and per-wave activation loads (four per tile,
//     mostly out-of-range lanes at small M) had doubled it;
//   - each wave runs a D-slot register pipeline over its slice: slot s holds, for one
//     128-deep tile step, the S weight tiles and the raw scales/zeros; computing slot s is
//     followed by refilling it with the step D positions later, so D steps are always in
//     flight (a slice of at most D steps is requested entirely before the first compute).
//     Steps past the slice are not loaded, and a short tail computes the remaining slots;
//   - all global loads are buffer loads: fixed per-lane offsets, a wave-uniform scalar
//     offset per step.  Activation chunks past the matrix (rows past M, k past K) read as
//     zero without memory traffic;
//   - weights are the MFMA A operand (rows = n), activations the B operand (columns = m);
//   - the NW partial sums meet in LDS and are added in a fixed wave order;
//   - with P > 1 every workgroup of a strip group writes its fp32 partial to the workspace,
//     then bumps the group's counter; the workgroup that arrives last adds the P partials
//     in split order, stores Y and sets the counter back to zero.  Nobody waits for
//     anybody, the sum order is fixed (results are deterministic for a given split), and
//     the counters are left as they were found, so the workspace needs zeroing only once.
#include <stdio.h>
#include <stdlib.h>

#include <type_traits>

#include "kernels.hpp"

namespace mpgemm {

namespace {

constexpr int kMaxWaves = 8;
// 16-byte activation chunks each lane may load into LDS in the prologue, and scale or zero
// chunks; the host keeps the blocks within (kFillLoads or kMetaLoads) * 64 * NW chunks.
constexpr int kFillLoads = 4;
constexpr int kMetaLoads = 2;
// Activations go through LDS at M <= kXLdsMaxM: the workgroup's block of M rows is then
// small, and one copy replaces each wave's four 16-row fragment loads per tile.  Larger M
// loads each wave's fragments with the weights (a 16-row fragment is 4x a weight tile's
// bytes; the strips of a workgroup share it).
constexpr int kXLdsMaxM = 4;

// LDS layout of a workgroup (all sizes from the host's launch plan):
//   activation block (XL): M rows of 2^xlog 16-byte chunks plus 16 bytes of padding (so
//     the 16 rows one MFMA operand reads fall on distinct banks), chunk c of row m at
//     m * x_row_bytes + 16 c holding k = 128 k_lo + 8 c .. +7;
//   scales: per strip si, 2^mlog 16-byte chunks, group row r (of the K range) at 32 r;
//   zeros (asymmetric codes): per strip si, 2^(mlog-1) rows of zrow bytes.
// Once every wave is done with them, the same bytes hold the waves' partial sums.
__host__ __device__ constexpr uint32_t x_row_bytes(int xlog) { return (16u << xlog) + 16u; }
__host__ __device__ constexpr int ceil_log2(int v) {
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

template <int MB, int S, int WV, bool XL>
struct Slot {
    u32x4_t w[S][WV];          // per strip: WV 16-byte pieces of packed tile = 4 MFMA k-steps
    u32x4_t x[XL ? 1 : 4][XL ? 1 : MB];   // activation A operands (when not in LDS)
};

// Waves per SIMD a configuration is compiled for: four (128 registers) where the strips'
// dequantization constants and operands fit beside the pipeline, two (256) where the
// activation fragments travel in the pipeline slots or a wave works on four strips.
template <int MB, int S, bool SYM, int G, int CODE, bool XL>
constexpr int decode_waves() {
    if constexpr (!XL || S == 4) return 2;
    return 4;
}

// Slots in flight per wave (128-deep steps): what the register budget of the occupancy
// above holds beside the accumulators, the activation operands and the per-strip
// dequantization constants (and, where group sums are scaled in fp32, the group
// accumulators); 2 to 8 (at most 4 for four strips, 3 for four strips with bf16 group sums
// or with sub-4-bit codes in 64-deep groups, 2 for four strips of 8-bit codes, 3 with the
// activations in the slots, 2 there for 64-deep groups: more did not fit without spilling).
// bf16 activations with 4-bit codes scale group sums in fp32 too (g = 128, one or two row
// blocks: the per-group activation sums of more did not fit beside the pipeline).
template <int ACT, int MB, int G, int CODE>
constexpr bool fold_bf16() {
    return ACT == kBF16 && CODE == kU4 && G == 128 && MB <= 2;
}

template <int ACT, int MB, int S, bool SYM, int G, int CODE, bool XL>
constexpr int pipeline_depth() {
    constexpr int bits = kCodeBits<CODE>;
    constexpr int regs = 512 / decode_waves<MB, S, SYM, G, CODE, XL>();
    constexpr int slot = S * (bits > 4 ? 8 : 4) + (XL ? 0 : 16 * MB);
    constexpr bool fold = CODE == kU4 || CODE == kU8;     // (8-bit: fp16 activations only)
    constexpr int fixed = 8 * S * MB + (XL ? 16 * MB : 0) + 3 * S * (kTileK / G) +
                          (bits < 4 ? 16 : 0) + (fold ? 8 * S * MB + 4 * S * (kTileK / G) : 0) +
                          64;
    constexpr int cap = !XL ? (G == 64 ? 2 : 3)
                            : (S == 4 ? (bits > 4 ? 2
                                         : fold_bf16<ACT, MB, G, CODE>() || (bits < 4 && G == 64)
                                             ? 3
                                             : 4)
                                      : 8);
    constexpr int d = (regs - fixed) / slot;
    return d > cap ? cap : (d < 2 ? 2 : d);
}

template <int ACT, int MB, int S, bool SYM, int G, int D, int CODE, bool XL>
__global__ __launch_bounds__(kMaxWaves * 64)
__attribute__((amdgpu_waves_per_eu(decode_waves<MB, S, SYM, G, CODE, XL>()))) void decode_kernel(
    const uint16_t *__restrict__ X, const uint32_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros, int M, int N, int K,
    int Kx, int Ny, uint16_t *__restrict__ Y, f32x4_t *__restrict__ part,
    uint32_t *__restrict__ cnt, int xlog, int mlog) {
    // N, K: the padded matrix of the packed planes; Kx: activation row length (the user K,
    // <= K); Ny: output row length (the user N, <= N).  Activations at k >= Kx read as zero.
    // xlog, mlog: log2 of the activation chunks per row and scale chunks per strip of the
    // LDS layout (at least the largest K range of any workgroup needs).
    constexpr int GPT = kTileK / G;              // groups per 128-k tile (1 or 2)
    // 128-bit pieces per lane and strip per 128-deep step: one 16 x 128 tile of 4-bit codes,
    // two 16 x 64 tiles of 8-bit codes; 2- and 3-bit codes fill 8 or 12 bytes of one piece.
    constexpr int BITS = kCodeBits<CODE>;
    constexpr int WV = BITS >= 4 ? BITS / 4 : 1;
    constexpr uint32_t kTileBytes = 256u * BITS;       // one 16 x 128 tile of the strip
    constexpr uint32_t kLaneBytes = BITS >= 4 ? 16u : 4u * BITS;
    constexpr bool kNibbleZeros = BITS <= 4;           // zeros stored as 4-bit values
    constexpr int zrow = kNibbleZeros ? 8 : 16;        // zero bytes per (strip, group)
    // fp16 activations with 4- or 8-bit integer codes: the MFMAs take the exact q - z and
    // each group's sum is scaled in fp32 (see dequant_word_f16_int).  bf16 activations with
    // 4-bit codes: the MFMAs take the exact 128 + q, and each group's sum less (128 + z)
    // times the group's activation sum (one more MFMA per step against a block of ones,
    // shared by the strips) is scaled in fp32 (see dequant_word_bf16_biased).
    constexpr bool kFoldB = fold_bf16<ACT, MB, G, CODE>();
    constexpr bool kFold = (ACT == kF16 && (CODE == kU4 || CODE == kU8)) || kFoldB;
    typedef Slot<MB, S, WV, XL> SlotT;
    extern __shared__ __align__(16) uint8_t lds[];

    const int NW = blockDim.x >> 6;
    // The wave index is uniform across the wave; saying so keeps the K-slice bounds, the
    // loop counter and every per-step scalar offset in scalar registers (otherwise each
    // buffer load would be wrapped in a loop over distinct offsets).
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int KT = K >> 7;
    // This workgroup's K range (split p of P), then this wave's share of it.
    const int P = gridDim.y, p = blockIdx.y;
    const int k_lo = (KT * p) / P, k_n = (KT * (p + 1)) / P - k_lo;
    const int t_begin = k_lo + (k_n * wave) / NW;
    const int n = k_lo + (k_n * (wave + 1)) / NW - t_begin;
    const int groups = K / G;
    const int strips = N >> 4;
    const int strip0 = blockIdx.x * S;
    const uint32_t xrow = x_row_bytes(xlog);
    const uint32_t meta0 = XL ? (uint32_t)M * xrow : 0u;                 // scales
    const uint32_t zeros0 = meta0 + ((uint32_t)S << mlog) * 16u;          // zeros
    const uint32_t zstrip = ((uint32_t)zrow << (mlog - 1));               // zero bytes / strip
    f32x4_t *red = reinterpret_cast<f32x4_t *>(lds);

    const rsrc_t wrs = make_rsrc(codes, (uint32_t)((size_t)strips * KT * kTileBytes));
    const rsrc_t xrs = make_rsrc(X, (uint32_t)((size_t)M * Kx * 2));
    const rsrc_t srs = make_rsrc(scales, (uint32_t)((size_t)groups * N * 2));
    const rsrc_t zrs = make_rsrc(zeros, (uint32_t)((size_t)groups * N / (kNibbleZeros ? 2 : 1)));
    const int nthreads = (int)blockDim.x;

    // Prologue fill, issued before any weight load (their LDS writes come after the weight
    // loads, so waiting for the fill does not wait for any weight):
    //  - activation block (XL): chunk c is row c >> xlog, 16-byte column c & (2^xlog - 1);
    //    columns past the workgroup's K range (or past the matrix) read as zero;
    //  - scales: strip si's k_n * GPT group rows are 32 * k_n * GPT contiguous bytes of the
    //    meta plane (strip-major), two 16-byte chunks per row;
    //  - zeros (asymmetric codes): zrow contiguous bytes per group row, one chunk each.
    const int xchunks = XL ? M << xlog : 0;
    const int fill_iters = __builtin_amdgcn_readfirstlane((xchunks + nthreads - 1) / nthreads);
    u32x4_t fx[kFillLoads];
#pragma unroll
    for (int it = 0; it < kFillLoads; ++it) {
        if (it < fill_iters) {
            const int c = threadIdx.x + it * nthreads;
            const int m = c >> xlog, cc = c & ((1 << xlog) - 1);
            const int k = k_lo * kTileK + cc * 8;
            const bool in = c < xchunks && cc < k_n * 16 && k < Kx;
            fx[it] = buf_load_b128(xrs, in ? (uint32_t)(m * Kx + k) * 2u : 0x80000000u, 0);
        }
    }
    const int mrows = k_n * GPT;                       // group rows per strip
    const int schunks = S << mlog;
    const int meta_iters = __builtin_amdgcn_readfirstlane((schunks + nthreads - 1) / nthreads);
    u32x4_t fs[kMetaLoads];
    u32x2_t fz8[kMetaLoads];
    u32x4_t fz16[kMetaLoads];
#pragma unroll
    for (int it = 0; it < kMetaLoads; ++it) {
        if (it < meta_iters) {
            const int c = threadIdx.x + it * nthreads;
            {
                const int si = c >> mlog, r = c & ((1 << mlog) - 1);
                const uint32_t strip = (uint32_t)min(strip0 + si, strips - 1);
                const uint32_t src = (strip * groups + k_lo * GPT) * 32u + (uint32_t)r * 16u;
                const bool in = c < schunks && r < mrows * 2;
                fs[it] = buf_load_b128(srs, in ? src : 0x80000000u, 0);
            }
            if constexpr (!SYM) {
                const int si = c >> (mlog - 1), r = c & ((1 << (mlog - 1)) - 1);
                const uint32_t strip = (uint32_t)min(strip0 + si, strips - 1);
                const uint32_t src = (strip * groups + k_lo * GPT + r) * (uint32_t)zrow;
                const bool in = c < (S << (mlog - 1)) && r < mrows;
                if constexpr (kNibbleZeros)
                    fz8[it] = buf_load_b64(zrs, in ? src : 0x80000000u, 0);
                else
                    fz16[it] = buf_load_b128(zrs, in ? src : 0x80000000u, 0);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // Per-lane byte offsets, fixed for the whole K slice.  Strips past N read the last real
    // strip (their outputs are never stored).
    uint32_t woff[S];
#pragma unroll
    for (int si = 0; si < S; ++si) {
        const uint32_t strip = (uint32_t)min(strip0 + si, strips - 1);
        woff[si] = (strip * KT + t_begin) * kTileBytes + lane * kLaneBytes;
    }
    constexpr uint32_t zmask = (1u << BITS) - 1;
    constexpr uint32_t zsym = 1u << (BITS - 1);        // symmetric zero: 2, 4, 8 or 128
    // Activation operand (MFMA A) of row block mb: row mb * 16 + lane % 16, k = 8 (lane / 16)
    // of each 32-deep step.  From LDS (XL; rows past M repeat row M - 1, whose outputs are
    // never stored) or from global memory (rows past M read as zero).
    uint32_t xlds[MB], xoff[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        xlds[mb] = (uint32_t)min(mb * 16 + (lane & 15), M - 1) * xrow + (lane >> 4) * 16u;
        xoff[mb] = ((uint32_t)(mb * 16 + (lane & 15)) * Kx + t_begin * kTileK + (lane >> 4) * 8) * 2u;
    }
    const int k_lane = t_begin * kTileK + (lane >> 4) * 8;
    const bool ragged = Kx != K;

    auto load = [&](SlotT &sl, int i) {
#pragma unroll
        for (int si = 0; si < S; ++si) {
            if constexpr (BITS == 2) {
                const u32x2_t v = buf_load_b64(wrs, woff[si], i * kTileBytes);
                sl.w[si][0] = u32x4_t{v.x, v.y, 0u, 0u};
            } else if constexpr (BITS == 3) {
                sl.w[si][0] = buf_load_b96(wrs, woff[si], i * kTileBytes);
            } else {
#pragma unroll
                for (int v = 0; v < WV; ++v)
                    sl.w[si][v] = buf_load_b128(wrs, woff[si], i * kTileBytes + v * 1024);
            }
        }
        if constexpr (!XL) {
            // The lane's 8-element chunk of 32-deep step j of tile t_begin + i starts at
            // k = k_lane + 128 i + 32 j; chunks at or past Kx take an offset outside the
            // activation descriptor, which reads as zero.
            const bool mask = ragged && (t_begin + i + 1) * kTileK > Kx;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool in = !mask || k_lane + i * kTileK + 32 * j < Kx;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    sl.x[j][mb] = buf_load_b128(xrs, in ? xoff[mb] : 0x80000000u,
                                                (i * kTileK + 32 * j) * 2);
            }
        }
    };

    f32x4_t acc[S][MB];
#pragma unroll
    for (int si = 0; si < S; ++si)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[si][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Step i of the wave's slice: tile t_begin + i, whose activations start at byte
    // (t_begin + i - k_lo) * 256 of every row of the block and whose meta rows are
    // (t_begin + i - k_lo) * GPT + h of each strip.  Weights are the MFMA B operand (column
    // n = lane % 16), activations the A operand, so each lane's results are rows
    // 4 (lane / 16) + r of its own weight column, whose scale the lane holds.
    auto compute = [&](const SlotT &sl, int i) {
        const int tl = t_begin + i - k_lo;
        u32x4_t xv[4][MB];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                if constexpr (XL)
                    xv[j][mb] = *reinterpret_cast<const u32x4_t *>(
                        lds + xlds[mb] + (uint32_t)tl * (kTileK * 2) + j * 64u);
                else
                    xv[j][mb] = sl.x[j][mb];
            }
        typedef DqFor<ACT, CODE> DqB;
        typename DqB::type dq[S][GPT];
        float sf[S][GPT], zf[S][GPT];
#pragma unroll
        for (int si = 0; si < S; ++si)
#pragma unroll
            for (int h = 0; h < GPT; ++h) {
                const uint32_t row = (uint32_t)(tl * GPT + h);
                const uint16_t sv = *reinterpret_cast<const uint16_t *>(
                    lds + meta0 + ((uint32_t)si << mlog) * 16u + row * 32u + (lane & 15) * 2);
                uint32_t zv = zsym;
                if constexpr (!SYM) {
                    const uint32_t zb = zeros0 + si * zstrip + row * zrow;
                    if constexpr (kNibbleZeros)
                        zv = (lds[zb + ((lane & 15) >> 1)] >> ((lane & 1) * 4)) & zmask;
                    else
                        zv = lds[zb + (lane & 15)];
                }
                if constexpr (!kFoldB) dq[si][h] = DqB::make(sv, zv);
                sf[si][h] = (float)bitcast<_Float16>(sv);
                zf[si][h] = -(128.0f + (float)zv);
            }
        if constexpr (kFold) {
            // Per strip and group: the MFMAs sum x * (q - z) (bf16: x * (128 + q)), products
            // exact, into a fresh accumulator, which is then added to the output scaled by
            // the group's s (bf16: after adding -(128 + z) times the group's activation sums,
            // which take the same output layout from MFMAs against ones).
            f32x4_t xs[kFoldB ? GPT : 1][MB];
            if constexpr (kFoldB) {
                const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
                for (int h = 0; h < GPT; ++h)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        xs[h][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int j = h * (4 / GPT); j < (h + 1) * (4 / GPT); ++j)
                            xs[h][mb] = mfma16x16x32<ACT>(xv[j][mb], ones, xs[h][mb]);
                    }
            }
#pragma unroll
            for (int si = 0; si < S; ++si)
#pragma unroll
                for (int h = 0; h < GPT; ++h) {
                    f32x4_t ag[MB];
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) ag[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = h * (4 / GPT); j < (h + 1) * (4 / GPT); ++j) {
                        u32x4_t b;
                        if constexpr (kFoldB)
                            b = dequant_word_bf16_biased(sl.w[si][0][j]);
                        else if constexpr (BITS == 4)
                            b = dequant_word_f16_int(sl.w[si][0][j], dq[si][h].nz_hi2,
                                                     dq[si][h].nz_lo2);
                        else
                            b = dequant_pair_w8_f16_int(sl.w[si][j / 2][2 * (j % 2)],
                                                        sl.w[si][j / 2][2 * (j % 2) + 1],
                                                        dq[si][h].nz_hi2);
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
                            ag[mb] = mfma16x16x32<ACT>(xv[j][mb], b, ag[mb]);
                    }
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            float g = ag[mb][r];
                            if constexpr (kFoldB) g = __builtin_fmaf(zf[si][h], xs[h][mb][r], g);
                            acc[si][mb][r] = __builtin_fmaf(sf[si][h], g, acc[si][mb][r]);
                        }
                }
        } else if constexpr (BITS < 4) {
            // Sub-4-bit codes: the four steps' operands of one strip at a time.  fp16: the
            // exact q - z, each group's sum scaled by its s in fp32 as above.
#pragma unroll
            for (int si = 0; si < S; ++si) {
                u32x4_t at[4];
                const typename DqB::type *d[4] = {&dq[si][0], &dq[si][32 / G], &dq[si][64 / G],
                                                  &dq[si][96 / G]};
                if constexpr (ACT == kF16) {
                    DqB::tile_int(sl.w[si][0], d, at);
#pragma unroll
                    for (int h = 0; h < GPT; ++h) {
                        f32x4_t ag[MB];
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb) ag[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int j = h * (4 / GPT); j < (h + 1) * (4 / GPT); ++j)
#pragma unroll
                            for (int mb = 0; mb < MB; ++mb)
                                ag[mb] = mfma16x16x32<ACT>(xv[j][mb], at[j], ag[mb]);
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                acc[si][mb][r] =
                                    __builtin_fmaf(sf[si][h], ag[mb][r], acc[si][mb][r]);
                    }
                } else {
                    DqB::tile(sl.w[si][0], d, at);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
                            acc[si][mb] = mfma16x16x32<ACT>(xv[j][mb], at[j], acc[si][mb]);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int si = 0; si < S; ++si) {
                    u32x4_t b;
                    if constexpr (BITS == 4)
                        b = DqB::word(sl.w[si][0][j], dq[si][(j * 32) / G]);
                    else
                        b = DqB::pair(sl.w[si][j / 2][2 * (j % 2)],
                                      sl.w[si][j / 2][2 * (j % 2) + 1], dq[si][(j * 32) / G]);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[si][mb] = mfma16x16x32<ACT>(xv[j][mb], b, acc[si][mb]);
                }
        }
    };

    SlotT slot[D];
#pragma unroll
    for (int s = 0; s < D; ++s) {
        if (s < n) load(slot[s], s);
        __builtin_amdgcn_sched_barrier(0);       // same load order as the loop's refills
    }
    // The prologue's blocks land in LDS (waiting only for their own loads, issued first).
#pragma unroll
    for (int it = 0; it < kFillLoads; ++it)
        if (it < fill_iters) {
            const int c = threadIdx.x + it * nthreads;
            if (c < xchunks)
                *reinterpret_cast<u32x4_t *>(lds + (uint32_t)(c >> xlog) * xrow +
                                             (uint32_t)(c & ((1 << xlog) - 1)) * 16u) = fx[it];
        }
#pragma unroll
    for (int it = 0; it < kMetaLoads; ++it) {
        if (it < meta_iters) {
            const int c = threadIdx.x + it * nthreads;
            if (c < schunks) *reinterpret_cast<u32x4_t *>(lds + meta0 + (uint32_t)c * 16u) = fs[it];
            if constexpr (!SYM) {
                if (c < (S << (mlog - 1))) {
                    if constexpr (kNibbleZeros)
                        *reinterpret_cast<u32x2_t *>(lds + zeros0 + (uint32_t)c * 8u) = fz8[it];
                    else
                        *reinterpret_cast<u32x4_t *>(lds + zeros0 + (uint32_t)c * 16u) = fz16[it];
                }
            }
        }
    }
    __syncthreads();

    if (n > 0) {
        const int n_main = n - n % D;
        for (int base = 0; base < n_main; base += D) {
#pragma unroll
            for (int s = 0; s < D; ++s) {
                // The barriers pin the order compute(s), refill(s), compute(s+1), ...: the
                // scheduler would otherwise sink every refill to the end of the batch and
                // the next batch would wait for all of them at once.  Steps past the slice
                // are not loaded (a wave-uniform branch).
                compute(slot[s], base + s);
                __builtin_amdgcn_sched_barrier(0);
                if (base + D + s < n) load(slot[s], base + D + s);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        const int rest = n - n_main;
#pragma unroll
        for (int s = 0; s < D - 1; ++s)
            if (s < rest) compute(slot[s], n_main + s);
    }

    // Lane l holds rows mb * 16 + 4 (l / 16) + r of column strip * 16 + l % 16.
    auto store_y = [&](int si, int mb, const f32x4_t &v) {
        const int col = (strip0 + si) * 16 + (lane & 15);
        if (col >= Ny) return;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = mb * 16 + 4 * (lane >> 4) + r;
            if (m < M) Y[(size_t)m * Ny + col] = round1<ACT>(v[r]);
        }
    };
    // Partials of block b (strip si = b / MB, row block mb = b % MB) of split q travel with
    // device-scope cache policy (sc1): the stores write through this XCD's L2 and the loads
    // bypass stale L2 lines, so no L2-wide writeback/invalidate fence is needed (those cost
    // far more than the partials themselves).
    const rsrc_t prs = make_rsrc(part, P > 1 ? (uint32_t)(gridDim.x * P * S * MB * 1024u) : 0u);
    auto part_off = [&](int q, int b) -> uint32_t {
        return (((blockIdx.x * P + q) * (S * MB) + b) * 64 + lane) * 16u;
    };
    auto put_part = [&](int q, int b, const f32x4_t &v) {
        buf_store_b128_device(prs, part_off(q, b), bitcast<u32x4_t>(v));
    };
    auto get_part = [&](int q, int b) -> f32x4_t {
        return bitcast<f32x4_t>(buf_load_b128_device(prs, part_off(q, b)));
    };
    if (NW == 1 && P == 1) {
#pragma unroll
        for (int si = 0; si < S; ++si)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) store_y(si, mb, acc[si][mb]);
        return;
    }
    if (NW == 1) {
#pragma unroll
        for (int si = 0; si < S; ++si)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) put_part(p, si * MB + mb, acc[si][mb]);
    } else {
        __syncthreads();                         // every wave is done with the LDS blocks
#pragma unroll
        for (int si = 0; si < S; ++si)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
                red[((wave * S + si) * MB + mb) * 64 + lane] = acc[si][mb];
        __syncthreads();
        for (int b = wave; b < S * MB; b += NW) {
            f32x4_t sum = red[b * 64 + lane];
            for (int w2 = 1; w2 < NW; ++w2) sum += red[(w2 * S * MB + b) * 64 + lane];
            if (P == 1)
                store_y(b / MB, b % MB, sum);
            else
                put_part(p, b, sum);
        }
        if (P == 1) return;
    }
    // Split-K fixup: each wave waits until its partial stores are acknowledged at device
    // scope, the workgroup meets, and one thread counts it in.  The last arriver's
    // device-scope loads are issued after it has seen every other workgroup's count, hence
    // after their stores completed.
    __shared__ uint32_t is_last;
    wait_vmem();
    __syncthreads();
    if (threadIdx.x == 0)
        is_last = __hip_atomic_fetch_add(&cnt[blockIdx.x], 1u, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(P - 1);
    __syncthreads();
    if (!is_last) return;
    for (int b = wave; b < S * MB; b += NW) {
        f32x4_t sum = get_part(0, b);
        for (int q = 1; q < P; ++q) sum += get_part(q, b);
        store_y(b / MB, b % MB, sum);
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&cnt[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workspace of a split: a fixed region of counters (one per strip group) at the start, then
// one 1 KiB fp32 block per (strip, row block, split).  The counter region has the same size
// for every shape, so partials of one call never land on counters of another call that
// shares the workspace (counters must read zero at every call's start).
constexpr size_t kCounterBytes = kSplitCounterBytes;
constexpr int kMaxGroups = (int)(kCounterBytes / 4);
constexpr size_t kMaxLds = 64 * 1024;         // per workgroup: two workgroups per CU

// Strips per workgroup (S), waves per workgroup (NW) and workgroups per strip group along
// K (P).  S > 1 lets one activation block in LDS feed S strips; NW and P split K inside and
// across workgroups.  MPGEMM_DECODE_SPLIT="S,NW" or "S,NW,P" overrides the choice for
// tuning sweeps (S in {1,2,4} with one row block, {1,2} with two, 1 above; NW in 1..8;
// P in 1..64); choices whose activation block does not fit are widened in P.
struct Split {
    int s, nw, p;
};

// Activations through LDS (XL) for one row block of at most kXLdsMaxM rows.
inline bool split_xl(int M, int mblocks) { return mblocks == 1 && M <= kXLdsMaxM; }
// log2 of the activation chunks per LDS row and of the scale chunks per strip, for the
// largest K range (kw tiles) of the launch.
inline int split_xlog(int kw) { return ceil_log2(kw * 16); }
inline int split_mlog(int kw, int group) { return ceil_log2(kw * (kTileK / group) * 2); }

// LDS bytes of a launch: the activation block (XL), scales and zeros, or the waves' partial
// sums where those are larger (they reuse the same bytes).  Zero rows are counted at their
// widest (8-bit codes), so the split, and with it the workspace, is the same for every
// code format.
size_t split_lds(const Split &sp, int M, int KT, int mblocks, int group) {
    const int kw = (KT + sp.p - 1) / sp.p;
    const size_t x = split_xl(M, mblocks) ? (size_t)M * x_row_bytes(split_xlog(kw)) : 0;
    const size_t meta = ((size_t)sp.s << split_mlog(kw, group)) * (16 + 8);
    const size_t red = sp.nw > 1 ? (size_t)sp.nw * sp.s * mblocks * 1024 : 0;
    return x + meta > red ? x + meta : red;
}

// The blocks fit in LDS and in the prologue's loads (kFillLoads activation and kMetaLoads
// scale or zero chunks per lane).
bool split_fits(const Split &sp, int M, int KT, int mblocks, int group) {
    const int kw = (KT + sp.p - 1) / sp.p;
    const int64_t lanes = (int64_t)64 * sp.nw;
    const int64_t xchunks = split_xl(M, mblocks) ? (int64_t)M << split_xlog(kw) : 0;
    const int64_t mchunks = (int64_t)sp.s << split_mlog(kw, group);
    return split_lds(sp, M, KT, mblocks, group) <= kMaxLds &&
           xchunks <= kFillLoads * lanes && mchunks <= kMetaLoads * lanes;
}

// Measured on MI355X (cold weights, the Llama-3-8B, Llama-3-70B and Qwen3-32B projection
// shapes; sweeps over S, NW and P):
//   - activations in LDS, one row: one strip per workgroup and no K split over workgroups
//     was best or within 5% everywhere, with eight waves where the strips alone give fewer
//     than 2048 waves and four otherwise;
//   - activations in LDS, three or four rows and at least 16384 strip tiles: two strips and
//     four waves (at M = 4: Qwen3-32B gate_up 38.0 us against 45.3, down 24.3 against 29.2;
//     Llama-3-70B gate_up 64.8 against 76.3); on smaller matrices and at two rows that
//     halved the waves of too few workgroups (Llama-3-8B O at M = 4: 8.3 us against 6.1);
//   - per-wave activation fragments: one strip and eight waves up to 256 strips
//     (Llama-3-8B O at M = 16: 7.6 us against 8.4 with two strips, for 2-, 3- and 4-bit
//     codes alike), two strips and eight waves up to 512, four strips and eight waves below
//     1024 (Qwen3-32B and Llama-3-70B QKV, 640 strips, at M = 16: 13.2 and 18.0 us against
//     16.1 and 23.8), four strips and four waves for wider matrices (five waves, the K / 8
//     rule at K = 5120, was 1.5x slower); long K split over about 256 workgroups, with eight
//     waves up to 8 rows (Llama-3-8B down at M = 8: 12.0 us against 14.4 with four; four
//     strips from 512 strips, Llama-3-70B down at M = 8: 28.6 against 32.8 with two) and four
//     above.
Split pick_split(int M, int strips, int KT, int mblocks, int group) {
    Split sp{1, 1, 1};
    if (split_xl(M, mblocks)) {
        if (M >= 3 && (int64_t)strips * KT >= 16384) {
            sp.s = 2;
            sp.nw = 4;
        } else {
            sp.nw = strips * 4 < 2048 ? 8 : 4;
        }
    } else if (mblocks == 1) {
        if (strips >= 1024) {
            sp.s = 4;
            sp.nw = 4;
        } else if (KT > 64) {
            sp.s = M > 8 || strips >= 512 ? 4 : 2;
            const int groups = (strips + sp.s - 1) / sp.s;
            sp.p = (256 + groups - 1) / groups;
            if (sp.p > 8) sp.p = 8;
            sp.nw = M > 8 ? 4 : 8;
        } else if (strips <= 256) {
            sp.s = 1;
            sp.nw = 8;
        } else if (strips > 512) {
            sp.s = 4;
            sp.nw = 8;
        } else {
            sp.s = 2;
            sp.nw = 8;
        }
    } else {
        sp.s = mblocks == 2 && strips >= 512 ? 2 : 1;
        sp.nw = KT / 8;
        if (KT > 64 && strips < 1024 && mblocks == 2) {
            sp.s = 2;
            const int groups = (strips + sp.s - 1) / sp.s;
            sp.p = (256 + groups - 1) / groups;
            if (sp.p > 8) sp.p = 8;
            sp.nw = 4;
        }
    }
    if (sp.nw > kMaxWaves) sp.nw = kMaxWaves;
    if (sp.nw > KT) sp.nw = KT;
    if (sp.nw < 1) sp.nw = 1;
    if (const char *env = getenv("MPGEMM_DECODE_SPLIT")) {
        int s = 0, nw = 0, p = 1;
        const int got = sscanf(env, "%d,%d,%d", &s, &nw, &p);
        if (got >= 2 && (s == 1 || s == 2 || s == 4) && nw >= 1 && nw <= kMaxWaves &&
            p >= 1 && p <= 64 && nw * p <= KT && (s == 1 || mblocks <= 2) &&
            (s < 4 || mblocks == 1)) {
            sp.s = s;
            sp.nw = nw;
            sp.p = got == 3 ? p : 1;
        }
    }
    // Widen P until the blocks fit (each part holds fewer tiles).
    while (!split_fits(sp, M, KT, mblocks, group) && sp.p < KT) ++sp.p;
    if ((strips + sp.s - 1) / sp.s > kMaxGroups) sp.p = 1;     // more groups than counters
    return sp;
}

size_t split_workspace(const Split &sp, int strips, int mblocks) {
    if (sp.p == 1) return 0;
    const size_t groups = (size_t)(strips + sp.s - 1) / sp.s;
    return kCounterBytes + groups * sp.p * sp.s * mblocks * 64 * sizeof(f32x4_t);
}

template <int ACT, int MB, int S, bool SYM, int G, int CODE, bool XL>
void launch_s(const GemmArgs &a, const Split &sp, hipStream_t stream) {
    constexpr int D = pipeline_depth<ACT, MB, S, SYM, G, CODE, XL>();
    const int strips = a.Np >> 4;
    const int wgs = (strips + S - 1) / S;
    const int KT = a.Kp >> 7;
    const int kw = (KT + sp.p - 1) / sp.p;
    const size_t lds = split_lds(sp, a.M, KT, MB, G);
    uint32_t *cnt = nullptr;
    f32x4_t *part = nullptr;
    if (sp.p > 1) {
        cnt = static_cast<uint32_t *>(a.workspace);
        part = reinterpret_cast<f32x4_t *>(static_cast<char *>(a.workspace) + kCounterBytes);
    }
    decode_kernel<ACT, MB, S, SYM, G, D, CODE, XL>
        <<<dim3(wgs, sp.p), dim3(sp.nw * 64), lds, stream>>>(
            a.X, a.codes, a.scales, a.zeros, a.M, a.Np, a.Kp, a.K, a.N, a.Y, part, cnt,
            split_xlog(kw), split_mlog(kw, G));
}

template <int ACT, int MB, bool SYM, int G, int CODE, bool XL>
void launch_xl(const GemmArgs &a, const Split &sp, hipStream_t stream) {
    if constexpr (MB == 1) {
        if (sp.s == 4) return launch_s<ACT, MB, 4, SYM, G, CODE, XL>(a, sp, stream);
    }
    if constexpr (MB <= 2) {
        if (sp.s == 2) return launch_s<ACT, MB, 2, SYM, G, CODE, XL>(a, sp, stream);
    }
    launch_s<ACT, MB, 1, SYM, G, CODE, XL>(a, sp, stream);
}

template <int ACT, int MB, bool SYM, int G, int CODE>
void launch_one(const GemmArgs &a, hipStream_t stream) {
    const Split sp = pick_split(a.M, a.Np >> 4, a.Kp >> 7, MB, a.group);
    if constexpr (MB == 1) {
        if (split_xl(a.M, MB)) return launch_xl<ACT, MB, SYM, G, CODE, true>(a, sp, stream);
    }
    launch_xl<ACT, MB, SYM, G, CODE, false>(a, sp, stream);
}

template <int ACT, int MB, int CODE>
void launch_mb(const GemmArgs &a, hipStream_t stream) {
    if constexpr (kCodeFp8<CODE>) {         // FP8 codes carry no zero point
        a.group == 128 ? launch_one<ACT, MB, true, 128, CODE>(a, stream)
                       : launch_one<ACT, MB, true, 64, CODE>(a, stream);
    } else {
        const bool sym = a.zeros == nullptr;
        if (a.group == 128) {
            sym ? launch_one<ACT, MB, true, 128, CODE>(a, stream)
                : launch_one<ACT, MB, false, 128, CODE>(a, stream);
        } else {
            sym ? launch_one<ACT, MB, true, 64, CODE>(a, stream)
                : launch_one<ACT, MB, false, 64, CODE>(a, stream);
        }
    }
}

template <int ACT, int CODE>
void launch_act(const GemmArgs &a, int mblocks, hipStream_t stream) {
    switch (mblocks) {
        case 1: launch_mb<ACT, 1, CODE>(a, stream); break;
        case 2: launch_mb<ACT, 2, CODE>(a, stream); break;
        case 3: launch_mb<ACT, 3, CODE>(a, stream); break;
        default: launch_mb<ACT, 4, CODE>(a, stream); break;
    }
}

template <int CODE>
void launch_code(const GemmArgs &a, int mblocks, hipStream_t stream) {
    a.act == kBF16 ? launch_act<kBF16, CODE>(a, mblocks, stream)
                   : launch_act<kF16, CODE>(a, mblocks, stream);
}

__global__ void fill_zero_kernel(uint16_t *__restrict__ Y, size_t count) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) Y[i] = 0;
}

}  // namespace

hipError_t launch_fill_zero(uint16_t *Y, size_t count, hipStream_t stream) {
    if (count) {
        const unsigned threads = 256;
        fill_zero_kernel<<<(unsigned)((count + threads - 1) / threads), threads, 0, stream>>>(Y, count);
    }
    return hipGetLastError();
}

size_t decode_workspace_bytes(int M, int N, int K, int group, int mblocks) {
    const int strips = padded_n(N) >> 4;
    return split_workspace(pick_split(M, strips, padded_k(K) >> 7, mblocks, group), strips,
                           mblocks);
}

hipError_t launch_decode(const GemmArgs &a, int mblocks, hipStream_t stream) {
    switch (a.code) {
        case kU2: launch_code<kU2>(a, mblocks, stream); break;
        case kU3: launch_code<kU3>(a, mblocks, stream); break;
        case kU8: launch_code<kU8>(a, mblocks, stream); break;
        case kE4M3: launch_code<kE4M3>(a, mblocks, stream); break;
        case kE5M2: launch_code<kE5M2>(a, mblocks, stream); break;
        default: launch_code<kU4>(a, mblocks, stream); break;
    }
    return hipGetLastError();
}

}  // namespace mpgemm
