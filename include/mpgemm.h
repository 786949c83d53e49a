/*
 * mpgemm -- W4A16 mixed-precision GEMM for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libmpgemm.so.  Every call takes plain pointers and sizes; no framework types.
 *
 * Source: "LMDeploy Accelerates Mixed-Precision LLM Inference with TurboMind"
 * (arXiv 2508.15601), abbreviated [TurboMind] below.  Its GEMM pipeline has two halves:
 * offline weight packing (technique (i), "hardware-aware weight packing"; Fig. 6 and Fig. 7
 * captions) and an online mixed-precision GEMM that turns the low-bit codes into 16-bit
 * values in registers ("I2F" conversion and scaling; Fig. 4 and Fig. 6 captions) and
 * overlaps that work with the matrix multiply (technique (iii); Fig. 9 caption).  This
 * header exposes exactly that: mpgemm_pack_weights (offline), mpgemm_w4a16 (online) and
 * mpgemm_unpack (the inverse of packing, for round-trip checks).
 *
 * ---------------------------------------------------------------------------------
 * Quantized weights (the caller's unpacked form)
 *   codes  uint8  [K][N] row-major, each an unsigned 4-bit integer q in 0..15
 *   scales fp16   [G][N] row-major (IEEE binary16 bits), one per (group, column),
 *                 G = ceil(K/g) group rows
 *   zeros  uint8  [G][N] row-major, each a 4-bit integer z in 0..15; or NULL for
 *                 symmetric codes, whose zero is 8
 *   A group is g consecutive rows of k: rows [r*g, (r+1)*g) share scale and zero row r
 *   (the last group is shorter when K % g != 0).
 *   Only the low 4 bits of codes and zeros are read (higher bits are ignored).
 *   Dequantized weight: w[k][n] = (q[k][n] - z[k/g][n]) * s[k/g][n], rounded once
 *   (round to nearest even) to the activation format.
 *
 * Packed layout, version 1 (MPGEMM_LAYOUT_VERSION)
 *   Codes plane, K*N/2 bytes.  The code matrix is cut into tiles of 16 columns x 128 rows
 *   of k.  Tile T = (n/16)*(K/128) + k/128 starts at byte T*1024, so the tiles of one
 *   16-column strip follow each other along k.  Inside a tile, with kk = k%128 and
 *   nn = n%16, the element belongs to lane L = nn + 16*((kk%32)/8) and word t = kk/32;
 *   that little-endian 32-bit word is at byte L*16 + t*4.  Element i = kk%8 of the word
 *   sits in nibble p(i) = i/2 (even i) or 4 + i/2 (odd i), i.e. the nibbles read
 *   e7 e5 e3 e1 e6 e4 e2 e0 from most to least significant -- the interleave shown in
 *   [TurboMind]'s diagram beside Fig. 24.
 *   Why: lane L of a 64-lane wave fetches its 16 bytes of a tile with one 128-bit load; word
 *   t is the A operand of the t-th 16x16x32 MFMA step for that lane (row nn, k = 8*(L/16)
 *   .. 8*(L/16)+7); and (word >> 4j) & 0x000F000F puts elements (2j, 2j+1) in the low and
 *   high halves of a 32-bit register, the order the MFMA operand register needs, so one
 *   bitwise OR with the fp16 pattern of 1024 turns them into 1024+q without any shuffle
 *   ([TurboMind], Fig. 6 caption: after I2F the data already match the MMA lane layout).
 *   Meta plane.  Scales first: fp16 at element index e = (n/16)*(K/g)*16 + (k/g)*16 + n%16
 *   ((K/g)*N*2 bytes; the scales of one strip are contiguous).  Then, for asymmetric codes
 *   only, zeros: 4-bit values at the same index e, byte e/2, low nibble for even e and high
 *   nibble for odd e ((K/g)*N/2 bytes).
 *   Ragged shapes [TurboMind, Fig. 24: a data matrix padded up to the hardware tile].  The
 *   formulas above (and those of the 8-bit layout below) take K and N as the padded sizes
 *   Kp x Np: Np = N rounded up to a multiple of 16; Kp = K rounded up to a multiple of
 *   128.  Every padded weight dequantizes to zero: padded
 *   columns (n >= N) hold code 0, scale 0 and zero 0; padded rows (k >= K) of real columns
 *   hold the element's zero point as their code (its group's zero, 0 in groups past G,
 *   8 -- or 128 for 8-bit codes -- when symmetric); groups past G hold scale 0 and zero 0.
 *
 * Conventions for every call
 *   - Pointers are device pointers (hipMalloc'd or equivalent) owned by the caller.  The
 *     library allocates nothing and keeps no state between calls.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; argument validation happens synchronously, before anything is
 *     enqueued, and on error nothing is enqueued.
 *   - Return value: MPGEMM_OK or a negative mpgemm_status.  MPGEMM_ERR_HIP means the HIP
 *     runtime rejected the launch (e.g. no gfx950 device); mpgemm_status_string() names it.
 *   - Calls are reentrant; concurrent calls must not write overlapping outputs.
 *   - Shape limits: K % 8 == 0 (activation rows stay 16-byte aligned), any N >= 0,
 *     g in {64, 128}, M >= 0; with the padded sizes Kp, Np: (M+128)*Kp, Kp*Np and M*Np each
 *     below 2^31.  M == 0 or N == 0 is a valid no-op.
 *   - Alignment: every device pointer 16-byte aligned (MPGEMM_ERR_ALIGNMENT otherwise).
 *     Rows of Y need not be: for N % 4 != 0 the kernels store 2-byte elements.
 */
#ifndef MPGEMM_H
#define MPGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MPGEMM_LAYOUT_VERSION 1

typedef enum {
    MPGEMM_OK = 0,
    MPGEMM_ERR_INVALID_ARG = -1,   /* null pointer, negative size, bad enum value */
    MPGEMM_ERR_UNSUPPORTED = -2,   /* shape or group size outside the limits above */
    MPGEMM_ERR_ALIGNMENT = -3,     /* a device pointer is not 16-byte aligned */
    MPGEMM_ERR_WORKSPACE = -4,     /* workspace smaller than mpgemm_workspace_bytes() */
    MPGEMM_ERR_HIP = -5            /* the HIP runtime reported an error for the launch */
} mpgemm_status;

typedef enum {
    MPGEMM_F16 = 0,                /* fp16 activations, fp16 output */
    MPGEMM_BF16 = 1                /* bf16 activations, bf16 output (scales stay fp16) */
} mpgemm_dtype;

/* Layout version of the packed planes this library reads and writes. */
int mpgemm_layout_version(void);

/* Size of the packed codes plane: Kp*Np/2 bytes.  0 if the shape is unsupported. */
size_t mpgemm_packed_code_bytes(int K, int N);

/* Size of the packed meta plane: (Kp/g)*Np*2 + (symmetric ? 0 : (Kp/g)*Np/2) bytes.
 * 0 if the shape or group size is unsupported. */
size_t mpgemm_packed_meta_bytes(int K, int N, int group, int symmetric);

/*
 * Offline packing [TurboMind, technique (i); Fig. 6 and Fig. 7 captions]: rewrites codes,
 * scales and zeros (layouts above) into the version-1 packed planes.  zeros == NULL packs
 * symmetric weights (zero 8) and writes no zero plane.  A pure bit permutation: lossless.
 *   codes        in  [K][N] uint8
 *   scales       in  [G][N] fp16 bits, G = ceil(K/g)
 *   zeros        in  [G][N] uint8, or NULL
 *   packed_codes out mpgemm_packed_code_bytes(K, N) bytes
 *   packed_meta  out mpgemm_packed_meta_bytes(K, N, group, zeros == NULL) bytes
 */
int mpgemm_pack_weights(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                        int K, int N, int group, void *packed_codes, void *packed_meta,
                        void *stream);

/*
 * Exact inverse of mpgemm_pack_weights (codes come back in 0..15).  With symmetric != 0
 * the meta plane has no zero plane and `zeros` is not written (may be NULL).
 */
int mpgemm_unpack(const void *packed_codes, const void *packed_meta, int K, int N, int group,
                  int symmetric, uint8_t *codes, uint16_t *scales, uint8_t *zeros,
                  void *stream);

/*
 * Device workspace (bytes) mpgemm_w4a16 and mpgemm_w4a16_config use for this problem on the
 * current device: nonzero when a small-M kernel splits K over several workgroups (the
 * largest need of the configurations that can run M rows, and of 64-row chunks when
 * M > 64), or when a tiled kernel (M > 32) splits the K range of its tiles because the
 * grid has fewer tiles than the device has compute units (a tiled configuration forced at
 * M <= 32 runs unsplit).  The 256 x 256 tile (id 14) is not counted: its partials are twice
 * the others', and it splits only when the workspace passed holds them (the selector takes
 * it only for grids that need no split).  The workspace holds arrival
 * counters in its first 256 KiB and fp32 partial sums after them.
 *   - It must be all zero before its first use; every call leaves the counters zero again,
 *     so one zeroed allocation serves any number of later calls.
 *   - Calls that share a workspace must not run concurrently (use one per stream).
 *   - For a small-M kernel, passing less than its need (or NULL when it is nonzero)
 *     returns MPGEMM_ERR_WORKSPACE and enqueues nothing.  The tiled kernels' split is
 *     optional: with less workspace they run every tile whole (the same result up to the
 *     order in which fp32 partial sums are added).  Results are deterministic for a given
 *     shape, device and workspace size.
 */
size_t mpgemm_workspace_bytes(int M, int N, int K, int group, int dtype);

/*
 * Online mixed-precision GEMM [TurboMind, GEMM pipeline; Fig. 6 and Fig. 9 captions]:
 *   Y[m][n] = sum_k X[m][k] * w[k][n],  w dequantized from the packed planes in registers,
 *   products accumulated in fp32, Y rounded to the activation format (nearest even).
 *   X            in  [M][K] row-major, fp16 or bf16 bits per `dtype`
 *   packed_*     in  planes written by mpgemm_pack_weights for (K, N, group, symmetric)
 *   Y            out [M][N] row-major, same format as X
 *   workspace    in/out  mpgemm_workspace_bytes() bytes, zeroed before its first use (may
 *                be NULL when that is 0); see mpgemm_workspace_bytes
 * K == 0 writes zeros to Y.  The kernel is chosen by shape (see mpgemm_select_config).
 */
int mpgemm_w4a16(const void *X, int dtype, const void *packed_codes, const void *packed_meta,
                 int M, int N, int K, int group, int symmetric, void *Y, void *workspace,
                 size_t workspace_bytes, void *stream);

/*
 * mpgemm_w4a16 for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, result
 * and kernel selection as mpgemm_w4a16 without the workspace: the kernels that split K
 * take their arrival counters and fp32 partials from a static device buffer of
 * MPGEMM_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs on until
 * the process ends (given the same workspace size, mpgemm_w4a16 splits identically, so
 * the two return the same bits).  Nothing is allocated by the call.
 *   - The first call on a device looks the buffer up (and, outside graph capture, clears
 *     its counters with a kernel on `stream`); make that first call outside capture.
 *   - Every call on one device shares that device's buffer, which keeps the last call's
 *     contents (the kernels leave its counters zero).  Calls that overlap in time on one
 *     device (two streams, or a graph replay beside another call) race and must not be
 *     made.
 *   - A problem whose workspace (mpgemm_workspace_bytes) exceeds the buffer returns
 *     MPGEMM_ERR_WORKSPACE and enqueues nothing.  On MI355X every W4A16 shape fits.
 */
#define MPGEMM_NOALLOC_SCRATCH_BYTES (((size_t)32 << 20) + ((size_t)256 << 10))
int mpgemm_w4a16_noalloc(const void *X, int dtype, const void *packed_codes,
                         const void *packed_meta, int M, int N, int K, int group,
                         int symmetric, void *Y, void *stream);

/*
 * Kernel selection.  mpgemm_select_config returns the configuration mpgemm_w4a16 uses for
 * a shape (a positive id); mpgemm_config_name describes an id ("" for unknown ids);
 * mpgemm_w4a16_config runs one configuration explicitly (same contract as mpgemm_w4a16;
 * config_id 0 means "select"; an id that cannot run the shape returns
 * MPGEMM_ERR_UNSUPPORTED; an unknown id returns MPGEMM_ERR_INVALID_ARG).  Ids: 1..4
 * small-M kernel with 1..4 row blocks of 16 (M <= 16*id); 12 tiled large-M kernel on
 * 32x32x16 MFMAs with an LDS activation ring (four stages; eight stages of only the rows
 * below M when one row of tiles leaves part of the tile empty and g = 128 with 4-bit
 * codes), 128 x 256 workgroup tile; 13 the same with a
 * 256 x 128 tile; 14 the same with a 256 x 256 tile.  Ids 12, 13 and 14 take every
 * shape.  The selector picks 1..2 for M <= 32, and 3..4 for
 * M <= 64 (48 for 4-bit codes with group 128) with N K <= 4096 * 4096; else for M <= 128
 * the tile whose grid (with its K split, on the current device's compute units, 256 when
 * none is current) fills more units (on a tie 12 when both fill every unit and K >= 16384,
 * else 13 when both fill every unit or only 13 runs unsplit, else 12; 12 when 13 alone
 * needs more than one round); 12 for 256 < M <= 384 with K < 16384; 14 when its grid of
 * 256 x 256 tiles covers at least three quarters of the compute units, or at least half
 * of them in one round while both other tiles' grids exceed one round; 12 for M >= 2048
 * with N < 16384 and K < 8192; else 13.
 * (2- and 3-bit codes take 1..4 for every M <= 64.)
 */
int mpgemm_select_config(int M, int N, int K, int group, int dtype);
const char *mpgemm_config_name(int config_id);

/*
 * Workgroup schedule of the tiled kernels (ids 12, 13 and 14), computed on the host for
 * inspection; makes no GPU call.  The pages fix no tile order: this is the library's own
 * (tiles spread over the eight XCDs in contiguous ranges, walked four M-tiles at a time;
 * a grid of fewer tiles than compute units splits every tile's K range into P parts,
 * reduced by a second kernel).  It is the schedule mpgemm_w4a16_config runs when its
 * workspace holds mpgemm_workspace_bytes() bytes on a device with `cus` compute units
 * (0: no K split; for id 14, a workspace that holds its partials).  One exception: where
 * id 14's grid has a last round that would fill at most half of the units, the library
 * runs its whole rounds over the leading columns and the rest as id 13 tiles, a second
 * launch; the schedule shown is that of the single id-14 grid.
 *   M, N, K, config_id  shape (K % 8 == 0) and id 12, 13 or 14
 *   cus       compute units (256 on MI355X)
 *   info      out, int[8]: grid size, tile rows, tile columns, M tiles, N tiles (over the
 *             padded N), workgroups that run a whole tile, parts per split tile (1: none),
 *             stage-loop K
 *   work      out, int[4 * grid] or NULL: for workgroup b in launch order, {M tile, N tile,
 *             K part, split tile index or -1}; written only when capacity >= grid
 * Returns the grid size (> 0), MPGEMM_ERR_INVALID_ARG for a null info, a non-positive
 * size or another id, MPGEMM_ERR_UNSUPPORTED for shapes mpgemm_w4a16 rejects.
 */
int mpgemm_prefill_schedule(int M, int N, int K, int config_id, int cus, int *info, int *work,
                            int capacity);

/*
 * Kernel launches one call of a tiled configuration (ids 12, 13, 14) makes on a device with
 * `cus` compute units, computed on the host for inspection (profilers list launches, not
 * calls); makes no GPU call.  1, or 2 where id 14 runs its last round's columns as id 13
 * tiles (the exception mpgemm_prefill_schedule describes); a K split's reduction kernel is
 * not counted.  *split_column (may be NULL): the first column of the second launch, or N.
 * Returns MPGEMM_ERR_INVALID_ARG for a non-positive size, negative cus or another id,
 * MPGEMM_ERR_UNSUPPORTED for shapes mpgemm_w4a16 rejects.
 */
int mpgemm_prefill_launches(int M, int N, int K, int config_id, int cus, int *split_column);
int mpgemm_w4a16_config(const void *X, int dtype, const void *packed_codes,
                        const void *packed_meta, int M, int N, int K, int group, int symmetric,
                        void *Y, void *workspace, size_t workspace_bytes, int config_id,
                        void *stream);

/*
 * ---------------------------------------------------------------------------------
 * 8-bit weights (W8A16).  [TurboMind, abstract (pg1)]: the GEMM pipeline generalizes
 * across precision formats.  Same group form with 8-bit integers:
 *   codes  uint8 [K][N], all 8 bits: q in 0..255
 *   zeros  uint8 [G][N], all 8 bits: z in 0..255; or NULL for symmetric codes (z = 128)
 *   scales fp16 [G][N] as above
 *   w[k][n] = (q - z) * s rounded once to the activation format.
 * Packed 8-bit layout (same layout version)
 *   Codes plane, K*N bytes.  Tiles of 16 columns x 64 rows of k, 1 KiB each; tile
 *   T = (n/16)*(K/64) + k/64 starts at byte T*1024 (a strip's tiles follow each other
 *   along k).  Inside a tile, with kk = k%64 and nn = n%16: lane L = nn + 16*((kk%32)/8),
 *   step t = kk/32, and the code sits at byte L*16 + t*8 + kk%8 (k ascending in each
 *   8-byte run).  Why: lane L's 16 bytes, one 128-bit load, are the A operands of two
 *   16x16x32 MFMA steps (row nn, k = 8*(L/16) .. +7), and a byte permute against the fp16
 *   pattern of 1024 turns each pair of codes into the (k, k+1) register pair 1024 + q.
 *   Meta plane.  Scales exactly as for 4-bit codes; then, for asymmetric codes only, one
 *   zero byte per element at the same index e ((K/g)*N bytes).
 * Shape limits and conventions as above (ragged shapes padded the same way, symmetric
 * padding code 128).  The workspace is sized by mpgemm_workspace_bytes (the same for both
 * code widths).
 */

/* Size of the packed 8-bit codes plane: Kp*Np bytes.  0 if the shape is unsupported. */
size_t mpgemm_packed_code_bytes_w8(int K, int N);

/* Size of the packed 8-bit meta plane: (Kp/g)*Np*2 + (symmetric ? 0 : (Kp/g)*Np) bytes. */
size_t mpgemm_packed_meta_bytes_w8(int K, int N, int group, int symmetric);

/* Offline packing of 8-bit codes into the 8-bit layout; contract as mpgemm_pack_weights
 * (zeros == NULL packs symmetric weights, zero 128, and writes no zero plane). */
int mpgemm_pack_weights_w8(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                           int K, int N, int group, void *packed_codes, void *packed_meta,
                           void *stream);

/* Exact inverse of mpgemm_pack_weights_w8; contract as mpgemm_unpack. */
int mpgemm_unpack_w8(const void *packed_codes, const void *packed_meta, int K, int N,
                     int group, int symmetric, uint8_t *codes, uint16_t *scales,
                     uint8_t *zeros, void *stream);

/*
 * Y[M][N] = X[M][K] * dequant(W8)[K][N] with fp32 accumulation; arguments as for
 * mpgemm_w4a16, with planes written by mpgemm_pack_weights_w8.  mpgemm_w8a16_config runs
 * one configuration (ids as for mpgemm_w4a16_config: 1..4 small-M, 12, 13 and 14 tiled
 * 32x32x16).
 */
int mpgemm_w8a16(const void *X, int dtype, const void *packed_codes, const void *packed_meta,
                 int M, int N, int K, int group, int symmetric, void *Y, void *workspace,
                 size_t workspace_bytes, void *stream);
int mpgemm_w8a16_config(const void *X, int dtype, const void *packed_codes,
                        const void *packed_meta, int M, int N, int K, int group, int symmetric,
                        void *Y, void *workspace, size_t workspace_bytes, int config_id,
                        void *stream);

/*
 * ---------------------------------------------------------------------------------
 * FP8 weights (W-FP8 A16).  [TurboMind, Fig. 19 caption]: the same engine serves an FP8
 * Qwen3 8B model.  Each code is an OCP 8-bit floating-point number with no zero point:
 *   codes  uint8 [K][N], FP8 bit patterns in the format fp8_format:
 *            MPGEMM_FP8_E4M3: 1 sign, 4 exponent bits (bias 7), 3 fraction bits, subnormals,
 *                             no infinities, 0x7F / 0xFF are NaN (largest finite 448);
 *            MPGEMM_FP8_E5M2: 1 sign, 5 exponent bits (bias 15), 2 fraction bits,
 *                             subnormals, infinities and NaNs as in binary16 (it is the
 *                             high byte of binary16);
 *   scales fp16 [G][N] as above
 *   w[k][n] = fp8(q) * s rounded once to the activation format (NaN and infinite codes
 *   propagate as the product does).
 * Packing: mpgemm_pack_weights_w8 with zeros == NULL (the codes are bytes, so the 8-bit
 * layout holds them unchanged); mpgemm_unpack_w8 with symmetric = 1 inverts it.  Shape
 * limits, workspace and configuration ids as for mpgemm_w8a16.
 */
typedef enum {
    MPGEMM_FP8_E4M3 = 0,
    MPGEMM_FP8_E5M2 = 1
} mpgemm_fp8_format;

/*
 * Y[M][N] = X[M][K] * dequant(FP8 W)[K][N] with fp32 accumulation; X, Y, dtype, sizes,
 * group, workspace and stream as for mpgemm_w4a16; packed planes from
 * mpgemm_pack_weights_w8 with zeros == NULL.  A bad fp8_format returns
 * MPGEMM_ERR_INVALID_ARG.  mpgemm_wfp8a16_config runs one configuration, as
 * mpgemm_w8a16_config.
 */
int mpgemm_wfp8a16(const void *X, int dtype, int fp8_format, const void *packed_codes,
                   const void *packed_meta, int M, int N, int K, int group, void *Y,
                   void *workspace, size_t workspace_bytes, void *stream);
int mpgemm_wfp8a16_config(const void *X, int dtype, int fp8_format, const void *packed_codes,
                          const void *packed_meta, int M, int N, int K, int group, void *Y,
                          void *workspace, size_t workspace_bytes, int config_id,
                          void *stream);

/*
 * ---------------------------------------------------------------------------------
 * 2-bit and 3-bit weights.  "Progressive Mixed-Precision Decoding for Efficient LLM
 * Inference" (arXiv 2410.13461), abstract: 2/3-bit weights ease the memory-boundedness of
 * decoding.  The same group form with b-bit integers (bits = b = 2 or 3):
 *   codes  uint8 [K][N], low b bits read: q in 0..2^b-1
 *   zeros  uint8 [G][N], low b bits read; or NULL for symmetric codes (z = 2^(b-1))
 *   scales fp16 [G][N] as above
 *   w[k][n] = (q - z) * s rounded once to the activation format.
 * Packed sub-4-bit layout (same layout version; ragged shapes padded to Kp x Np as above,
 * symmetric padding code 2^(b-1))
 *   Codes plane, Kp*Np*b/8 bytes.  Tiles of 16 columns x 128 rows of k, 256*b bytes each;
 *   tile T = (n/16)*(Kp/128) + k/128 at byte T*256*b.  With kk = k%128 and nn = n%16:
 *   lane L = nn + 16*((kk%32)/8), step t = kk/32, element i = kk%8; lane L's b
 *   little-endian 32-bit words start at byte L*4*b of the tile.  The element belongs to
 *   pair register r = 4t + i/2, in its low 16-bit half (h = 0) for even i and its high
 *   half (h = 1) for odd i:
 *     b = 2: word r/8, code at bits 16h + 2*(r%4) + 8*((r%8)/4) .. +1;
 *     b = 3: r < 15: word r/5, code at bits 16h + 3*(r%5) .. +2;
 *            r = 15: bit c (c = 0, 1, 2) of the code at bit 16h + 15 of word c.
 *   Why: every code field sits inside the fp16 mantissa of its half (after at most one
 *   shift: by 8 for 2-bit, by 9 for 3-bit fields at 9 and 12), so one v_and_or_b32 with the
 *   fp16 pattern of the power of two whose mantissa step at that bit is 1 yields the pair
 *   (B + q_lo, B + q_hi), ready for the exact subtraction of B + z and the scaling; the
 *   register is the 16x16x32 MFMA A operand of step t (row nn, k = 8*(L/16) + 2*(i/2)).
 *   Meta plane exactly as for 4-bit codes (zeros as 4-bit values).
 * The GEMM runs the small-M kernel (configurations 1..4).  For M > 64 the codes are
 * rewritten in the 4-bit layout in the workspace (bits: 2 and 3-bit codes are valid 4-bit
 * codes; symmetric codes shift onto the 4-bit zero 8, so every weight dequantizes to the
 * same value) and a 32x32x16 tiled kernel runs on them with the same meta plane
 * (configurations 0, 12, 13 and 14).  That needs mpgemm_workspace_bytes_lowbit() bytes;
 * configuration 0 with less runs the small-M kernel on 64-row chunks instead (reading the
 * weights once per chunk), configurations 12, 13 and 14 return MPGEMM_ERR_WORKSPACE.  A
 * bits value other than 2 or 3 returns MPGEMM_ERR_INVALID_ARG.
 */

/* Workspace for mpgemm_wlowbit_a16(_config): that of mpgemm_workspace_bytes, and for
 * M > 64 room for the 4-bit rewrite of the codes (Kp*Np/2 bytes) past the tiled kernels'
 * region; same zero-initialization and sharing rules.  0 for a bits value other than 2, 3. */
size_t mpgemm_workspace_bytes_lowbit(int bits, int M, int N, int K, int group, int dtype);

/* Size of the packed sub-4-bit codes plane: Kp*Np*bits/8 bytes (0 if unsupported).  The
 * meta plane is sized by mpgemm_packed_meta_bytes. */
size_t mpgemm_packed_code_bytes_lowbit(int bits, int K, int N);

/* Offline packing of b-bit codes; contract as mpgemm_pack_weights. */
int mpgemm_pack_weights_lowbit(int bits, const uint8_t *codes, const uint16_t *scales,
                               const uint8_t *zeros, int K, int N, int group,
                               void *packed_codes, void *packed_meta, void *stream);

/* Exact inverse of mpgemm_pack_weights_lowbit (codes come back in 0..2^b-1). */
int mpgemm_unpack_lowbit(int bits, const void *packed_codes, const void *packed_meta, int K,
                         int N, int group, int symmetric, uint8_t *codes, uint16_t *scales,
                         uint8_t *zeros, void *stream);

/* Y[M][N] = X[M][K] * dequant(Wb)[K][N]; arguments as for mpgemm_w4a16. */
int mpgemm_wlowbit_a16(int bits, const void *X, int dtype, const void *packed_codes,
                       const void *packed_meta, int M, int N, int K, int group, int symmetric,
                       void *Y, void *workspace, size_t workspace_bytes, void *stream);
int mpgemm_wlowbit_a16_config(int bits, const void *X, int dtype, const void *packed_codes,
                              const void *packed_meta, int M, int N, int K, int group,
                              int symmetric, void *Y, void *workspace, size_t workspace_bytes,
                              int config_id, void *stream);

/*
 * ---------------------------------------------------------------------------------
 * Attention decode over an 8-bit KV cache.  [TurboMind, attention pipeline; Fig. 4 and
 * Fig. 10 captions]: the low-bit KV cache is dequantized to 16-bit values by I2F scaling,
 * V sits in a transposed tile layout for the matrix cores, KV streams in 64-token tiles.
 * Quantized KV (the caller's form, per token):
 *   kc, vc  uint8 [n][Hkv][D] codes;  ks, vs  fp16 [n][Hkv] scales;  kz, vz  uint8 [n][Hkv]
 *   zeros: k[t][d] = (kc - kz[t]) * ks[t] rounded once to the activation format, v alike.
 * Head sizes (adaptive head alignment [TurboMind abstract, technique (ii); Fig. 24 caption:
 * padding for MMA data misalignment]): D is any multiple of 16 from 16 to 256; a head is
 * stored padded to Dp = D rounded up to a multiple of 64 (the k depth of one 8-bit tile),
 * with codes 0 at d >= D.  Q and O rows keep D values.
 * Packed KV cache: an array of blocks of 64 tokens of one sequence, all KV heads, of
 * mpgemm_kv_block_bytes(Hkv, D) = Hkv * (128*Dp + 384) bytes each; block j of sequence b is
 * block block_table[b*table_stride + j] (token t in block t/64, slot t%64).  KV head h of a
 * block occupies HB = 128*Dp + 384 bytes at h*HB:
 *   [0, 64*Dp)       K codes in the 8-bit weight layout (above) of the Dp x 64 matrix K^T
 *                    (k = d, n = slot), i.e. 16-slot strips of 64-deep 1 KiB tiles;
 *   [64*Dp, 128*Dp)  V codes in the 8-bit weight layout of the 64 x Dp matrix V (k = slot,
 *                    n = d): V transposed, so 16 values of d x 8 consecutive tokens form
 *                    one matrix-core operand;
 *   then K scales [64] fp16, V scales [64] fp16, K zeros [64] uint8, V zeros [64] uint8.
 * Hq is a multiple of Hkv with Hq/Hkv <= 16.
 */

/* Bytes of one cache block (0 if Hkv or D is unsupported). */
size_t mpgemm_kv_block_bytes(int Hkv, int D);

/*
 * Writes tokens t0 .. t0 + n_tokens - 1 of one sequence (the caller's form above, device
 * pointers; ks, vs, table_row 4-byte aligned, kc, vc, cache 16-byte aligned) into the cache
 * through that sequence's block-table row (table_len entries; t0 + n_tokens <= 64 *
 * table_len).  Entries outside [0, num_blocks) are skipped.  Prefill and every decode
 * step's append are calls of this one function.  kz and vz are NULL together for FP8 codes
 * (no zero points).
 */
int mpgemm_kv_pack(const uint8_t *kc, const uint16_t *ks, const uint8_t *kz, const uint8_t *vc,
                   const uint16_t *vs, const uint8_t *vz, int n_tokens, int t0, int Hkv, int D,
                   const int *table_row, int table_len, int num_blocks, void *cache,
                   void *stream);

/* Device workspace (bytes) mpgemm_attention_decode_kv8 needs: fp32 partials when the
 * block range of a sequence is split over several waves; 0 otherwise. */
size_t mpgemm_attention_workspace_bytes(int B, int Hq, int Hkv, int D, int max_len);

/*
 * One decode step of attention for B sequences, one query token each:
 *   o[b][h] = sum_t p[t] v[t],  p = softmax_t<lens[b] (scale * q[b][h] . k[t]),
 *   with query head h reading KV head h / (Hq / Hkv); fp32 scores, softmax and
 *   accumulation (the probabilities, times V's scale, enter the matrix cores as 16-bit
 *   values), o rounded to the activation format.  lens[b] == 0 gives zeros.
 *   Q, O         [B][Hq][D] fp16 or bf16 bits per dtype (16-byte aligned)
 *   cache        num_blocks packed blocks; block_table [B][table_stride] int32; lens [B]
 *                int32 (device), each <= max_len (a host bound that sizes the launch);
 *                table entries outside [0, num_blocks) are skipped
 *   workspace    mpgemm_attention_workspace_bytes(B, Hq, Hkv, D, max_len) bytes (may be
 *                NULL when that is 0); its contents need no initialization
 */
int mpgemm_attention_decode_kv8(const void *Q, int dtype, const void *cache, int num_blocks,
                                const int *block_table, int table_stride, const int *lens,
                                int B, int Hq, int Hkv, int D, int max_len, float scale,
                                void *O, void *workspace, size_t workspace_bytes,
                                void *stream);

/*
 * The same over an FP8 KV cache: codes are OCP FP8 numbers in fp8_format
 * (MPGEMM_FP8_E4M3 / MPGEMM_FP8_E5M2), k = fp8(kc) * ks and v = fp8(vc) * vs rounded once
 * to the activation format, no zero points (pack with kz = vz = NULL; the zero fields of
 * the blocks are then written as 0 and not read).  Arguments otherwise as
 * mpgemm_attention_decode_kv8; a bad fp8_format returns MPGEMM_ERR_INVALID_ARG.
 */
int mpgemm_attention_decode_kvfp8(const void *Q, int dtype, int fp8_format, const void *cache,
                                  int num_blocks, const int *block_table, int table_stride,
                                  const int *lens, int B, int Hq, int Hkv, int D, int max_len,
                                  float scale, void *O, void *workspace, size_t workspace_bytes,
                                  void *stream);

/* Static, human-readable name of a status code. */
const char *mpgemm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MPGEMM_H */
