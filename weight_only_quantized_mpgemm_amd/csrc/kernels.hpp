// Host-side launchers of the gfx950 kernels; the C ABI (api.hip) validates arguments and
// calls these.  Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device.hpp"

namespace mpgemm {

hipError_t launch_pack(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                       int K, int N, int group, void *packed_codes, void *packed_meta,
                       hipStream_t stream);

hipError_t launch_unpack(const void *packed_codes, const void *packed_meta, int K, int N,
                         int group, int symmetric, uint8_t *codes, uint16_t *scales,
                         uint8_t *zeros, hipStream_t stream);

// The same for 8-bit codes (16 x 64 one-byte tiles, byte zeros).
hipError_t launch_pack_w8(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                          int K, int N, int group, void *packed_codes, void *packed_meta,
                          hipStream_t stream);
hipError_t launch_unpack_w8(const void *packed_codes, const void *packed_meta, int K, int N,
                            int group, int symmetric, uint8_t *codes, uint16_t *scales,
                            uint8_t *zeros, hipStream_t stream);

// Ragged shapes: the packed planes of a K x N weight matrix describe the matrix padded to
// padded_k(K) x padded_n(N), whose padded weights dequantize to zero (include/mpgemm.h).
__host__ __device__ inline int padded_k(int K) { return (K + 127) / 128 * 128; }
__host__ __device__ inline int padded_n(int N) { return (N + 15) / 16 * 16; }

// The same for 2-bit and 3-bit codes (bits = 2 or 3; tiles of 16 columns x 128 k, 4-bit
// meta plane).
hipError_t launch_pack_lowbit(int bits, const uint8_t *codes, const uint16_t *scales,
                              const uint8_t *zeros, int K, int N, int group, void *packed_codes,
                              void *packed_meta, hipStream_t stream);
hipError_t launch_unpack_lowbit(int bits, const void *packed_codes, const void *packed_meta,
                                int K, int N, int group, int symmetric, uint8_t *codes,
                                uint16_t *scales, uint8_t *zeros, hipStream_t stream);

// Arguments of one GEMM; planes as written by launch_pack (code kU4), launch_pack_w8 (kU8,
// and the FP8 formats kE4M3 / kE5M2, which have no zero plane) or launch_pack_lowbit (kU2,
// kU3).
struct GemmArgs {
    const uint16_t *X;          // [M][K] activation bits (row stride K)
    const uint32_t *codes;      // packed codes plane (Kp x Np matrix)
    const uint16_t *scales;     // meta plane: scales
    const uint8_t *zeros;       // meta plane: zeros (nullptr when symmetric)
    uint16_t *Y;                // [M][N] output bits (row stride ldy, or N when 0)
    int M, N, K, group;         // user shape (K % 8 == 0)
    int Kp, Np;                 // padded shape of the packed planes
    int act;                    // Act
    int code;                   // Code: format of the packed codes
    void *workspace;            // split-K partials and counters (decode and tiled kernels)
    size_t workspace_bytes;     // its size (0 without a workspace)
    int ldy = 0;                // Y's row stride when it is not N (a column range of Y)
};

// Both split-K schemes keep their arrival counters in the first kSplitCounterBytes of the
// workspace and their partials after it.  The counters must be zero before the first call;
// every call leaves them zero.
constexpr size_t kSplitCounterBytes = 256 * 1024;

// Small-M kernel: S 16-column strips per workgroup, the K range split over the waves of the
// workgroup (and over workgroups), `mblocks` row blocks of 16 (M <= 16 * mblocks, mblocks in
// 1..4).
hipError_t launch_decode(const GemmArgs &a, int mblocks, hipStream_t stream);
// Workspace bytes launch_decode needs for this shape and group size, for any code format
// (0 when K is not split over workgroups).  The counter region must be zero before the
// first call; calls leave it zero.  N, K: the user shape.
size_t decode_workspace_bytes(int M, int N, int K, int group, int mblocks);

// Tiled large-M kernel on 32x32x16 MFMAs with a 128 (m) x 256 (n) workgroup tile.
hipError_t launch_prefill_x32(const GemmArgs &a, hipStream_t stream);
// The 32x32x16 kernel with a 256 (m) x 128 (n) workgroup tile.
hipError_t launch_prefill_x32_tall(const GemmArgs &a, hipStream_t stream);
// The 32x32x16 kernel with a 256 (m) x 256 (n) workgroup tile.
hipError_t launch_prefill_x32_wide(const GemmArgs &a, hipStream_t stream);
// Their instantiations per code format, one translation unit each (sh: tile shape, 1 for
// 256 x 128, 2 for 128 x 256, 3 for 256 x 256).
hipError_t launch_prefill_x32_u4(const GemmArgs &a, int sh, hipStream_t stream);
hipError_t launch_prefill_x32_u8(const GemmArgs &a, int sh, hipStream_t stream);
hipError_t launch_prefill_x32_fp8(const GemmArgs &a, int sh, hipStream_t stream);
// Sub-4-bit packed codes (Kp x Np, padded sizes) rewritten in the 4-bit packed layout
// (Kp*Np/2 bytes at `out`, 16-byte aligned), so that the 4-bit kernels with the same meta
// plane dequantize every weight to the same value (symmetric codes are shifted by
// 8 - 2^(bits-1) onto the 4-bit symmetric zero 8).
hipError_t launch_repack_lowbit_u4(int bits, bool symmetric, const void *packed_codes, int Kp,
                                   int Np, void *out, hipStream_t stream);
// Workspace bytes with which the 128 x 256 and 256 x 128 kernels split the K range of their
// tiles (grids of fewer tiles than compute units); 0 when they never do for this shape.
// The 256 x 256 kernel splits when the workspace it gets also holds its partials, and runs
// unsplit otherwise.  N, K: user shape.
size_t x32_workspace_bytes(int M, int N, int K);
// Workgroups of a 32x32x16 launch in tile shape sh, with the K split it takes
// on the current device (256 compute units when none is current); *parts: its part count,
// *cus: the compute units assumed (either pointer may be NULL).
int x32_grid(int M, int N, int K, int sh, int *parts, int *cus);
// Workgroup schedule of a 32x32x16 launch in tile shape sh (host only):
// info[8] and work[4 grid] as mpgemm_prefill_schedule documents; returns the grid size.
int x32_schedule(int M, int N, int K, int sh, int cus, int *info, int *work, int capacity);
// The 256 x 256 kernel on `cus` compute units: the first column it leaves to a second launch
// of 256 x 128 tiles (its last round's columns), or 0 when it runs in one launch.  N: user N.
int x32_wide_split_column(int M, int N, int cus);

// Decode attention over an 8-bit KV cache (attention.hip).
struct AttnArgs {
    const uint16_t *Q;          // [B][Hq][D] activation bits
    const uint8_t *cache;       // packed KV cache: num_blocks blocks
    int num_blocks;
    const int *table;           // [B][table_stride] block indices
    int table_stride;
    const int *lens;            // [B] context lengths
    int B, Hq, Hkv, D;          // D: the caller's head size (stored as kv_padded_d(D))
    int act;
    int kv_code;                // Code of the KV codes: kU8, kE4M3 or kE5M2
    int bps, splits;            // blocks per split, splits per (sequence, KV head)
    float scale_log2;           // softmax scale * log2(e)
    uint16_t *O;                // [B][Hq][D]
    float *part;                // split partials (splits > 1)
};
// A head of D values (a multiple of 16) is stored padded to a multiple of 64, the k depth
// of one 8-bit tile, with zero codes past D.
constexpr int kv_padded_d(int D) { return (D + 63) / 64 * 64; }
// Split partials for the caller's head size D.
size_t attn_part_bytes(int B, int Hq, int D, int splits);
hipError_t launch_attention_kv8(const AttnArgs &a, hipStream_t stream);
hipError_t launch_kv_pack(const uint8_t *kc, const uint16_t *ks, const uint8_t *kz,
                          const uint8_t *vc, const uint16_t *vs, const uint8_t *vz, int n, int t0,
                          int Hkv, int D, const int *table_row, int table_len, int num_blocks,
                          void *cache, hipStream_t stream);

// Writes zeros to Y (the K == 0 case).
hipError_t launch_fill_zero(uint16_t *Y, size_t count, hipStream_t stream);

}  // namespace mpgemm
