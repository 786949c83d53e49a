// C ABI of libmpgemm (declared and specified in include/mpgemm.h): argument validation,
// kernel selection by shape, and dispatch to the gfx950 kernels.
//
// Source of the method: "LMDeploy Accelerates Mixed-Precision LLM Inference with TurboMind"
// (arXiv 2508.15601): an offline packing step and an online mixed-precision GEMM.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

#include "mpgemm.h"
#include "kernels.hpp"

// Workspace of mpgemm_w4a16_noalloc (see scratch_of_current_device).
static __device__ __align__(256) uint8_t scratch[MPGEMM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kIndexLimit = (int64_t)1 << 31;

enum ConfigId {
    kConfigSelect = 0,
    kConfigDecode1 = 1,
    kConfigDecode2 = 2,
    kConfigDecode3 = 3,
    kConfigDecode4 = 4,
    kConfigPrefillX32 = 12,    // 32x32x16 kernel, 128 x 256 workgroup tile
    kConfigPrefillX32Tall = 13,  // same, 256 x 128 workgroup tile
    kConfigPrefillX32Wide = 14,  // same, 256 x 256 workgroup tile
};

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Any N >= 0 and any K >= 0 with K % 8 == 0 (activation rows stay 16-byte aligned); the
// packed planes hold the matrix padded to padded_k(K) x padded_n(N).
int check_shape(int M, int N, int K, int group) {
    if (M < 0 || N < 0 || K < 0) return MPGEMM_ERR_INVALID_ARG;
    if (group != 64 && group != 128) return MPGEMM_ERR_UNSUPPORTED;
    if (K % 8 != 0 || K > (1 << 30) || N > (1 << 30)) return MPGEMM_ERR_UNSUPPORTED;
    // Kernels address planes with 32-bit byte offsets, including one-past-the-end rows.
    const int64_t Kp = mpgemm::padded_k(K), Np = mpgemm::padded_n(N);
    if ((int64_t)(M + 128) * Kp >= kIndexLimit || Kp * Np >= kIndexLimit ||
        (int64_t)M * Np >= kIndexLimit)
        return MPGEMM_ERR_UNSUPPORTED;
    return MPGEMM_OK;
}

int64_t packed_cells(int K, int N, int group) {
    return (int64_t)(mpgemm::padded_k(K) / group) * mpgemm::padded_n(N);
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return MPGEMM_OK;
    if (getenv("MPGEMM_LOG")) fprintf(stderr, "mpgemm: HIP error %s\n", hipGetErrorString(e));
    return MPGEMM_ERR_HIP;
}

// Small M streams the weights once (HBM-bound): the split-K strip kernel with one or two
// row blocks of 16.  Above 32 rows each of its strip groups re-reads an activation block
// of M rows, M / (4 S) times the weight bytes, and the tiled kernels -- which stage
// activations once per tile through LDS and split the K range of small grids -- were 1.2
// to 3.3x faster on MI355X (cold weights; Llama-3-70B bf16 QKV at M = 64: 43 us against 98,
// gate_up 137 against 457; Qwen3-32B down 86 against 193), except on the smallest
// matrices (N K <= 4096 x 4096) up to 64 rows, or 48 with 4-bit codes at g = 128, whose
// tiled kernels keep the live rows in an eight-stage ring (Llama-3-8B O: three row blocks
// 14.0 us against 14.5 at M = 40, four 18.6 against 14.7 at M = 64).  Up to 128 rows both
// tiles run one tile row (their MFMAs skip the row blocks past M), and the one whose grid,
// with its K split, fills more compute units wins: Llama-3-8B shapes went to the
// 256 x 128 tile (QKV M = 64: 192 workgroups against 96, 19.4 us against 20.5; gate_up,
// unsplit against split in two, 31.4 against 36.4), and so did grids that both fill every
// unit (Llama-3-70B O: 24.8 against 25.6 at M = 64) unless K >= 16384 (Llama-3-70B down,
// 128 x 256 split eight ways against 256 x 128 split four: 49.4 against 53.3 at M = 64,
// 67.5 against 73.1 at M = 128); the Llama-3-70B and Qwen3-32B QKV and gate_up
// went to the 128 x 256 one (equal partial fill, or a 256 x 128 grid of more than one round:
// 70B gate_up 115 against 125 us).  Above 128 rows the 256 x 128 tile, whose
// dequantized weights each feed 256 rows (0-15% faster from 160 to 8192 rows on all three
// workloads), except for 257..384 rows with K < 16384 (the 128-row tile pads less) and
// M >= 2048 at N < 16384, K < 8192 (Llama-3-8B QKV and O), where the two measured within a
// few percent either way from box to box.
int pick_tile(int M, int N, int K) {
    int p12 = 1, p13 = 1, cus = 256;
    const int g12 = mpgemm::x32_grid(M, N, K, 2, &p12, &cus);
    const int g13 = mpgemm::x32_grid(M, N, K, 1, &p13, nullptr);
    if (g13 > cus && g12 <= cus) return kConfigPrefillX32;
    const int f12 = g12 < cus ? g12 : cus, f13 = g13 < cus ? g13 : cus;
    if (f13 > f12) return kConfigPrefillX32Tall;
    if (f13 == f12 && f13 == cus && K >= 16384) return kConfigPrefillX32;
    if (f13 == f12 && (f13 == cus || (p13 == 1 && p12 > 1))) return kConfigPrefillX32Tall;
    return kConfigPrefillX32;
}

bool tiled_config(int cfg) {
    return cfg == kConfigPrefillX32 || cfg == kConfigPrefillX32Tall ||
           cfg == kConfigPrefillX32Wide;
}
hipError_t launch_tiled(int cfg, const mpgemm::GemmArgs &a, hipStream_t s) {
    if (cfg == kConfigPrefillX32Tall) return mpgemm::launch_prefill_x32_tall(a, s);
    if (cfg == kConfigPrefillX32Wide) return mpgemm::launch_prefill_x32_wide(a, s);
    return mpgemm::launch_prefill_x32(a, s);
}

// The 256 x 256 tile (4-bit codes) where its grid covers at least three quarters of the
// compute units: it then beat both other tiles on every measured shape, by 2-15%
// (Llama-3-8B QKV at M = 2048: 192 tiles, 91 us against 98 and 104; gate_up 2048: 392
// against 401; at M = 8192 7-10% on all four Llama-3-8B projections, 8% on Llama-3-70B
// bf16 gate_up and down at M = 4096, 6-10% on Qwen3-32B gate_up and down).  Smaller grids
// would need its K split, whose partials are twice the other tiles' (and more than the
// reported workspace holds): there the other tiles, split, were up to twice as fast.
// Also where its grid is one round of at least half the units while the 256 x 128 tiles
// would need a second, partial one (Qwen3-32B QKV at M = 1024: 160 wide tiles, 107 us
// against 132 for 320 tiles of 256 x 128 and 129 for 320 of 128 x 256).
bool wide_fills(int M, int N, int K) {
    int cus = 256;
    mpgemm::x32_grid(M, N, K, 3, nullptr, &cus);        // the device's units (256 if none)
    const int64_t Np = mpgemm::padded_n(N);
    const int64_t tiles = (int64_t)((M + 255) / 256) * ((Np + 255) / 256);
    if (4 * tiles >= 3 * (int64_t)cus) return true;
    const int64_t t13 = (int64_t)((M + 255) / 256) * ((Np + 127) / 128);
    const int64_t t12 = (int64_t)((M + 127) / 128) * ((Np + 255) / 256);
    return tiles <= cus && 2 * tiles >= cus && t13 > cus && t12 > cus;
}

int select_config(int M, int N, int K, int group, int code) {
    if (M <= 16) return kConfigDecode1;
    const int64_t nk = (int64_t)N * K;
    // The tiled kernels' eight-stage ring (4-bit codes, g = 128) beats four row blocks of
    // the small-M kernel on the smallest matrices too.
    const int small_m = code == mpgemm::kU4 && group == 128 ? 48 : 64;
    if (M <= 32 || (M <= small_m && nk <= 4096 * 4096)) return (M + 15) / 16;
    if (M <= 128) return pick_tile(M, N, K);
    if (M > 256 && M <= 384 && K < 16384) return kConfigPrefillX32;
    if (wide_fills(M, N, K)) return kConfigPrefillX32Wide;
    if (M >= 2048 && N < 16384 && K < 8192) return kConfigPrefillX32;
    return kConfigPrefillX32Tall;
}

// 2- and 3-bit codes at M > 64: the sub-4-bit codes are rewritten in the 4-bit layout in
// the workspace (past the region the tiled kernels' K split may use) and the 32x32x16
// kernel runs on them with the same meta plane.  Measured on the Llama-3-8B projections,
// this beats the small-M kernel on 64-row chunks from M = 128 on (2.2-3.7x there, 9x at
// M = 2048).  MPGEMM_LOWBIT_REPACK_M sets a higher threshold (tuning sweeps).
size_t lowbit_repack_offset(int M, int N, int K) {
    size_t r = mpgemm::kSplitCounterBytes;
    const size_t x = mpgemm::x32_workspace_bytes(M, N, K);
    if (x > r) r = x;
    return (r + 255) / 256 * 256;
}
size_t lowbit_repack_bytes(int M, int N, int K) {
    return lowbit_repack_offset(M, N, K) +
           (size_t)mpgemm::padded_k(K) * (size_t)mpgemm::padded_n(N) / 2;
}
int lowbit_repack_min_m() {
    if (const char *env = getenv("MPGEMM_LOWBIT_REPACK_M")) {
        const int v = atoi(env);
        if (v > 64) return v;
    }
    return 65;
}

int gemm_impl(int code, const void *X, int dtype, const void *packed_codes,
              const void *packed_meta, int M, int N, int K, int group, int symmetric, void *Y,
              void *workspace, size_t workspace_bytes, int config_id, void *stream) {
    if (dtype != MPGEMM_F16 && dtype != MPGEMM_BF16) return MPGEMM_ERR_INVALID_ARG;
    if (symmetric != 0 && symmetric != 1) return MPGEMM_ERR_INVALID_ARG;
    const int st = check_shape(M, N, K, group);
    if (st != MPGEMM_OK) return st;
    if (config_id != kConfigSelect &&
        !((config_id >= kConfigDecode1 && config_id <= kConfigDecode4) || tiled_config(config_id)))
        return MPGEMM_ERR_INVALID_ARG;
    if (M == 0 || N == 0) return MPGEMM_OK;
    if (Y == nullptr) return MPGEMM_ERR_INVALID_ARG;
    if (!aligned16(Y)) return MPGEMM_ERR_ALIGNMENT;
    hipStream_t s = (hipStream_t)stream;
    if (K == 0) return hip_status(mpgemm::launch_fill_zero((uint16_t *)Y, (size_t)M * N, s));
    if (X == nullptr || packed_codes == nullptr || packed_meta == nullptr)
        return MPGEMM_ERR_INVALID_ARG;
    if (!aligned16(X) || !aligned16(packed_codes) || !aligned16(packed_meta))
        return MPGEMM_ERR_ALIGNMENT;

    // 2- and 3-bit codes reach the tiled kernels only through the 4-bit rewrite (M > 64):
    // up to 64 rows they take the strip kernel at every N.
    const bool lowbit = code == mpgemm::kU2 || code == mpgemm::kU3;
    const int cfg = config_id != kConfigSelect ? config_id
                    : lowbit && M <= 64     ? (M + 15) / 16
                                            : select_config(M, N, K, group, code);
    if (cfg >= kConfigDecode1 && cfg <= kConfigDecode4 && M > 16 * cfg)
        return MPGEMM_ERR_UNSUPPORTED;
    const int Kp = mpgemm::padded_k(K);

    mpgemm::GemmArgs a;
    a.X = (const uint16_t *)X;
    a.codes = (const uint32_t *)packed_codes;
    a.scales = (const uint16_t *)packed_meta;
    a.zeros = symmetric ? nullptr : (const uint8_t *)packed_meta + packed_cells(K, N, group) * 2;
    a.code = code;
    a.Kp = Kp;
    a.Np = mpgemm::padded_n(N);
    a.Y = (uint16_t *)Y;
    a.M = M;
    a.N = N;
    a.K = K;
    a.group = group;
    a.act = dtype == MPGEMM_BF16 ? mpgemm::kBF16 : mpgemm::kF16;
    a.workspace = workspace;
    a.workspace_bytes = workspace ? workspace_bytes : 0;
    if (cfg >= kConfigDecode1 && cfg <= kConfigDecode4) {
        const size_t need = mpgemm::decode_workspace_bytes(M, N, K, group, cfg);
        if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
            return MPGEMM_ERR_WORKSPACE;
    }
    if (lowbit && M > 64) {
        const bool tiled = config_id != kConfigSelect || M >= lowbit_repack_min_m();
        if (tiled && workspace != nullptr && aligned16(workspace) &&
            workspace_bytes >= lowbit_repack_bytes(M, N, K)) {
            const size_t off = lowbit_repack_offset(M, N, K);
            void *codes4 = static_cast<char *>(workspace) + off;
            int st = hip_status(mpgemm::launch_repack_lowbit_u4(code == mpgemm::kU2 ? 2 : 3,
                                                                symmetric != 0, packed_codes,
                                                                a.Kp, a.Np, codes4, s));
            if (st != MPGEMM_OK) return st;
            mpgemm::GemmArgs c = a;
            c.codes = (const uint32_t *)codes4;
            c.code = mpgemm::kU4;
            c.workspace_bytes = off;
            const int xcfg =
                config_id != kConfigSelect ? cfg : select_config(M, N, K, group, mpgemm::kU4);
            if (getenv("MPGEMM_LOG"))
                fprintf(stderr, "mpgemm: W%dA16 M=%d N=%d K=%d g=%d -> 4-bit repack, %s\n",
                        code == mpgemm::kU2 ? 2 : 3, M, N, K, group, mpgemm_config_name(xcfg));
            return hip_status(launch_tiled(xcfg, c, s));
        }
        if (config_id != kConfigSelect) return MPGEMM_ERR_WORKSPACE;
        const size_t need = mpgemm::decode_workspace_bytes(64, N, K, group, kConfigDecode4);
        if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
            return MPGEMM_ERR_WORKSPACE;
        if (getenv("MPGEMM_LOG"))
            fprintf(stderr, "mpgemm: W%dA16 M=%d N=%d K=%d g=%d -> %s in %d row chunks\n",
                    code == mpgemm::kU2 ? 2 : 3, M, N, K, group,
                    mpgemm_config_name(kConfigDecode4), (M + 63) / 64);
        for (int m0 = 0; m0 < M; m0 += 64) {
            mpgemm::GemmArgs c = a;
            c.X = a.X + (size_t)m0 * K;
            c.Y = a.Y + (size_t)m0 * N;
            c.M = M - m0 < 64 ? M - m0 : 64;
            const int st = hip_status(mpgemm::launch_decode(c, kConfigDecode4, s));
            if (st != MPGEMM_OK) return st;
        }
        return MPGEMM_OK;
    }
    if (getenv("MPGEMM_LOG")) {
        static const char *const names[] = {"W4A16", "W8A16", "W(E4M3)A16", "W(E5M2)A16",
                                            "W2A16", "W3A16"};
        fprintf(stderr, "mpgemm: %s M=%d N=%d K=%d g=%d dtype=%d sym=%d -> %s\n", names[code],
                M, N, K, group, dtype, symmetric, mpgemm_config_name(cfg));
    }
    if (tiled_config(cfg)) return hip_status(launch_tiled(cfg, a, s));
    return hip_status(mpgemm::launch_decode(a, cfg, s));
}

// ------------------------------------------------------------ allocation-free scratch --
// The workspace of mpgemm_w4a16_noalloc: a file-scope device array, one copy per device,
// held until the process ends.  In host code `scratch` names a host-side stand-in, not a
// device address: the device address comes from hipGetSymbolAddress, looked up once per
// device with that device current, and only that pointer is handed to kernels.
constexpr size_t kScratchBytes = MPGEMM_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes > mpgemm::kSplitCounterBytes, "scratch holds the counters");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];

// The current device's scratch address (looked up and, outside graph capture, its counter
// region cleared by a kernel on `stream`, at the first call on that device).
int scratch_of_current_device(void *stream, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MPGEMM_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return MPGEMM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return MPGEMM_ERR_HIP;
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing((hipStream_t)stream, &cap) != hipSuccess) return MPGEMM_ERR_HIP;
        if (cap == hipStreamCaptureStatusNone) {
            const int st = hip_status(mpgemm::launch_fill_zero(
                static_cast<uint16_t *>(p), mpgemm::kSplitCounterBytes / 2, (hipStream_t)stream));
            if (st != MPGEMM_OK) return st;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MPGEMM_OK;
}

}  // namespace

extern "C" {

int mpgemm_layout_version(void) { return MPGEMM_LAYOUT_VERSION; }

size_t mpgemm_packed_code_bytes(int K, int N) {
    if (check_shape(0, N, K, 128) != MPGEMM_OK) return 0;
    return (size_t)mpgemm::padded_k(K) * (size_t)mpgemm::padded_n(N) / 2;
}

size_t mpgemm_packed_meta_bytes(int K, int N, int group, int symmetric) {
    if (check_shape(0, N, K, group) != MPGEMM_OK) return 0;
    const size_t cells = (size_t)packed_cells(K, N, group);
    return cells * 2 + (symmetric ? 0 : cells / 2);
}

int mpgemm_pack_weights(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                        int K, int N, int group, void *packed_codes, void *packed_meta,
                        void *stream) {
    const int st = check_shape(0, N, K, group);
    if (st != MPGEMM_OK) return st;
    if ((size_t)K * N == 0) return MPGEMM_OK;
    if (codes == nullptr || scales == nullptr || packed_codes == nullptr ||
        packed_meta == nullptr)
        return MPGEMM_ERR_INVALID_ARG;
    if (!aligned16(codes) || !aligned16(scales) || (zeros && !aligned16(zeros)) ||
        !aligned16(packed_codes) || !aligned16(packed_meta))
        return MPGEMM_ERR_ALIGNMENT;
    return hip_status(mpgemm::launch_pack(codes, scales, zeros, K, N, group, packed_codes,
                                          packed_meta, (hipStream_t)stream));
}

int mpgemm_unpack(const void *packed_codes, const void *packed_meta, int K, int N, int group,
                  int symmetric, uint8_t *codes, uint16_t *scales, uint8_t *zeros,
                  void *stream) {
    if (symmetric != 0 && symmetric != 1) return MPGEMM_ERR_INVALID_ARG;
    const int st = check_shape(0, N, K, group);
    if (st != MPGEMM_OK) return st;
    if ((size_t)K * N == 0) return MPGEMM_OK;
    if (packed_codes == nullptr || packed_meta == nullptr || codes == nullptr ||
        scales == nullptr || (!symmetric && zeros == nullptr))
        return MPGEMM_ERR_INVALID_ARG;
    if (!aligned16(packed_codes) || !aligned16(packed_meta) || !aligned16(codes) ||
        !aligned16(scales) || (!symmetric && !aligned16(zeros)))
        return MPGEMM_ERR_ALIGNMENT;
    return hip_status(mpgemm::launch_unpack(packed_codes, packed_meta, K, N, group, symmetric,
                                            codes, scales, zeros, (hipStream_t)stream));
}

size_t mpgemm_workspace_bytes_lowbit(int bits, int M, int N, int K, int group, int dtype) {
    if (bits != 2 && bits != 3) return 0;
    size_t need = mpgemm_workspace_bytes(M, N, K, group, dtype);
    if (M > 64 && N > 0 && K > 0 && check_shape(M, N, K, group) == MPGEMM_OK) {
        const size_t r = lowbit_repack_bytes(M, N, K);
        if (r > need) need = r;
    }
    return need;
}

size_t mpgemm_workspace_bytes(int M, int N, int K, int group, int dtype) {
    (void)dtype;
    if (check_shape(M, N, K, group) != MPGEMM_OK || M == 0 || N == 0 || K == 0) return 0;
    size_t need = 0;
    for (int mblocks = (M + 15) / 16; mblocks <= 4; ++mblocks) {
        const size_t b = mpgemm::decode_workspace_bytes(M, N, K, group, mblocks);
        if (b > need) need = b;
    }
    if (M > 64) {                   // 2- and 3-bit codes: 64-row chunks of the small-M kernel
        const size_t b = mpgemm::decode_workspace_bytes(64, N, K, group, 4);
        if (b > need) need = b;
    }
    if (M > 32) {                   // the tiled kernels' K split (small grids)
        const size_t x = mpgemm::x32_workspace_bytes(M, N, K);
        if (x > need) need = x;
    }
    return need;
}

int mpgemm_w4a16(const void *X, int dtype, const void *packed_codes, const void *packed_meta,
                 int M, int N, int K, int group, int symmetric, void *Y, void *workspace,
                 size_t workspace_bytes, void *stream) {
    return gemm_impl(mpgemm::kU4, X, dtype, packed_codes, packed_meta, M, N, K, group,
                     symmetric, Y, workspace, workspace_bytes, kConfigSelect, stream);
}

int mpgemm_w4a16_noalloc(const void *X, int dtype, const void *packed_codes,
                         const void *packed_meta, int M, int N, int K, int group,
                         int symmetric, void *Y, void *stream) {
    if (dtype != MPGEMM_F16 && dtype != MPGEMM_BF16) return MPGEMM_ERR_INVALID_ARG;
    const int st = check_shape(M, N, K, group);
    if (st != MPGEMM_OK) return st;
    if (mpgemm_workspace_bytes(M, N, K, group, dtype) > kScratchBytes)
        return MPGEMM_ERR_WORKSPACE;
    void *ws = nullptr;
    const int sst = scratch_of_current_device(stream, &ws);
    if (sst != MPGEMM_OK) return sst;
    return gemm_impl(mpgemm::kU4, X, dtype, packed_codes, packed_meta, M, N, K, group,
                     symmetric, Y, ws, kScratchBytes, kConfigSelect, stream);
}

int mpgemm_w4a16_config(const void *X, int dtype, const void *packed_codes,
                        const void *packed_meta, int M, int N, int K, int group, int symmetric,
                        void *Y, void *workspace, size_t workspace_bytes, int config_id,
                        void *stream) {
    return gemm_impl(mpgemm::kU4, X, dtype, packed_codes, packed_meta, M, N, K, group,
                     symmetric, Y, workspace, workspace_bytes, config_id, stream);
}

size_t mpgemm_packed_code_bytes_w8(int K, int N) {
    if (check_shape(0, N, K, 128) != MPGEMM_OK) return 0;
    return (size_t)mpgemm::padded_k(K) * (size_t)mpgemm::padded_n(N);
}

size_t mpgemm_packed_meta_bytes_w8(int K, int N, int group, int symmetric) {
    if (check_shape(0, N, K, group) != MPGEMM_OK) return 0;
    const size_t cells = (size_t)packed_cells(K, N, group);
    return cells * 2 + (symmetric ? 0 : cells);
}

int mpgemm_pack_weights_w8(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                           int K, int N, int group, void *packed_codes, void *packed_meta,
                           void *stream) {
    const int st = check_shape(0, N, K, group);
    if (st != MPGEMM_OK) return st;
    if ((size_t)K * N == 0) return MPGEMM_OK;
    if (codes == nullptr || scales == nullptr || packed_codes == nullptr ||
        packed_meta == nullptr)
        return MPGEMM_ERR_INVALID_ARG;
    if (!aligned16(codes) || !aligned16(scales) || (zeros && !aligned16(zeros)) ||
        !aligned16(packed_codes) || !aligned16(packed_meta))
        return MPGEMM_ERR_ALIGNMENT;
    return hip_status(mpgemm::launch_pack_w8(codes, scales, zeros, K, N, group, packed_codes,
                                             packed_meta, (hipStream_t)stream));
}

int mpgemm_unpack_w8(const void *packed_codes, const void *packed_meta, int K, int N, int group,
                     int symmetric, uint8_t *codes, uint16_t *scales, uint8_t *zeros,
                     void *stream) {
    if (symmetric != 0 && symmetric != 1) return MPGEMM_ERR_INVALID_ARG;
    const int st = check_shape(0, N, K, group);
    if (st != MPGEMM_OK) return st;
    if ((size_t)K * N == 0) return MPGEMM_OK;
    if (packed_codes == nullptr || packed_meta == nullptr || codes == nullptr ||
        scales == nullptr || (!symmetric && zeros == nullptr))
        return MPGEMM_ERR_INVALID_ARG;
    if (!aligned16(packed_codes) || !aligned16(packed_meta) || !aligned16(codes) ||
        !aligned16(scales) || (!symmetric && !aligned16(zeros)))
        return MPGEMM_ERR_ALIGNMENT;
    return hip_status(mpgemm::launch_unpack_w8(packed_codes, packed_meta, K, N, group, symmetric,
                                               codes, scales, zeros, (hipStream_t)stream));
}

int mpgemm_w8a16(const void *X, int dtype, const void *packed_codes, const void *packed_meta,
                 int M, int N, int K, int group, int symmetric, void *Y, void *workspace,
                 size_t workspace_bytes, void *stream) {
    return gemm_impl(mpgemm::kU8, X, dtype, packed_codes, packed_meta, M, N, K, group,
                     symmetric, Y, workspace, workspace_bytes, kConfigSelect, stream);
}

int mpgemm_w8a16_config(const void *X, int dtype, const void *packed_codes,
                        const void *packed_meta, int M, int N, int K, int group, int symmetric,
                        void *Y, void *workspace, size_t workspace_bytes, int config_id,
                        void *stream) {
    return gemm_impl(mpgemm::kU8, X, dtype, packed_codes, packed_meta, M, N, K, group,
                     symmetric, Y, workspace, workspace_bytes, config_id, stream);
}

int mpgemm_wfp8a16_config(const void *X, int dtype, int fp8_format, const void *packed_codes,
                          const void *packed_meta, int M, int N, int K, int group, void *Y,
                          void *workspace, size_t workspace_bytes, int config_id,
                          void *stream) {
    if (fp8_format != MPGEMM_FP8_E4M3 && fp8_format != MPGEMM_FP8_E5M2)
        return MPGEMM_ERR_INVALID_ARG;
    const int code = fp8_format == MPGEMM_FP8_E4M3 ? mpgemm::kE4M3 : mpgemm::kE5M2;
    return gemm_impl(code, X, dtype, packed_codes, packed_meta, M, N, K, group, 1, Y,
                     workspace, workspace_bytes, config_id, stream);
}

int mpgemm_wfp8a16(const void *X, int dtype, int fp8_format, const void *packed_codes,
                   const void *packed_meta, int M, int N, int K, int group, void *Y,
                   void *workspace, size_t workspace_bytes, void *stream) {
    return mpgemm_wfp8a16_config(X, dtype, fp8_format, packed_codes, packed_meta, M, N, K,
                                 group, Y, workspace, workspace_bytes, kConfigSelect, stream);
}

size_t mpgemm_packed_code_bytes_lowbit(int bits, int K, int N) {
    if ((bits != 2 && bits != 3) || check_shape(0, N, K, 128) != MPGEMM_OK) return 0;
    return (size_t)mpgemm::padded_k(K) * (size_t)mpgemm::padded_n(N) * bits / 8;
}

int mpgemm_pack_weights_lowbit(int bits, const uint8_t *codes, const uint16_t *scales,
                               const uint8_t *zeros, int K, int N, int group, void *packed_codes,
                               void *packed_meta, void *stream) {
    if (bits != 2 && bits != 3) return MPGEMM_ERR_INVALID_ARG;
    const int st = check_shape(0, N, K, group);
    if (st != MPGEMM_OK) return st;
    if ((size_t)K * N == 0) return MPGEMM_OK;
    if (codes == nullptr || scales == nullptr || packed_codes == nullptr ||
        packed_meta == nullptr)
        return MPGEMM_ERR_INVALID_ARG;
    if (!aligned16(codes) || !aligned16(scales) || (zeros && !aligned16(zeros)) ||
        !aligned16(packed_codes) || !aligned16(packed_meta))
        return MPGEMM_ERR_ALIGNMENT;
    return hip_status(mpgemm::launch_pack_lowbit(bits, codes, scales, zeros, K, N, group,
                                                 packed_codes, packed_meta, (hipStream_t)stream));
}

int mpgemm_unpack_lowbit(int bits, const void *packed_codes, const void *packed_meta, int K,
                         int N, int group, int symmetric, uint8_t *codes, uint16_t *scales,
                         uint8_t *zeros, void *stream) {
    if ((bits != 2 && bits != 3) || (symmetric != 0 && symmetric != 1))
        return MPGEMM_ERR_INVALID_ARG;
    const int st = check_shape(0, N, K, group);
    if (st != MPGEMM_OK) return st;
    if ((size_t)K * N == 0) return MPGEMM_OK;
    if (packed_codes == nullptr || packed_meta == nullptr || codes == nullptr ||
        scales == nullptr || (!symmetric && zeros == nullptr))
        return MPGEMM_ERR_INVALID_ARG;
    if (!aligned16(packed_codes) || !aligned16(packed_meta) || !aligned16(codes) ||
        !aligned16(scales) || (!symmetric && !aligned16(zeros)))
        return MPGEMM_ERR_ALIGNMENT;
    return hip_status(mpgemm::launch_unpack_lowbit(bits, packed_codes, packed_meta, K, N, group,
                                                   symmetric, codes, scales, zeros,
                                                   (hipStream_t)stream));
}

int mpgemm_wlowbit_a16_config(int bits, const void *X, int dtype, const void *packed_codes,
                              const void *packed_meta, int M, int N, int K, int group,
                              int symmetric, void *Y, void *workspace, size_t workspace_bytes,
                              int config_id, void *stream) {
    if (bits != 2 && bits != 3) return MPGEMM_ERR_INVALID_ARG;
    return gemm_impl(bits == 2 ? mpgemm::kU2 : mpgemm::kU3, X, dtype, packed_codes, packed_meta,
                     M, N, K, group, symmetric, Y, workspace, workspace_bytes, config_id, stream);
}

int mpgemm_wlowbit_a16(int bits, const void *X, int dtype, const void *packed_codes,
                       const void *packed_meta, int M, int N, int K, int group, int symmetric,
                       void *Y, void *workspace, size_t workspace_bytes, void *stream) {
    return mpgemm_wlowbit_a16_config(bits, X, dtype, packed_codes, packed_meta, M, N, K, group,
                                     symmetric, Y, workspace, workspace_bytes, kConfigSelect,
                                     stream);
}

// ------------------------------------------------------------ attention decode ------

}  // extern "C"

namespace {

bool kv_shape_ok(int Hkv, int D) { return Hkv >= 1 && Hkv <= 1024 && D >= 16 && D <= 256 && D % 16 == 0; }

// Blocks per split and splits per (sequence, KV head): about 1024 waves (one per SIMD at
// this kernel's register use), and at most 64 splits (a wider combine costs more than it
// saves).  Measured on MI355X, Llama-3-8B heads: this picks the best of 1..16 blocks per
// split for batch x context 1 x 8192, 1 x 32768, 8 x 4096, 16 x 2048 and 64 x 2048.
// MPGEMM_ATTN_BPS overrides the blocks per split (tuning sweeps).
void attn_plan(int B, int Hkv, int max_len, int *bps, int *splits) {
    const int64_t nblk = (max_len + 63) / 64;
    const int64_t total = (int64_t)B * Hkv * nblk;
    int64_t per = (total + 1023) / 1024;
    if (per < (nblk + 63) / 64) per = (nblk + 63) / 64;
    if (per < 1) per = 1;
    if (const char *env = getenv("MPGEMM_ATTN_BPS")) {
        const int v = atoi(env);
        if (v >= 1) per = v;
    }
    if (per < (nblk + 1023) / 1024) per = (nblk + 1023) / 1024;   // combine takes <= 1024 splits
    *bps = (int)per;
    *splits = nblk > 0 ? (int)((nblk + per - 1) / per) : 1;
}

bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

}  // namespace

extern "C" {

size_t mpgemm_kv_block_bytes(int Hkv, int D) {
    return kv_shape_ok(Hkv, D) ? (size_t)Hkv * (128 * (size_t)mpgemm::kv_padded_d(D) + 384) : 0;
}

int mpgemm_kv_pack(const uint8_t *kc, const uint16_t *ks, const uint8_t *kz, const uint8_t *vc,
                   const uint16_t *vs, const uint8_t *vz, int n_tokens, int t0, int Hkv, int D,
                   const int *table_row, int table_len, int num_blocks, void *cache,
                   void *stream) {
    if (!kv_shape_ok(Hkv, D)) return MPGEMM_ERR_UNSUPPORTED;
    if (n_tokens < 0 || t0 < 0 || table_len < 0 || num_blocks < 0) return MPGEMM_ERR_INVALID_ARG;
    if ((int64_t)t0 + n_tokens > (int64_t)table_len * 64) return MPGEMM_ERR_INVALID_ARG;
    if ((int64_t)n_tokens * Hkv >= kIndexLimit) return MPGEMM_ERR_UNSUPPORTED;
    if (n_tokens == 0) return MPGEMM_OK;
    if (!kc || !ks || !vc || !vs || !table_row || !cache || (!kz) != (!vz))
        return MPGEMM_ERR_INVALID_ARG;
    if (!aligned16(kc) || !aligned16(vc) || !aligned4(ks) || !aligned4(vs) || !aligned4(table_row) ||
        !aligned16(cache))
        return MPGEMM_ERR_ALIGNMENT;
    return hip_status(mpgemm::launch_kv_pack(kc, ks, kz, vc, vs, vz, n_tokens, t0, Hkv, D,
                                             table_row, table_len, num_blocks, cache,
                                             (hipStream_t)stream));
}

size_t mpgemm_attention_workspace_bytes(int B, int Hq, int Hkv, int D, int max_len) {
    if (B < 0 || max_len < 0 || !kv_shape_ok(Hkv, D) || Hq < Hkv || Hq % Hkv) return 0;
    int bps, splits;
    attn_plan(B, Hkv, max_len, &bps, &splits);
    return mpgemm::attn_part_bytes(B, Hq, D, splits);
}

}  // extern "C"

namespace {

int attention_impl(int kv_code, const void *Q, int dtype, const void *cache, int num_blocks,
                   const int *block_table, int table_stride, const int *lens, int B, int Hq,
                   int Hkv, int D, int max_len, float scale, void *O, void *workspace,
                   size_t workspace_bytes, void *stream) {
    if (dtype != MPGEMM_F16 && dtype != MPGEMM_BF16) return MPGEMM_ERR_INVALID_ARG;
    if (B < 0 || max_len < 0 || num_blocks < 0 || table_stride < 0 || Hkv < 1 || Hq < 1)
        return MPGEMM_ERR_INVALID_ARG;
    if (!kv_shape_ok(Hkv, D) || Hq % Hkv != 0 || Hq / Hkv > 16) return MPGEMM_ERR_UNSUPPORTED;
    if (!(scale == scale) || scale == INFINITY || scale == -INFINITY) return MPGEMM_ERR_INVALID_ARG;
    if ((int64_t)B * Hq * D >= kIndexLimit || (int64_t)B * table_stride >= kIndexLimit)
        return MPGEMM_ERR_UNSUPPORTED;
    if (B == 0) return MPGEMM_OK;
    if (!Q || !O || !lens || (max_len > 0 && (!cache || !block_table))) return MPGEMM_ERR_INVALID_ARG;
    if (!aligned16(Q) || !aligned16(O) || !aligned4(lens) || (cache && !aligned16(cache)) ||
        (block_table && !aligned4(block_table)))
        return MPGEMM_ERR_ALIGNMENT;
    mpgemm::AttnArgs a;
    attn_plan(B, Hkv, max_len, &a.bps, &a.splits);
    const size_t need = mpgemm::attn_part_bytes(B, Hq, D, a.splits);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
        return MPGEMM_ERR_WORKSPACE;
    a.Q = (const uint16_t *)Q;
    a.cache = (const uint8_t *)cache;
    a.num_blocks = cache ? num_blocks : 0;
    a.table = block_table;
    a.table_stride = block_table ? table_stride : 0;
    a.lens = lens;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    a.act = dtype == MPGEMM_BF16 ? mpgemm::kBF16 : mpgemm::kF16;
    a.kv_code = kv_code;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.O = (uint16_t *)O;
    a.part = (float *)workspace;
    if (getenv("MPGEMM_LOG"))
        fprintf(stderr, "mpgemm: attention B=%d Hq=%d Hkv=%d D=%d max_len=%d -> %d splits of %d blocks\n",
                B, Hq, Hkv, D, max_len, a.splits, a.bps);
    return hip_status(mpgemm::launch_attention_kv8(a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int mpgemm_attention_decode_kv8(const void *Q, int dtype, const void *cache, int num_blocks,
                                const int *block_table, int table_stride, const int *lens, int B,
                                int Hq, int Hkv, int D, int max_len, float scale, void *O,
                                void *workspace, size_t workspace_bytes, void *stream) {
    return attention_impl(mpgemm::kU8, Q, dtype, cache, num_blocks, block_table, table_stride,
                          lens, B, Hq, Hkv, D, max_len, scale, O, workspace, workspace_bytes,
                          stream);
}

int mpgemm_attention_decode_kvfp8(const void *Q, int dtype, int fp8_format, const void *cache,
                                  int num_blocks, const int *block_table, int table_stride,
                                  const int *lens, int B, int Hq, int Hkv, int D, int max_len,
                                  float scale, void *O, void *workspace, size_t workspace_bytes,
                                  void *stream) {
    if (fp8_format != MPGEMM_FP8_E4M3 && fp8_format != MPGEMM_FP8_E5M2) return MPGEMM_ERR_INVALID_ARG;
    return attention_impl(fp8_format == MPGEMM_FP8_E4M3 ? mpgemm::kE4M3 : mpgemm::kE5M2, Q, dtype,
                          cache, num_blocks, block_table, table_stride, lens, B, Hq, Hkv, D,
                          max_len, scale, O, workspace, workspace_bytes, stream);
}

int mpgemm_select_config(int M, int N, int K, int group, int dtype) {
    (void)dtype;
    return select_config(M < 0 ? 0 : M, N, K, group, mpgemm::kU4);
}

int mpgemm_prefill_schedule(int M, int N, int K, int config_id, int cus, int *info, int *work,
                            int capacity) {
    if (info == nullptr || M <= 0 || N <= 0 || K <= 0 || cus < 0 || capacity < 0)
        return MPGEMM_ERR_INVALID_ARG;
    if (!tiled_config(config_id)) return MPGEMM_ERR_INVALID_ARG;
    if (const int st = check_shape(M, N, K, 128)) return st;
    const int sh = config_id == kConfigPrefillX32Tall ? 1 : config_id == kConfigPrefillX32 ? 2 : 3;
    return mpgemm::x32_schedule(M, N, K, sh, cus, info, work, capacity);
}

int mpgemm_prefill_launches(int M, int N, int K, int config_id, int cus, int *split_column) {
    if (M <= 0 || N <= 0 || K <= 0 || cus < 0) return MPGEMM_ERR_INVALID_ARG;
    if (!tiled_config(config_id)) return MPGEMM_ERR_INVALID_ARG;
    if (const int st = check_shape(M, N, K, 128)) return st;
    const int n1 = config_id == kConfigPrefillX32Wide ? mpgemm::x32_wide_split_column(M, N, cus) : 0;
    if (split_column) *split_column = n1 ? n1 : N;
    return n1 ? 2 : 1;
}

const char *mpgemm_config_name(int config_id) {
    switch (config_id) {
        case kConfigDecode1: return "decode_splitk_m16";
        case kConfigDecode2: return "decode_splitk_m32";
        case kConfigDecode3: return "decode_splitk_m48";
        case kConfigDecode4: return "decode_splitk_m64";
        case kConfigPrefillX32: return "prefill_x32_128x256";
        case kConfigPrefillX32Tall: return "prefill_x32_256x128";
        case kConfigPrefillX32Wide: return "prefill_x32_256x256";
        default: return "";
    }
}

const char *mpgemm_status_string(int status) {
    switch (status) {
        case MPGEMM_OK: return "MPGEMM_OK";
        case MPGEMM_ERR_INVALID_ARG: return "MPGEMM_ERR_INVALID_ARG: null pointer, negative size or bad enum";
        case MPGEMM_ERR_UNSUPPORTED: return "MPGEMM_ERR_UNSUPPORTED: shape or group size outside the supported limits";
        case MPGEMM_ERR_ALIGNMENT: return "MPGEMM_ERR_ALIGNMENT: a device pointer is not 16-byte aligned";
        case MPGEMM_ERR_WORKSPACE: return "MPGEMM_ERR_WORKSPACE: workspace too small";
        case MPGEMM_ERR_HIP: return "MPGEMM_ERR_HIP: the HIP runtime reported an error";
        default: return "unknown mpgemm status";
    }
}

}  // extern "C"
