// Small-M (decode) W4A16 GEMM for gfx950.
//
// [TurboMind, GEMM pipeline; Fig. 6 and Fig. 9 captions]: the packed 4-bit weights are
// loaded straight into registers, turned into 16-bit values by I2F conversion and scaling,
// and fed to the matrix cores while the next tiles' loads are in flight.  Source: "LMDeploy
// Accelerates Mixed-Precision LLM Inference with TurboMind" (arXiv 2508.15601).
//
// At M <= 64 the GEMM is bound by HBM bandwidth: every weight byte is read once and used
// for at most M multiply-adds.  Design for MI355X:
//   - one workgroup per 16-column strip; its NW waves split the strip's K range into
//     contiguous slices (split-K inside the workgroup), so even N = 4096 gives 256
//     workgroups x 8 waves and every CU has several KiB of weight loads in flight;
//   - each lane fetches its 16 bytes of a 1 KiB tile with one 128-bit load (a wave reads
//     1 KiB contiguously); U tiles are requested before any is used;
//   - weights are the MFMA A operand (rows = n), activations the B operand (columns = m),
//     read as one 16-byte row chunk per lane from L2 (they are small and shared by all
//     workgroups);
//   - the NW partial sums meet in LDS and are added in a fixed wave order, so results are
//     deterministic; no global workspace and no atomics.
#include "kernels.hpp"

namespace mpgemm {

namespace {

constexpr int kDecodeWaves = 8;

template <int ACT, int MB, bool SYM, int G, int NW, int U>
__global__ __launch_bounds__(NW * 64) void decode_kernel(
    const uint16_t *__restrict__ X, const uint32_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros, int M, int N, int K,
    uint16_t *__restrict__ Y) {
    constexpr int GPT = kTileK / G;              // groups per 128-k tile (1 or 2)
    typedef typename Dq<ACT>::type DqT;

    const int strip = blockIdx.x;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int KT = K >> 7;
    const int t_begin = (KT * wave) / NW;
    const int t_end = (KT * (wave + 1)) / NW;
    const int groups = K / G;

    const u32x4_t *tiles =
        reinterpret_cast<const u32x4_t *>(codes) + (size_t)strip * KT * 64 + lane;
    const size_t meta_lane = (size_t)strip * groups * 16 + (lane & 15);
    const int mrow = lane & 15;
    const int ksub = (lane >> 4) * 8;

    f32x4_t acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int t0 = t_begin; t0 < t_end; t0 += U) {
        u32x4_t w[U];
        DqT dq[U][GPT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0 + u;
            if (t < t_end) {
                w[u] = tiles[(size_t)t * 64];
#pragma unroll
                for (int h = 0; h < GPT; ++h) {
                    const size_t e = meta_lane + (size_t)(t * GPT + h) * 16;
                    const uint32_t z = SYM ? 8u : read_zero(zeros, e);
                    dq[u][h] = Dq<ACT>::make(scales[e], z);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0 + u;
            if (t < t_end) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const u32x4_t a = Dq<ACT>::word(w[u][j], dq[u][(j * 32) / G]);
                    const int k = t * kTileK + 32 * j + ksub;
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        // Rows past M read the last real row: their products land in
                        // output columns that are never stored.
                        const int m = min(mb * 16 + mrow, M - 1);
                        const u32x4_t b = *reinterpret_cast<const u32x4_t *>(X + (size_t)m * K + k);
                        acc[mb] = mfma16x16x32<ACT>(a, b, acc[mb]);
                    }
                }
            }
        }
    }

    __shared__ f32x4_t red[NW * MB * 64];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) red[(wave * MB + mb) * 64 + lane] = acc[mb];
    __syncthreads();
    for (int mb = wave; mb < MB; mb += NW) {
        f32x4_t s = red[mb * 64 + lane];
        for (int w2 = 1; w2 < NW; ++w2) s += red[(w2 * MB + mb) * 64 + lane];
        const int m = mb * 16 + mrow;
        if (m < M) {
            const int n = strip * 16 + 4 * (lane >> 4);
            *reinterpret_cast<u32x2_t *>(Y + (size_t)m * N + n) = round4<ACT>(s);
        }
    }
}

template <int ACT, int MB, bool SYM, int G>
void launch_one(const GemmArgs &a, hipStream_t stream) {
    constexpr int NW = kDecodeWaves;
    const int KT = a.K >> 7;
    const dim3 grid(a.N >> 4), block(NW * 64);
    if (KT >= 8 * NW) {
        decode_kernel<ACT, MB, SYM, G, NW, 8><<<grid, block, 0, stream>>>(
            a.X, a.codes, a.scales, a.zeros, a.M, a.N, a.K, a.Y);
    } else {
        decode_kernel<ACT, MB, SYM, G, NW, 4><<<grid, block, 0, stream>>>(
            a.X, a.codes, a.scales, a.zeros, a.M, a.N, a.K, a.Y);
    }
}

template <int ACT, int MB>
void launch_mb(const GemmArgs &a, hipStream_t stream) {
    const bool sym = a.zeros == nullptr;
    if (a.group == 128) {
        sym ? launch_one<ACT, MB, true, 128>(a, stream) : launch_one<ACT, MB, false, 128>(a, stream);
    } else {
        sym ? launch_one<ACT, MB, true, 64>(a, stream) : launch_one<ACT, MB, false, 64>(a, stream);
    }
}

template <int ACT>
void launch_act(const GemmArgs &a, int mblocks, hipStream_t stream) {
    switch (mblocks) {
        case 1: launch_mb<ACT, 1>(a, stream); break;
        case 2: launch_mb<ACT, 2>(a, stream); break;
        case 3: launch_mb<ACT, 3>(a, stream); break;
        default: launch_mb<ACT, 4>(a, stream); break;
    }
}

}  // namespace

hipError_t launch_decode(const GemmArgs &a, int mblocks, hipStream_t stream) {
    if (a.act == kBF16) {
        launch_act<kBF16>(a, mblocks, stream);
    } else {
        launch_act<kF16>(a, mblocks, stream);
    }
    return hipGetLastError();
}

}  // namespace mpgemm
