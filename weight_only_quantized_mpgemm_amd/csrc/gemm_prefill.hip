// Large-M (prefill) W4A16 GEMM for gfx950.
//
// [TurboMind, technique (iii), Fig. 9 caption]: a software-pipelined main loop keeps the
// matrix cores busy on tile k with already-dequantized fragments while the integer/float
// ALUs dequantize and the memory pipeline fetches later tiles.  Source: "LMDeploy
// Accelerates Mixed-Precision LLM Inference with TurboMind" (arXiv 2508.15601).
//
// At M >= 128 the GEMM is bound by the matrix cores.  Design for MI355X:
//   - workgroup tile 128 (m) x 256 (n), four waves side by side along n; each wave owns a
//     128 x 64 block = 8 x 4 MFMA 16x16x32 blocks (128 fp32 accumulators per lane), so
//     every dequantized weight fragment feeds 8 MFMAs and the dequantization VALU work is
//     about half of the MFMA time (the ratio falls as 60 / wave-M);
//   - weights go straight from HBM into registers (one 64-bit load per lane per strip per
//     64-k step, the lane's half of its 16-byte tile slice) and are dequantized in
//     registers; each wave owns its strips, so no weight byte is loaded twice per workgroup;
//   - activations are shared by the four waves through LDS: 128 x 64 fp16 tiles, double
//     buffered (one barrier per step), rows XOR-swizzled in 16-byte chunks (chunk ^ row%8)
//     so the 16-byte operand reads of 8 consecutive lanes (8 rows, one chunk) hit 8
//     distinct bank groups;
//   - the 64-k step never crosses a quantization group (g is 64 or 128), so each lane needs
//     one scale/zero per strip per step.
#include "kernels.hpp"

namespace mpgemm {

namespace {

constexpr int kBM = 128;
constexpr int kBN = 256;
constexpr int kBK = 64;
constexpr int kThreads = 256;
constexpr int kChunksPerRow = kBK / 8;                // 16-byte chunks per LDS row
constexpr int kXChunks = kBM * kChunksPerRow;         // per buffer
constexpr int kXLoads = kXChunks / kThreads;          // 16-byte loads per thread per step

template <int ACT, bool SYM, int G>
__global__ __launch_bounds__(kThreads) void prefill_kernel(
    const uint16_t *__restrict__ X, const uint32_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros, int M, int N, int K,
    uint16_t *__restrict__ Y) {
    typedef typename Dq<ACT>::type DqT;
    __shared__ u32x4_t xs[2][kXChunks];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int m_blk = blockIdx.y * kBM;
    const int KT = K >> 7;
    const int steps = K / kBK;
    const int groups = K / G;
    const int strips = N >> 4;
    const int strip0 = blockIdx.x * (kBN / 16) + wave * 4;

    // Loads never branch: rows past M and strips past N are clamped onto the last real
    // ones.  The products they feed land only in accumulators that are never stored
    // (row m of Y depends on row m of X alone, strip s on strip s of W alone).
    bool valid[4];
    size_t wstrip[4];
#pragma unroll
    for (int si = 0; si < 4; ++si) {
        valid[si] = (strip0 + si) < strips;
        wstrip[si] = (size_t)min(strip0 + si, strips - 1);
    }

    f32x4_t acc[4][8];
#pragma unroll
    for (int si = 0; si < 4; ++si)
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) acc[si][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto load_x = [&](int step, u32x4_t(&xr)[kXLoads]) {
        const int k0 = step * kBK;
#pragma unroll
        for (int i = 0; i < kXLoads; ++i) {
            const int c = tid + kThreads * i;
            const int r = c / kChunksPerRow;
            const int ch = c % kChunksPerRow;
            const int m = min(m_blk + r, M - 1);
            xr[i] = *reinterpret_cast<const u32x4_t *>(X + (size_t)m * K + k0 + ch * 8);
        }
    };
    auto store_x = [&](int buf, const u32x4_t(&xr)[kXLoads]) {
#pragma unroll
        for (int i = 0; i < kXLoads; ++i) {
            const int c = tid + kThreads * i;
            const int r = c / kChunksPerRow;
            const int ch = c % kChunksPerRow;
            xs[buf][r * kChunksPerRow + (ch ^ (r & 7))] = xr[i];
        }
    };
    // Raw scale bits and zero byte are kept as loaded; the dequantization constants are
    // formed only when the step that needs them starts, so nothing waits on the loads early.
    // The zero's nibble (element index e odd/even) is the lane's n parity: e%2 == lane%2.
    const uint32_t zshift = (lane & 1) * 4;
    auto load_w = [&](int step, u32x2_t(&wr)[4], uint32_t(&sr)[4], uint32_t(&zr)[4]) {
        const int k0 = step * kBK;
        const int tile = k0 >> 7;
        const int word0 = (k0 & 127) >> 5;            // 0 or 2
        const int grp = k0 / G;
#pragma unroll
        for (int si = 0; si < 4; ++si) {
            const size_t strip = wstrip[si];
            wr[si] = *reinterpret_cast<const u32x2_t *>(
                codes + (strip * KT + tile) * kTileWords + lane * 4 + word0);
            const size_t e = strip * groups * 16 + (size_t)grp * 16 + (lane & 15);
            sr[si] = scales[e];
            zr[si] = SYM ? 0u : zeros[e >> 1];
        }
    };
    auto make_dq = [&](const uint32_t(&sr)[4], const uint32_t(&zr)[4], DqT(&dq)[4]) {
#pragma unroll
        for (int si = 0; si < 4; ++si)
            dq[si] = Dq<ACT>::make((uint16_t)sr[si], SYM ? 8u : ((zr[si] >> zshift) & 0xFu));
    };

    u32x4_t xr[kXLoads];
    u32x2_t wcur[4], wnext[4];
    uint32_t scur[4], snext[4], zcur[4], znext[4];

    load_x(0, xr);
    store_x(0, xr);
    load_w(0, wcur, scur, zcur);
    __syncthreads();

    // The loop body is one basic block (no data-dependent branches), which keeps the
    // accumulators in place across iterations.  The last step prefetches a redundant copy
    // of itself into the idle buffer instead of branching.
    for (int step = 0; step < steps; ++step) {
        const int buf = step & 1;
        const int next = min(step + 1, steps - 1);
        load_x(next, xr);
        load_w(next, wnext, snext, znext);
        // Keep the next step's loads ahead of this step's MFMAs: they then have a whole
        // step of matrix work to arrive in.
        __builtin_amdgcn_sched_barrier(0);
        DqT dcur[4];
        make_dq(scur, zcur, dcur);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            u32x4_t a[4];
#pragma unroll
            for (int si = 0; si < 4; ++si) a[si] = Dq<ACT>::word(wcur[si][s], dcur[si]);
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) {
                const int r = mb * 16 + (lane & 15);
                const int c = s * 4 + (lane >> 4);
                const u32x4_t b = xs[buf][r * kChunksPerRow + (c ^ (r & 7))];
#pragma unroll
                for (int si = 0; si < 4; ++si) acc[si][mb] = mfma16x16x32<ACT>(a[si], b, acc[si][mb]);
            }
        }
        store_x(buf ^ 1, xr);
#pragma unroll
        for (int si = 0; si < 4; ++si) {
            wcur[si] = wnext[si];
            scur[si] = snext[si];
            zcur[si] = znext[si];
        }
        __syncthreads();
    }

#pragma unroll
    for (int si = 0; si < 4; ++si) {
        if (!valid[si]) continue;
        const int n = (strip0 + si) * 16 + 4 * (lane >> 4);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            const int m = m_blk + mb * 16 + (lane & 15);
            if (m < M) *reinterpret_cast<u32x2_t *>(Y + (size_t)m * N + n) = round4<ACT>(acc[si][mb]);
        }
    }
}

template <int ACT, bool SYM, int G>
void launch_one(const GemmArgs &a, hipStream_t stream) {
    const dim3 grid((a.N + kBN - 1) / kBN, (a.M + kBM - 1) / kBM);
    prefill_kernel<ACT, SYM, G><<<grid, dim3(kThreads), 0, stream>>>(
        a.X, a.codes, a.scales, a.zeros, a.M, a.N, a.K, a.Y);
}

template <int ACT>
void launch_act(const GemmArgs &a, hipStream_t stream) {
    const bool sym = a.zeros == nullptr;
    if (a.group == 128) {
        sym ? launch_one<ACT, true, 128>(a, stream) : launch_one<ACT, false, 128>(a, stream);
    } else {
        sym ? launch_one<ACT, true, 64>(a, stream) : launch_one<ACT, false, 64>(a, stream);
    }
}

__global__ void fill_zero_kernel(uint16_t *__restrict__ Y, size_t count) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) Y[i] = 0;
}

}  // namespace

hipError_t launch_prefill(const GemmArgs &a, hipStream_t stream) {
    if (a.act == kBF16) {
        launch_act<kBF16>(a, stream);
    } else {
        launch_act<kF16>(a, stream);
    }
    return hipGetLastError();
}

hipError_t launch_fill_zero(uint16_t *Y, size_t count, hipStream_t stream) {
    if (count) {
        const unsigned threads = 256;
        fill_zero_kernel<<<(unsigned)((count + threads - 1) / threads), threads, 0, stream>>>(Y, count);
    }
    return hipGetLastError();
}

}  // namespace mpgemm
