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
    int Ny, uint16_t *__restrict__ Y) {
    // N: the padded column count of the packed planes; Ny: output row length (the user N).
    typedef typename Dq<ACT>::type DqT;
    constexpr int GPT = kTileK / G;               // groups per 128-k tile (1 or 2)
    __shared__ u32x4_t xs[2][kXChunks];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int m_blk = blockIdx.y * kBM;
    const int KT = K >> 7;
    const int groups = K / G;
    const int strips = N >> 4;
    const int strip0 = blockIdx.x * (kBN / 16) + wave * 4;

    const rsrc_t xrs = make_rsrc(X, (uint32_t)((size_t)M * K * 2));
    const rsrc_t wrs = make_rsrc(codes, (uint32_t)((size_t)strips * KT * 1024));
    const rsrc_t srs = make_rsrc(scales, (uint32_t)((size_t)groups * N * 2));
    const rsrc_t zrs = make_rsrc(zeros, (uint32_t)((size_t)groups * N / 2));

    // Per-thread byte offsets, fixed for the whole K loop (a wave-uniform scalar offset
    // advances them).  Activation rows past M point one row past the end of X and read as
    // zero; strips past N read the last real strip.  Their products land only in
    // accumulators that are never stored (row m of Y depends on row m of X alone, strip s
    // on strip s of W alone).  A lane's meta element is a multiple of 16 plus lane % 16,
    // so its scale is half (lane & 1) of a dword and its zero nibble (lane & 7) of a dword.
    uint32_t xoff[kXLoads];
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
        const int c = tid + kThreads * i;
        const uint32_t row = (uint32_t)min(m_blk + c / kChunksPerRow, M);
        xoff[i] = (row * K + (c % kChunksPerRow) * 8) * 2u;
    }
    bool valid[4];
    uint32_t woff[4], soff[4], zoff[4];
#pragma unroll
    for (int si = 0; si < 4; ++si) {
        valid[si] = (strip0 + si) < strips;
        const uint32_t strip = (uint32_t)min(strip0 + si, strips - 1);
        woff[si] = strip * KT * 1024u + lane * 16u;
        const uint32_t e = strip * groups * 16u + (lane & 15);
        soff[si] = (e >> 1) * 4u;
        zoff[si] = (e >> 3) * 4u;
    }
    const uint32_t sshift = (lane & 1) * 16;
    const uint32_t zshift = (lane & 7) * 4;

    f32x4_t acc[4][8];
#pragma unroll
    for (int si = 0; si < 4; ++si)
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) acc[si][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // X stage: one 64-deep half of a 128-deep tile.
    auto load_x = [&](int half_step, u32x4_t(&xr)[kXLoads]) {
#pragma unroll
        for (int i = 0; i < kXLoads; ++i) xr[i] = buf_load_b128(xrs, xoff[i], half_step * kBK * 2);
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
    // Weights and raw meta of one 128-deep tile: 16 bytes per lane per strip.
    auto load_w = [&](int t, u32x4_t(&wr)[4], uint32_t(&sr)[4][GPT], uint32_t(&zr)[4][GPT]) {
#pragma unroll
        for (int si = 0; si < 4; ++si) {
            wr[si] = buf_load_b128(wrs, woff[si], t * 1024);
#pragma unroll
            for (int h = 0; h < GPT; ++h) {
                sr[si][h] = buf_load_b32(srs, soff[si], (t * GPT + h) * 32);
                zr[si][h] = SYM ? 0u : buf_load_b32(zrs, zoff[si], (t * GPT + h) * 8);
            }
        }
    };
    // 64-deep half `half` of the current tile from LDS buffer `buf`.
    auto compute_half = [&](int buf, int half, const u32x4_t(&wr)[4], const DqT(&dq)[4][GPT]) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int word = half * 2 + s;
            // All eight activation operands of this 32-deep step are requested first; the
            // dequantization below then covers their LDS latency.
            u32x4_t b[8];
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) {
                const int r = mb * 16 + (lane & 15);
                const int c = s * 4 + (lane >> 4);
                b[mb] = xs[buf][r * kChunksPerRow + (c ^ (r & 7))];
            }
            u32x4_t a[4];
#pragma unroll
            for (int si = 0; si < 4; ++si) a[si] = Dq<ACT>::word(wr[si][word], dq[si][(word * 32) / G]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
#pragma unroll
                for (int si = 0; si < 4; ++si) acc[si][mb] = mfma16x16x32<ACT>(a[si], b[mb], acc[si][mb]);
        }
    };

    // Weight/meta registers ping-pong between two sets (tile t computes from one set while
    // tile t+1 is loaded into the other), so nothing is copied between iterations.
    struct WSet {
        u32x4_t w[4];
        uint32_t s[4][GPT], z[4][GPT];
    };
    u32x4_t xr[kXLoads];
    WSet set0, set1;

    // Tile t: compute from `cur` while `nxt` receives tile tn.  Its two 64-deep halves use
    // the two LDS buffers; every iteration ends with the X stage of tile tn in buffer 0.
    auto tile = [&](int t, int tn, const WSet &cur, WSet &nxt) {
        load_x(2 * t + 1, xr);
        load_w(tn, nxt.w, nxt.s, nxt.z);
        __builtin_amdgcn_sched_barrier(0);       // next loads go out before this tile's MFMAs
        DqT dq[4][GPT];
#pragma unroll
        for (int si = 0; si < 4; ++si)
#pragma unroll
            for (int h = 0; h < GPT; ++h)
                dq[si][h] = Dq<ACT>::make((uint16_t)(cur.s[si][h] >> sshift),
                                          SYM ? 8u : ((cur.z[si][h] >> zshift) & 0xFu));
        compute_half(0, 0, cur.w, dq);
        store_x(1, xr);
        __syncthreads();
        load_x(2 * tn, xr);
        __builtin_amdgcn_sched_barrier(0);
        compute_half(1, 1, cur.w, dq);
        store_x(0, xr);
        __syncthreads();
    };

    load_x(0, xr);
    store_x(0, xr);
    load_w(0, set0.w, set0.s, set0.z);
    __syncthreads();

    // The loop body is one basic block; past the last tile the prefetches clamp onto it.
    int t = 0;
    for (; t + 1 < KT; t += 2) {
        tile(t, t + 1, set0, set1);
        tile(t + 1, min(t + 2, KT - 1), set1, set0);
    }
    if (t < KT) tile(t, t, set0, set1);

#pragma unroll
    for (int si = 0; si < 4; ++si) {
        if (!valid[si]) continue;
        const int n = (strip0 + si) * 16 + 4 * (lane >> 4);
        if (n >= Ny) continue;
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            const int m = m_blk + mb * 16 + (lane & 15);
            if (m < M) store4<ACT>(Y + (size_t)m * Ny + n, Ny - n, acc[si][mb]);
        }
    }
}

template <int ACT, bool SYM, int G>
void launch_one(const GemmArgs &a, hipStream_t stream) {
    const dim3 grid((a.Np + kBN - 1) / kBN, (a.M + kBM - 1) / kBM);
    prefill_kernel<ACT, SYM, G><<<grid, dim3(kThreads), 0, stream>>>(
        a.X, a.codes, a.scales, a.zeros, a.M, a.Np, a.K, a.N, a.Y);
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
