// Large-M (prefill) W4A16 GEMM for gfx950: LDS ring fed by direct-to-LDS loads, and a
// software-pipelined inner loop.
//
// [TurboMind, technique (iii), Fig. 9 caption]: a software-pipelined main loop keeps the
// matrix cores busy on step k with already-dequantized fragments while the integer/float
// ALUs dequantize step k+1 and the memory pipeline fetches later tiles.  Source: "LMDeploy
// Accelerates Mixed-Precision LLM Inference with TurboMind" (arXiv 2508.15601).
//
// Design for MI355X (requires K % 256 == 0; other K use the two-buffer kernel):
//   - workgroup tile 128 (m) x 256 (n), four waves side by side along n, each owning a
//     128 x 64 block (8 x 4 MFMA 16x16x32 blocks, 128 fp32 accumulators per lane); every
//     dequantized weight fragment feeds 8 MFMAs;
//   - activations: a ring of four 128 x 64 fp16 LDS stages (64 KiB).  Each stage is filled
//     by buffer_load_dwordx4 ... lds (HBM/L2 straight into LDS, no register staging),
//     issued three stages ahead; each wave DMAs four 1 KiB blocks per stage.  (The kernel is
//     written for an eight-stage ring as well; measured, the deeper ring bought nothing.)  Rows are
//     XOR-swizzled in 16-byte chunks (chunk ^ row % 8) by choosing each lane's source
//     address, so the LDS block stays contiguous while the operand reads of eight
//     consecutive lanes hit eight distinct bank groups.  One barrier per stage: a wave
//     waits for its own DMA of the next stage, then the barrier makes every wave's DMA
//     visible and frees the stage about to be refilled;
//   - weights: one 128-bit buffer load per lane per strip per 128-deep tile, one tile
//     ahead, in two register sets that alternate between tiles;
//   - inner loop over 32-deep MFMA steps: while step s runs its 32 MFMAs, step s+1's
//     weight fragments are dequantized (VALU) and its activation operands are read from
//     LDS; the accumulators stay in place in AGPRs (inline-asm MFMA, see mfma_acc).
#include "kernels.hpp"

namespace mpgemm {

namespace {

constexpr int kRBM = 128;
constexpr int kRBN = 256;
constexpr int kRThreads = 256;
constexpr int kRStages = 4;                  // 64-deep LDS stages in the ring
constexpr int kRWSets = kRStages / 2;        // weight register sets (tiles in flight)
constexpr int kRChunks = kRBM * 8;           // 16-byte chunks per stage (8 per 64-deep row)

template <int N>
struct IC {
    static constexpr int value = N;
};

// Wait until at most n vector-memory operations of this wave are outstanding, then meet
// the rest of the workgroup.  The memory clobber keeps the compiler from moving LDS
// accesses across it; no implicit fence (and no wait for all loads) is added.
template <int NV>
__device__ __forceinline__ void wait_vm_barrier() {
    static_assert(NV >= 0 && NV < 64, "vmcnt range");
    constexpr int imm = (NV & 15) | ((NV >> 4) << 14) | (7 << 4) | (15 << 8);
    asm volatile("s_waitcnt %0\n\ts_barrier" ::"n"(imm) : "memory");
}

// In-place accumulation c += a * b with the accumulator pinned to AGPRs.  (The compiler's
// builtin form renames accumulators between MFMAs and pays a copy per MFMA.)  Written as
// inline asm, the MFMA is invisible to the compiler's hazard tracking, so every caller
// separates it from VALU writes of its sources with s_nop padding (see step_fence), and
// the main loop drains the matrix pipeline (mfma_drain) before any code after it.
template <int ACT>
__device__ __forceinline__ void mfma_acc(f32x4_t &c, const u32x4_t &a, const u32x4_t &b);
template <>
__device__ __forceinline__ void mfma_acc<kF16>(f32x4_t &c, const u32x4_t &a, const u32x4_t &b) {
    asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
template <>
__device__ __forceinline__ void mfma_acc<kBF16>(f32x4_t &c, const u32x4_t &a, const u32x4_t &b) {
    asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// One 32-bit packed word dequantized in eight pieces, so the work can be spread between
// MFMAs (piece p runs after MFMA p of its 8-MFMA window).  Same arithmetic as
// Dq<ACT>::word: fp16 pieces 0-3 isolate the four (k, k+1) pairs as 1024+q / 64+q, pieces
// 4-7 subtract the zero and scale (one rounding); bf16 spreads the nibbles to bytes, forms
// (q - z) * s exactly in fp32 and rounds once to bf16.
struct PieceTmp {
    uint32_t a, b, c, d;
};
template <int ACT>
__device__ __forceinline__ void dq_piece(int p, uint32_t w, const typename Dq<ACT>::type &d,
                                         PieceTmp &t, u32x4_t &out);
template <>
__device__ __forceinline__ void dq_piece<kF16>(int p, uint32_t w, const DqF16 &d, PieceTmp &t,
                                               u32x4_t &out) {
    const half2_t s2 = bitcast<half2_t>(d.s2);
    switch (p) {
        case 0: t.a = and_or(w, 0x000F000Fu, 0x64006400u); break;
        case 1: t.b = and_or(w, 0x00F000F0u, 0x54005400u); break;
        case 2: t.c = and_or(w >> 8, 0x000F000Fu, 0x64006400u); break;
        case 3: t.d = and_or(w >> 8, 0x00F000F0u, 0x54005400u); break;
        case 4: out[0] = bitcast<uint32_t>((bitcast<half2_t>(t.a) + bitcast<half2_t>(d.nz_hi2)) * s2); break;
        case 5: out[1] = bitcast<uint32_t>((bitcast<half2_t>(t.b) + bitcast<half2_t>(d.nz_lo2)) * s2); break;
        case 6: out[2] = bitcast<uint32_t>((bitcast<half2_t>(t.c) + bitcast<half2_t>(d.nz_hi2)) * s2); break;
        default: out[3] = bitcast<uint32_t>((bitcast<half2_t>(t.d) + bitcast<half2_t>(d.nz_lo2)) * s2); break;
    }
}
template <>
__device__ __forceinline__ void dq_piece<kBF16>(int p, uint32_t w, const DqBF16 &d, PieceTmp &t,
                                                u32x4_t &out) {
    // lo bytes: e0 e4 e1 e5; hi bytes: e2 e6 e3 e7 (see dequant_word_bf16)
    switch (p) {
        case 0: t.a = w & 0x0F0F0F0Fu; t.b = (w >> 4) & 0x0F0F0F0Fu; break;
        case 1: out[0] = pack_bf16x2(__builtin_fmaf(ubyte(t.a, 0), d.s, d.nzs),
                                     __builtin_fmaf(ubyte(t.a, 2), d.s, d.nzs)); break;
        case 2: out[1] = pack_bf16x2(__builtin_fmaf(ubyte(t.b, 0), d.s, d.nzs),
                                     __builtin_fmaf(ubyte(t.b, 2), d.s, d.nzs)); break;
        case 3: out[2] = pack_bf16x2(__builtin_fmaf(ubyte(t.a, 1), d.s, d.nzs),
                                     __builtin_fmaf(ubyte(t.a, 3), d.s, d.nzs)); break;
        case 4: out[3] = pack_bf16x2(__builtin_fmaf(ubyte(t.b, 1), d.s, d.nzs),
                                     __builtin_fmaf(ubyte(t.b, 3), d.s, d.nzs)); break;
        default: break;
    }
}

// Step boundary: no instruction moves across it, and five wait states separate the last
// VALU writes / MFMA source reads of one 32-deep step from the MFMAs of the next.
__device__ __forceinline__ void step_fence() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 4" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <int ACT, bool SYM, int G, int NST, int NWS>
__global__ __launch_bounds__(kRThreads) void prefill_ring_kernel(
    const uint16_t *__restrict__ X, const uint32_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros, int M, int N, int K,
    int Ny, uint16_t *__restrict__ Y) {
    // N: the padded column count of the packed planes; Ny: output row length (the user N).
    typedef typename Dq<ACT>::type DqT;
    constexpr int GPT = kTileK / G;          // groups per 128-deep tile (1 or 2)
    // Loads each wave issues per weight tile: codes + scales (+ zeros), four strips.
    constexpr int kWLoads = 4 * (1 + GPT * (SYM ? 1 : 2));
    // Stage j issues the DMA of stage j + NST - 1 and, when j is even, the weights of tile
    // j/2 + NWS - 1 (the tiles 0 .. NWS-2 come from the prologue, so NWS = NST / 2).  Stage
    // j needs the DMA of stage j + 1, issued at stage j + 2 - NST; the wave issued at least
    // the DMAs of the NST - 3 stages after it since (4 loads each).  vmcnt counts a wave's
    // loads in issue order, so leaving at most that many in flight finds stage j + 1 in
    // LDS.  The weight loads are not counted: the compiler may move them (their memory
    // never changes) or drop them when dead, as in the final stages; DMAs write LDS and
    // stay where they are.  (This over-waits a little when weights follow the last DMA.)
    static_assert(NWS * 2 == NST && (NST == 4 || NST == 8), "ring shape");
    constexpr int kWait = 4 * (NST - 3);
    // Before stage 0: stage 0's DMA, followed by the DMAs of stages 1 .. NST-2 (tile 0's
    // weights are waited for by the compiler where they are used).
    constexpr int kProWait = 4 * (NST - 2);
    (void)kWLoads;
    __shared__ u32x4_t xs[NST][kRChunks];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int m_blk = blockIdx.y * kRBM;
    const int KT = K >> 7;                   // 128-deep weight tiles
    const int S = K >> 6;                    // 64-deep stages (a multiple of 4)
    const int groups = K / G;
    const int strips = N >> 4;
    const int strip0 = blockIdx.x * (kRBN / 16) + wave * 4;

    const rsrc_t xrs = make_rsrc(X, (uint32_t)((size_t)M * K * 2));
    const rsrc_t wrs = make_rsrc(codes, (uint32_t)((size_t)strips * KT * 1024));
    const rsrc_t srs = make_rsrc(scales, (uint32_t)((size_t)groups * N * 2));
    const rsrc_t zrs = make_rsrc(zeros, (uint32_t)((size_t)groups * N / 2));

    // DMA source offsets.  Wave w fills blocks b = 4w + i (i < 4) of every stage; block b
    // holds rows 8b .. 8b+7, and lane l writes LDS chunk 64b + l = (row 8b + l/8, physical
    // chunk l%8), which holds logical chunk (l%8) ^ (row%8) = (l%8) ^ (l/8).  Rows past M
    // point one row past the end of X and read zeros.
    uint32_t xoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * (wave * 4 + i) + (lane >> 3);
        const uint32_t row = (uint32_t)min(m_blk + r, M);
        xoff[i] = (row * K + (((lane & 7) ^ (lane >> 3)) * 8)) * 2u;
    }
    // Weight and meta offsets (strips past N read the last real strip; never stored).
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
    // LDS chunk index of this lane's operand row for row block 0; step s adds its chunk.
    const int brow = (lane & 15) * 8;
    const int bsw = lane & 7;                // row % 8 of every row this lane reads

    f32x4_t acc[4][8];
#pragma unroll
    for (int si = 0; si < 4; ++si)
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) acc[si][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    struct WSet {
        u32x4_t w[4];
        uint32_t s[4][GPT], z[4][GPT];
    };
    WSet ws[NWS];
    DqT dq[2][4][GPT];
    u32x4_t A[2][4], B[2][8];

    auto dma = [&](int st, auto buf) __attribute__((always_inline)) {
        const uint32_t soff_k = (uint32_t)min(st, S - 1) * 128u;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xrs, (__attribute__((address_space(3))) void *)&xs[decltype(buf)::value][(wave * 4 + i) * 64],
                16, xoff[i], soff_k, 0, 0);
    };
    auto load_w = [&](int t, WSet &w) __attribute__((always_inline)) {
        t = min(t, KT - 1);
#pragma unroll
        for (int si = 0; si < 4; ++si) {
            w.w[si] = buf_load_b128(wrs, woff[si], t * 1024);
#pragma unroll
            for (int h = 0; h < GPT; ++h) {
                w.s[si][h] = buf_load_b32(srs, soff[si], (t * GPT + h) * 32);
                if (!SYM) w.z[si][h] = buf_load_b32(zrs, zoff[si], (t * GPT + h) * 8);
            }
        }
    };
    auto make_dq = [&](const WSet &w, DqT(&d)[4][GPT]) __attribute__((always_inline)) {
#pragma unroll
        for (int si = 0; si < 4; ++si)
#pragma unroll
            for (int h = 0; h < GPT; ++h)
                d[si][h] = Dq<ACT>::make((uint16_t)(w.s[si][h] >> sshift),
                                         SYM ? 8u : ((w.z[si][h] >> zshift) & 0xFu));
    };
    auto read_b = [&](auto buf, int s, u32x4_t(&b)[8]) __attribute__((always_inline)) {
        const int c = (s * 4 + (lane >> 4)) ^ bsw;
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) b[mb] = xs[decltype(buf)::value][mb * 128 + brow + c];
    };
    auto dequant_a = [&](const WSet &w, const DqT(&d)[4][GPT], int word, u32x4_t(&a)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int si = 0; si < 4; ++si) a[si] = Dq<ACT>::word(w.w[si][word], d[si][(word * 32) / G]);
    };
    // One 32-deep step: MFMA i (row block i/4, strip i%4) runs on the current operands,
    // followed by slice i of the next step's preparation -- an LDS read of the next
    // activation operand every fourth MFMA and piece i%8 of the next weight word of strip
    // i/8 -- so the matrix, vector and LDS pipes stay busy together.
    auto step = [&](const u32x4_t(&a)[4], const u32x4_t(&b)[8], u32x4_t(&an)[4],
                    u32x4_t(&bn)[8], const WSet &wn, const DqT(&dn)[4][GPT], int word_n,
                    auto bufn, int s_n) __attribute__((always_inline)) {
        const int c = (s_n * 4 + (lane >> 4)) ^ bsw;
        PieceTmp tmp;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int mb = i >> 2, si = i & 3;
            mfma_acc<ACT>(acc[si][mb], a[si], b[mb]);
            if ((i & 3) == 0) bn[i >> 2] = xs[decltype(bufn)::value][(i >> 2) * 128 + brow + c];
            const int ws_i = i >> 3;
            dq_piece<ACT>(i & 7, wn.w[ws_i][word_n], dn[ws_i][(word_n * 32) / G], tmp, an[ws_i]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // One 64-deep stage st (ring buffer BUF = st % NST, tile t = st / 2, half H = st % 2,
    // TW = t % NWS: the weight set of tile t; dequant constants alternate by t % 2).  Step 0
    // runs word 2H while step 1's operands are prepared; step 1 runs word 2H+1 while the
    // next stage's first operands are prepared.
    auto stage = [&](int st, auto BUF, auto H, auto TW) __attribute__((always_inline)) {
        constexpr int buf = decltype(BUF)::value, h = decltype(H)::value;
        constexpr int tw = decltype(TW)::value, td = tw % 2;
        constexpr int nbuf = (buf + 1) % NST, nw = (tw + 1) % NWS, nd = 1 - td;
        const int t = st >> 1;
        wait_vm_barrier<kWait>();
        dma(st + NST - 1, IC<(buf + NST - 1) % NST>());
        if (h == 0) load_w(t + NWS - 1, ws[(tw + NWS - 1) % NWS]);
        // step 0: word 2h of tile t; prepares word 2h+1 from this stage's buffer
        step_fence();
        step(A[0], B[0], A[1], B[1], ws[tw], dq[td], 2 * h + 1, BUF, 1);
        // step 1: word 2h+1; prepares stage st+1's first step (next tile when h == 1)
        step_fence();
        if (h == 1) {
            make_dq(ws[nw], dq[nd]);
            step(A[1], B[1], A[0], B[0], ws[nw], dq[nd], 0, IC<nbuf>(), 0);
        } else {
            step(A[1], B[1], A[0], B[0], ws[tw], dq[td], 2, IC<nbuf>(), 0);
        }
    };
    // Stages u .. u+3 of an NST-stage block (u = 0 or 4).
    auto four = [&](int st, auto U) __attribute__((always_inline)) {
        constexpr int u = decltype(U)::value;
        stage(st + 0, IC<u + 0>(), IC<0>(), IC<(u / 2) % NWS>());
        stage(st + 1, IC<u + 1>(), IC<1>(), IC<(u / 2) % NWS>());
        stage(st + 2, IC<u + 2>(), IC<0>(), IC<(u / 2 + 1) % NWS>());
        stage(st + 3, IC<u + 3>(), IC<1>(), IC<(u / 2 + 1) % NWS>());
    };

    // The zeroed accumulators are written by VALU; pad before the first MFMA reads them.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 4" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    // Prologue, in the loop's issue order: the DMAs of stages 0 .. NST-2, with the weights
    // of tiles 0 .. NWS-2 after the DMAs of stages 1, 3, ...; then stage 0's first operands.
    dma(0, IC<0>());
    dma(1, IC<1>());
    load_w(0, ws[0]);
    dma(2, IC<2>());
    if constexpr (NST == 8) {
        dma(3, IC<3>());
        load_w(1, ws[1]);
        dma(4, IC<4>());
        dma(5, IC<5>());
        load_w(2, ws[2]);
        dma(6, IC<6>());
    }
    wait_vm_barrier<kProWait>();
    make_dq(ws[0], dq[0]);
    read_b(IC<0>(), 0, B[0]);
    dequant_a(ws[0], dq[0], 0, A[0]);

    // S is a multiple of 4; NST-stage blocks, then a four-stage tail when S % 8 == 4 (the
    // tail's stages are a block's first four, so its buffers and weight sets line up).
    // Each pass ends with mfma_drain, so whatever the compiler places after the loop (it
    // may copy accumulators between registers right at the loop exit) finds the inline-asm
    // MFMAs' results written.
    int st = 0;
    for (; st + NST <= S; st += NST) {
        four(st, IC<0>());
        if constexpr (NST == 8) four(st + 4, IC<4>());
        mfma_drain();
    }
    if constexpr (NST == 8) {
        if (st < S) {
            four(st, IC<0>());
            mfma_drain();
        }
    }
    // The last stages prefetched (redundant) LDS data; let every DMA land before the wave
    // can retire, so no write reaches LDS after the workgroup has released it.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

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
    const dim3 grid((a.Np + kRBN - 1) / kRBN, (a.M + kRBM - 1) / kRBM);
    prefill_ring_kernel<ACT, SYM, G, kRStages, kRWSets><<<grid, dim3(kRThreads), 0, stream>>>(
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

}  // namespace

hipError_t launch_prefill_ring(const GemmArgs &a, hipStream_t stream) {
    if (a.act == kBF16) {
        launch_act<kBF16>(a, stream);
    } else {
        launch_act<kF16>(a, stream);
    }
    return hipGetLastError();
}

}  // namespace mpgemm
