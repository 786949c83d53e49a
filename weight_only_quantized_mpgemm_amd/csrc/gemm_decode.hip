// Small-M (decode) W4A16 / W8A16 GEMM for gfx950.
//
// [TurboMind, GEMM pipeline; Fig. 6 and Fig. 9 captions]: the packed 4-bit weights are
// loaded straight into registers, turned into 16-bit values by I2F conversion and scaling,
// and fed to the matrix cores while later tiles' loads are in flight.  Source: "LMDeploy
// Accelerates Mixed-Precision LLM Inference with TurboMind" (arXiv 2508.15601).
//
// At M <= 64 the GEMM is bound by HBM bandwidth: every weight byte is read once and used
// for at most M multiply-adds.  Design for MI355X:
//   - a workgroup owns S adjacent 16-column strips; its NW waves split the K range into
//     contiguous slices (split-K inside the workgroup).  The host picks S and NW by shape
//     (pick_split below);
//   - each wave runs a D-slot register pipeline over its K slice: slot s holds, for one
//     128-deep tile step, the S weight tiles (one 128-bit load per lane and strip; a wave
//     reads 1 KiB contiguously per strip), the activation fragments of that step (shared by
//     the S strips) and the raw scales/zeros; computing slot s is followed by refilling it
//     with the step D positions later, so D steps are always in flight.  The loop body has
//     no branches; refills past the slice are clamped onto its last step (cache hits) and a
//     short tail computes the remaining slots;
//   - all loads are buffer loads: fixed per-lane offsets, a wave-uniform scalar offset per
//     step.  Activation rows past M fall outside the activation descriptor and read as
//     zero without any memory traffic, so M = 1 moves 1/16 of a full row block;
//   - weights are the MFMA A operand (rows = n), activations the B operand (columns = m);
//   - the NW partial sums meet in LDS and are added in a fixed wave order;
//   - optionally the K range is also split over P workgroups (grid.y).  Every workgroup of
//     a strip group writes its fp32 partial to the workspace, then bumps the group's
//     counter; the workgroup that arrives last adds the P partials in split order, stores
//     Y and sets the counter back to zero.  Nobody waits for anybody, the sum order is
//     fixed (results are deterministic for a given split), and the counters are left as
//     they were found, so the workspace needs zeroing only once.  P > 1 balances the work
//     over the CUs and lets several strips share one activation fragment (S) without
//     leaving CUs idle at small N.
#include <stdio.h>
#include <stdlib.h>

#include <type_traits>

#include "kernels.hpp"

namespace mpgemm {

namespace {

constexpr int kMaxWaves = 8;

template <int MB, int S, int GPT, int WV>
struct Slot {
    u32x4_t w[S][WV];          // per strip: WV 16-byte pieces of packed tile = 4 MFMA k-steps
    u32x4_t x[4][MB];          // activation B operands per k-step and row block
    uint32_t s[S][GPT];        // dword holding the lane's fp16 scale, per strip and group
    uint32_t z[S][GPT];        // dword holding the lane's 4-bit zero, per strip and group
};

template <int ACT, int MB, int S, bool SYM, int G, int D, int CODE>
__global__ __launch_bounds__(kMaxWaves * 64) void decode_kernel(
    const uint16_t *__restrict__ X, const uint32_t *__restrict__ codes,
    const uint16_t *__restrict__ scales, const uint8_t *__restrict__ zeros, int M, int N, int K,
    int Kx, int Ny, uint16_t *__restrict__ Y, f32x4_t *__restrict__ part,
    uint32_t *__restrict__ cnt) {
    // N, K: the padded matrix of the packed planes; Kx: activation row length (the user K,
    // <= K); Ny: output row length (the user N, <= N).  Activations at k >= Kx read as zero.
    constexpr int GPT = kTileK / G;              // groups per 128-k tile (1 or 2)
    // 128-bit pieces per lane and strip per 128-deep step: one 16 x 128 tile of 4-bit codes,
    // two 16 x 64 tiles of 8-bit codes; 2- and 3-bit codes fill 8 or 12 bytes of one piece.
    constexpr int BITS = kCodeBits<CODE>;
    constexpr int WV = BITS >= 4 ? BITS / 4 : 1;
    constexpr uint32_t kTileBytes = 256u * BITS;       // one 16 x 128 tile of the strip
    constexpr uint32_t kLaneBytes = BITS >= 4 ? 16u : 4u * BITS;
    constexpr bool kNibbleZeros = BITS <= 4;           // zeros stored as 4-bit values
    typedef Slot<MB, S, GPT, WV> SlotT;
    extern __shared__ f32x4_t red[];             // [NW][S][MB][64]

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

    const rsrc_t wrs = make_rsrc(codes, (uint32_t)((size_t)strips * KT * kTileBytes));
    const rsrc_t xrs = make_rsrc(X, (uint32_t)((size_t)M * Kx * 2));
    const rsrc_t srs = make_rsrc(scales, (uint32_t)((size_t)groups * N * 2));
    const rsrc_t zrs = make_rsrc(zeros, (uint32_t)((size_t)groups * N / (kNibbleZeros ? 2 : 1)));

    // Per-lane byte offsets, fixed for the whole K slice.  Strips past N read the last real
    // strip (their outputs are never stored).  The meta element of a lane's column is a
    // multiple of 16 plus lane % 16, so its scale is half (lane & 1) of a dword and its zero
    // is nibble (lane & 7) of a dword (4-bit codes) or byte (lane & 3) (8-bit codes).
    uint32_t woff[S], soff[S], zoff[S];
#pragma unroll
    for (int si = 0; si < S; ++si) {
        const uint32_t strip = (uint32_t)min(strip0 + si, strips - 1);
        woff[si] = (strip * KT + t_begin) * kTileBytes + lane * kLaneBytes;
        const uint32_t e = strip * groups * 16u + t_begin * GPT * 16u + (lane & 15);
        soff[si] = (e >> 1) * 4u;
        zoff[si] = kNibbleZeros ? (e >> 3) * 4u : (e >> 2) * 4u;
    }
    uint32_t xoff[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        xoff[mb] = ((uint32_t)(mb * 16 + (lane & 15)) * Kx + t_begin * kTileK + (lane >> 4) * 8) * 2u;
    // Ragged K: the lane's 8-element chunk of 32-deep step j of tile t_begin + i starts at
    // k = k_lane + 128 i + 32 j; chunks at or past Kx take an offset outside the activation
    // descriptor, which reads as zero.  Only tiles that reach past Kx take this path.
    const int k_lane = t_begin * kTileK + (lane >> 4) * 8;
    const bool ragged = Kx != K;
    const uint32_t sshift = (lane & 1) * 16;
    const uint32_t zshift = kNibbleZeros ? (lane & 7) * 4 : (lane & 3) * 8;
    constexpr uint32_t zmask = (1u << BITS) - 1;
    constexpr uint32_t zsym = 1u << (BITS - 1);        // symmetric zero: 2, 4, 8 or 128
    constexpr int zrow = kNibbleZeros ? 8 : 16;        // zero bytes per (strip, group)

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
        if (ragged && (t_begin + i + 1) * kTileK > Kx) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool in = k_lane + i * kTileK + 32 * j < Kx;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    sl.x[j][mb] = buf_load_b128(xrs, in ? xoff[mb] : 0x80000000u,
                                                (i * kTileK + 32 * j) * 2);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    sl.x[j][mb] = buf_load_b128(xrs, xoff[mb], (i * kTileK + 32 * j) * 2);
        }
#pragma unroll
        for (int si = 0; si < S; ++si)
#pragma unroll
            for (int h = 0; h < GPT; ++h) {
                sl.s[si][h] = buf_load_b32(srs, soff[si], (i * GPT + h) * 32);
                sl.z[si][h] = SYM ? 0u : buf_load_b32(zrs, zoff[si], (i * GPT + h) * zrow);
            }
    };

    f32x4_t acc[S][MB];
#pragma unroll
    for (int si = 0; si < S; ++si)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[si][mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const SlotT &sl) {
        typedef DqFor<ACT, CODE> DqB;
        typename DqB::type dq[S][GPT];
#pragma unroll
        for (int si = 0; si < S; ++si)
#pragma unroll
            for (int h = 0; h < GPT; ++h)
                dq[si][h] = DqB::make((uint16_t)(sl.s[si][h] >> sshift),
                                      SYM ? zsym : ((sl.z[si][h] >> zshift) & zmask));
        if constexpr (BITS < 4) {
            // Sub-4-bit codes: the four steps' operands of each strip at once.
            u32x4_t at[S][4];
#pragma unroll
            for (int si = 0; si < S; ++si) {
                const typename DqB::type *d[4] = {&dq[si][0], &dq[si][32 / G], &dq[si][64 / G],
                                                  &dq[si][96 / G]};
                DqB::tile(sl.w[si][0], d, at[si]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int si = 0; si < S; ++si)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[si][mb] = mfma16x16x32<ACT>(at[si][j], sl.x[j][mb], acc[si][mb]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int si = 0; si < S; ++si) {
                    u32x4_t a;
                    if constexpr (BITS == 4)
                        a = DqB::word(sl.w[si][0][j], dq[si][(j * 32) / G]);
                    else
                        a = DqB::pair(sl.w[si][j / 2][2 * (j % 2)],
                                      sl.w[si][j / 2][2 * (j % 2) + 1], dq[si][(j * 32) / G]);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[si][mb] = mfma16x16x32<ACT>(a, sl.x[j][mb], acc[si][mb]);
                }
        }
    };

    if (n > 0) {
        SlotT slot[D];
#pragma unroll
        for (int s = 0; s < D; ++s) {
            load(slot[s], min(s, n - 1));
            __builtin_amdgcn_sched_barrier(0);   // same load order as the loop's refills
        }
        const int n_main = n - n % D;
        for (int base = 0; base < n_main; base += D) {
#pragma unroll
            for (int s = 0; s < D; ++s) {
                // The barriers pin the order compute(s), refill(s), compute(s+1), ...: the
                // scheduler would otherwise sink every refill to the end of the batch and
                // the next batch would wait for all of them at once.
                compute(slot[s]);
                __builtin_amdgcn_sched_barrier(0);
                load(slot[s], min(base + D + s, n - 1));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        const int rest = n - n_main;
#pragma unroll
        for (int s = 0; s < D - 1; ++s)
            if (s < rest) compute(slot[s]);
    }

    const int col_lane = 4 * (lane >> 4);
    auto store_y = [&](int si, int mb, const f32x4_t &v) {
        const int m = mb * 16 + (lane & 15);
        const int n = (strip0 + si) * 16 + col_lane;
        if (m < M && n < Ny) store4<ACT>(Y + (size_t)m * Ny + n, Ny - n, v);
    };
    // Partial of block b (strip si = b / MB, row block mb = b % MB) of split q.
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
    // Split-K fixup: publish this partial, count it, and let the last arriver finish.  Every
    // wave fences its own partial stores (a fence only waits for the issuing wave's memory
    // operations) before the barrier; then one thread counts the workgroup in.
    // Each wave waits until its partial stores are acknowledged at device scope, the
    // workgroup meets, and one thread counts it in.  The last arriver's device-scope loads
    // are issued after it has seen every other workgroup's count, hence after their stores
    // completed.
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

// Strips per workgroup (S), waves per workgroup (NW) and workgroups per strip group along
// K (P).  S > 1 lets one activation fragment feed S strips (less L2 traffic per weight
// byte, which matters as M grows); NW and P split K inside and across workgroups.
// MPGEMM_DECODE_SPLIT="S,NW" or "S,NW,P" overrides the choice for tuning sweeps (S in
// {1,2,4} with one row block, {1,2} with two, 1 above; NW in 1..8; P in 1..16).
struct Split {
    int s, nw, p;
};
Split pick_split(int M, int strips, int KT, int mblocks) {
    Split sp{1, 1, 1};
    if (mblocks == 1) sp.s = strips >= 1024 ? 4 : (strips >= 256 && KT <= 64 ? 2 : 1);
    else if (mblocks == 2) sp.s = strips >= 512 ? 2 : 1;
    sp.nw = KT / 8;
    if (sp.nw < 1) sp.nw = 1;
    if (sp.nw > kMaxWaves) sp.nw = kMaxWaves;
    // Long K with fewer strips: the activation fragments, re-read by every strip group,
    // cost more than the weights (a 16-row fragment is 4x a weight tile's bytes).  Widen S
    // to its register limit and split K over P workgroups so that about 256 remain.
    // Measured on the 14336 x 4096 projection: 13 us instead of 19.5 at M = 16.
    // (At M <= 8 the fragments are mostly zero rows and S = 2 does as well.)
    if (KT > 64 && strips < 1024 && mblocks <= 2) {
        sp.s = mblocks == 1 && M > 8 ? 4 : 2;
        const int groups = (strips + sp.s - 1) / sp.s;
        sp.p = (256 + groups - 1) / groups;
        if (sp.p > 8) sp.p = 8;
        sp.nw = 4;                               // NW * P <= 32 < KT
    }
    if (const char *env = getenv("MPGEMM_DECODE_SPLIT")) {
        int s = 0, nw = 0, p = 1;
        const int got = sscanf(env, "%d,%d,%d", &s, &nw, &p);
        if (got >= 2 && (s == 1 || s == 2 || s == 4) && nw >= 1 && nw <= kMaxWaves &&
            p >= 1 && p <= 16 && nw * p <= KT && (s == 1 || mblocks <= 2) &&
            (s < 4 || mblocks == 1)) {
            sp.s = s;
            sp.nw = nw;
            sp.p = got == 3 ? p : 1;
        }
    }
    if ((strips + sp.s - 1) / sp.s > kMaxGroups) sp.p = 1;     // more groups than counters
    return sp;
}

size_t split_workspace(const Split &sp, int strips, int mblocks) {
    if (sp.p == 1) return 0;
    const size_t groups = (size_t)(strips + sp.s - 1) / sp.s;
    return kCounterBytes + groups * sp.p * sp.s * mblocks * 64 * sizeof(f32x4_t);
}

template <int ACT, int MB, int S, bool SYM, int G, int CODE>
void launch_s(const GemmArgs &a, const Split &sp, hipStream_t stream) {
    constexpr int slot_regs = S * kCodeBits<CODE> + 16 * MB + 2 * S;
    constexpr int D = slot_regs <= 24 ? 4 : (slot_regs <= 40 ? 3 : 2);
    const int strips = a.Np >> 4;
    const int wgs = (strips + S - 1) / S;
    const size_t lds = sp.nw > 1 ? (size_t)sp.nw * S * MB * 64 * sizeof(f32x4_t) : 0;
    uint32_t *cnt = nullptr;
    f32x4_t *part = nullptr;
    if (sp.p > 1) {
        cnt = static_cast<uint32_t *>(a.workspace);
        part = reinterpret_cast<f32x4_t *>(static_cast<char *>(a.workspace) + kCounterBytes);
    }
    decode_kernel<ACT, MB, S, SYM, G, D, CODE><<<dim3(wgs, sp.p), dim3(sp.nw * 64), lds, stream>>>(
        a.X, a.codes, a.scales, a.zeros, a.M, a.Np, a.Kp, a.K, a.N, a.Y, part, cnt);
}

template <int ACT, int MB, bool SYM, int G, int CODE>
void launch_one(const GemmArgs &a, hipStream_t stream) {
    const Split sp = pick_split(a.M, a.Np >> 4, a.Kp >> 7, MB);
    if constexpr (MB == 1) {
        if (sp.s == 4) return launch_s<ACT, MB, 4, SYM, G, CODE>(a, sp, stream);
    }
    if constexpr (MB <= 2) {
        if (sp.s == 2) return launch_s<ACT, MB, 2, SYM, G, CODE>(a, sp, stream);
    }
    launch_s<ACT, MB, 1, SYM, G, CODE>(a, sp, stream);
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

size_t decode_workspace_bytes(int M, int N, int K, int mblocks) {
    const int strips = padded_n(N) >> 4;
    return split_workspace(pick_split(M, strips, padded_k(K) >> 7, mblocks), strips, mblocks);
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
