// Decode attention over an 8-bit or FP8 KV cache for gfx950, and the KV-cache packer.
//
// [TurboMind, attention pipeline; Fig. 4 and Fig. 10 captions]: the low-bit KV cache is
// dequantized to 16-bit values by I2F conversion and scaling, V is kept in a transposed
// (column-major) tile layout for the matrix cores, and KV is streamed in 64-token
// macro-tiles.  Source: "LMDeploy Accelerates Mixed-Precision LLM Inference with
// TurboMind" (arXiv 2508.15601).
//
// Cache layout (include/mpgemm.h): 64-token blocks holding every KV head; head h of a block
// is HB = 128 D + 384 bytes: K codes as the 8-bit weight packing of K^T (k = d, n = token),
// V codes as that of V (k = token, n = d), then K and V scales (fp16) and zeros (uint8).
//
// Design for MI355X (one 64-lane wave per (sequence, KV head, split of the blocks)):
//   - S = K Q^T on 16x16x32 MFMAs: A = dequantized K (rows = 16 tokens of a strip, k = d;
//     each lane's 16-byte load of a K tile is exactly two MFMA A operands, as for weights),
//     B = the G <= 16 query heads of the KV head (columns), loaded once;
//   - online softmax in the exp2 domain.  Every score and every output a lane holds
//     belongs to head lane % 16, so rescaling is lane-local; block maxima and sums need
//     two cross-lane exchanges;
//   - FP8 codes (E4M3 / E5M2, no zero points): K by the FP8 weight dequantizer, V's codes
//     converted exactly to the activation format, no zero correction;
//   - O += V^T P' on MFMAs: A = V codes (rows = 16 values of d, k = tokens -- the
//     transposed layout), B = P' (columns = heads, k = tokens) through 2 KiB of LDS.  V's
//     per-token scale is folded into P' = round(p * s_v), and its zero point into one
//     correction per head, sum_t P'_t z_t, subtracted at the end -- so V's codes enter the
//     MFMA as exact integers (a byte permute and one exact packed add);
//   - block j + 1's loads are issued before block j is computed (two register sets; one for
//     D = 256, whose two sets would not fit);
//   - splits of the block range write unnormalized partials (O, max, sum) to a workspace,
//     split-contiguous per output element; a second kernel combines them with independent
//     16-byte loads.  One split writes the output directly;
//   - a block-table entry outside the cache is skipped (no access); every load goes
//     through a buffer descriptor bounded to its block.
#include "kernels.hpp"

namespace mpgemm {

namespace {

constexpr int kKvTokens = 64;                  // tokens per cache block

__device__ __forceinline__ float xor_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 16, 64));
    return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float xor_sum(float v) {
    v += __shfl_xor(v, 16, 64);
    return v + __shfl_xor(v, 32, 64);
}

template <int ACT>
__device__ __forceinline__ uint16_t round_act(float x) {
    if constexpr (ACT == kF16) return bitcast<uint16_t>((_Float16)x);
    else return (uint16_t)pack_bf16x2(x, 0.f);
}
template <int ACT>
__device__ __forceinline__ float act_to_f32(uint16_t h) {
    if constexpr (ACT == kF16) return (float)bitcast<_Float16>(h);
    else return __uint_as_float((uint32_t)h << 16);
}

// Eight V codes (two words, k ascending) as exact 16-bit values in MFMA operand order:
// 8-bit integers, or FP8 values (every E4M3 / E5M2 value is an fp16 and a bf16 value).
template <int ACT, int KVC>
__device__ __forceinline__ u32x4_t v_codes_exact(uint32_t w0, uint32_t w1) {
    u32x4_t r;
    if constexpr (kCodeFp8<KVC> && ACT == kF16) {
        r[0] = fp8_pair_f16<KVC, false>(w0);
        r[1] = fp8_pair_f16<KVC, true>(w0);
        r[2] = fp8_pair_f16<KVC, false>(w1);
        r[3] = fp8_pair_f16<KVC, true>(w1);
    } else if constexpr (kCodeFp8<KVC>) {
        const f32x2_t a = fp8_pair_f32<KVC, false>(w0), b = fp8_pair_f32<KVC, true>(w0);
        const f32x2_t c = fp8_pair_f32<KVC, false>(w1), d = fp8_pair_f32<KVC, true>(w1);
        r[0] = pack_bf16x2(a.x, a.y);
        r[1] = pack_bf16x2(b.x, b.y);
        r[2] = pack_bf16x2(c.x, c.y);
        r[3] = pack_bf16x2(d.x, d.y);
    } else if constexpr (ACT == kF16) {
        // (1024 + v) pairs by a byte permute against 0x64, then - 1024 exactly
        const half2_t m1024 = bitcast<half2_t>(0xE400E400u);
        r[0] = bitcast<uint32_t>(bitcast<half2_t>(__builtin_amdgcn_perm(0x64646464u, w0, 0x04010400u)) + m1024);
        r[1] = bitcast<uint32_t>(bitcast<half2_t>(__builtin_amdgcn_perm(0x64646464u, w0, 0x04030402u)) + m1024);
        r[2] = bitcast<uint32_t>(bitcast<half2_t>(__builtin_amdgcn_perm(0x64646464u, w1, 0x04010400u)) + m1024);
        r[3] = bitcast<uint32_t>(bitcast<half2_t>(__builtin_amdgcn_perm(0x64646464u, w1, 0x04030402u)) + m1024);
    } else {
        r[0] = pack_bf16x2(ubyte(w0, 0), ubyte(w0, 1));
        r[1] = pack_bf16x2(ubyte(w0, 2), ubyte(w0, 3));
        r[2] = pack_bf16x2(ubyte(w1, 0), ubyte(w1, 1));
        r[3] = pack_bf16x2(ubyte(w1, 2), ubyte(w1, 3));
    }
    return r;
}

// KVC: format of the KV codes (kU8 with zero points, or kE4M3 / kE5M2 without).
template <int ACT, int D, int KVC>
__global__ __launch_bounds__(64) void attn_decode_kv8_kernel(
    const uint16_t *__restrict__ Q, const uint8_t *__restrict__ cache, int num_blocks,
    const int *__restrict__ table, int table_stride, const int *__restrict__ lens, int Hq,
    int Hkv, int bps, int splits, float scale_log2, uint16_t *__restrict__ O,
    float *__restrict__ part, int Du) {
    // D: the stored head size (a multiple of 64); Du <= D: the caller's head size (a
    // multiple of 16), the row length of Q and O.  Query elements past Du load as zeros,
    // so the zero codes stored past Du add nothing to a score, and outputs past Du are
    // not stored.
    constexpr int DS = D / 32;                 // 32-deep k steps of Q K^T
    constexpr int KT = D / 64;                 // 64-deep K tiles per 16-token strip
    constexpr int VS = D / 16;                 // 16-row strips of V^T
    constexpr uint32_t HB = 128u * D + 384u;   // bytes of one KV head in a block
    __shared__ u32x4_t pl4[16 * kKvTokens / 8];   // P'[head][token], 16-bit values
    u32x2_t *const pl = reinterpret_cast<u32x2_t *>(pl4);

    const int lane = threadIdx.x;
    const int split = blockIdx.x % splits;
    const int bh = blockIdx.x / splits;
    const int hk = bh % Hkv, b = bh / Hkv;
    const int G = Hq / Hkv;
    const int g = lane & 15;                   // this lane's head column
    const int q4 = lane >> 4;
    const int len = min(lens[b], table_stride * kKvTokens);
    const int nblk = (len + kKvTokens - 1) / kKvTokens;
    const int j0 = split * bps, j1 = min(nblk, j0 + bps);

    // B operand of Q K^T: head g, k = 32 s + 8 (lane / 16) .. +7 (heads past G: zeros).
    u32x4_t qb[DS];
    {
        const uint16_t *qrow = Q + ((size_t)b * Hq + hk * G + min(g, G - 1)) * Du;
#pragma unroll
        for (int s = 0; s < DS; ++s)
            qb[s] = g < G && 32 * s + 8 * q4 < Du
                        ? *reinterpret_cast<const u32x4_t *>(qrow + 32 * s + 8 * q4)
                        : u32x4_t{0u, 0u, 0u, 0u};
    }

    f32x4_t oacc[VS];
#pragma unroll
    for (int i = 0; i < VS; ++i) oacc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f, c = 0.f;

    // One block's loads: K tiles and the lane's token scale/zero, V tiles and the V scales /
    // zeros of the lane's score tokens.  Two sets alternate, so block j + 1 loads while
    // block j computes.
    struct Blk {
        u32x4_t kw[4][KT];
        uint32_t ksw[4], kzw[4];
        u32x4_t vw[VS];
        u32x2_t vsw[4];
        uint32_t vzw[4];
        bool ok;
    };
    auto load_blk = [&](int j, Blk &bl) __attribute__((always_inline)) {
        const int pb = table[(size_t)b * table_stride + j];
        bl.ok = pb >= 0 && pb < num_blocks;
        if (!bl.ok) return;
        const uint8_t *hbase = cache + (size_t)pb * HB * Hkv + (size_t)hk * HB;
        const rsrc_t rs = make_rsrc(hbase, HB);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
                bl.kw[s][kt] = buf_load_b128(rs, lane * 16u, (s * KT + kt) * 1024u);
            const uint32_t tok = 16 * s + g;
            bl.ksw[s] = buf_load_b32(rs, 128u * D + (tok & ~1u) * 2u, 0);
            bl.kzw[s] = buf_load_b32(rs, 128u * D + 256u + (tok & ~3u), 0);
        }
#pragma unroll
        for (int sd = 0; sd < VS; ++sd) bl.vw[sd] = buf_load_b128(rs, lane * 16u, 64u * D + sd * 1024u);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t tok = 16 * s + 4 * q4;
            bl.vsw[s] = buf_load_b64(rs, 128u * D + 128u + tok * 2u, 0);
            bl.vzw[s] = buf_load_b32(rs, 128u * D + 320u + tok, 0);
        }
    };
    auto compute_blk = [&](int j, const Blk &bl) __attribute__((always_inline)) {
        if (!bl.ok) return;
        // S = K Q^T, strip by strip; lane holds tokens 16 s + 4 (lane / 16) + r of head g.
        f32x4_t sacc[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t tok = 16 * s + g;
            const uint16_t ks = (uint16_t)(bl.ksw[s] >> ((tok & 1) * 16));
            const uint32_t kz = (bl.kzw[s] >> ((tok & 3) * 8)) & 0xFFu;
            typedef DqFor<ACT, KVC> DqK;
            const typename DqK::type dq = DqK::make(ks, kz);
            sacc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kt = 0; kt < KT; ++kt)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    sacc[s] = mfma16x16x32<ACT>(DqK::pair(bl.kw[s][kt][2 * h], bl.kw[s][kt][2 * h + 1], dq),
                                                qb[2 * kt + h], sacc[s]);
        }
        // Online softmax (log2 domain) with masking of tokens past len.
        float sc[4][4];
        float bmax = -INFINITY;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = j * kKvTokens + 16 * s + 4 * q4 + r;
                sc[s][r] = t < len ? sacc[s][r] * scale_log2 : -INFINITY;
                bmax = fmaxf(bmax, sc[s][r]);
            }
        bmax = xor_max(bmax);
        const float mn = fmaxf(m, bmax);
        if (mn == -INFINITY) return;           // nothing unmasked yet (uniform)
        const float alpha = exp2f(m - mn);
        m = mn;
        c *= alpha;
        float psum = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint16_t pr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = exp2f(sc[s][r] - mn);
                psum += p;
                const float vscale = (float)bitcast<_Float16>((uint16_t)(bl.vsw[s][r >> 1] >> ((r & 1) * 16)));
                pr[r] = round_act<ACT>(p * vscale);
                if constexpr (!kCodeFp8<KVC>)
                    c += act_to_f32<ACT>(pr[r]) * (float)((bl.vzw[s] >> (8 * r)) & 0xFFu);
            }
            pl[(g * kKvTokens + 16 * s + 4 * q4) / 4] =
                u32x2_t{(uint32_t)pr[0] | ((uint32_t)pr[1] << 16), (uint32_t)pr[2] | ((uint32_t)pr[3] << 16)};
        }
        l = l * alpha + xor_sum(psum);
#pragma unroll
        for (int sd = 0; sd < VS; ++sd) oacc[sd] *= alpha;
        __syncthreads();
        // O += V^T P': k = tokens 32 u + 8 (lane / 16) .. +7 of head g.
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const u32x4_t pbv = pl4[(g * kKvTokens + 32 * u + 8 * q4) / 8];
#pragma unroll
            for (int sd = 0; sd < VS; ++sd)
                oacc[sd] = mfma16x16x32<ACT>(v_codes_exact<ACT, KVC>(bl.vw[sd][2 * u], bl.vw[sd][2 * u + 1]),
                                             pbv, oacc[sd]);
        }
        __syncthreads();
    };

    if constexpr (D <= 128) {
        Blk ba, bb;
        if (j0 < j1) load_blk(j0, ba);
        for (int j = j0; j < j1; j += 2) {
            if (j + 1 < j1) load_blk(j + 1, bb);
            compute_blk(j, ba);
            if (j + 1 >= j1) break;
            if (j + 2 < j1) load_blk(j + 2, ba);
            compute_blk(j + 1, bb);
        }
    } else {                                   // D = 192, 256: one set (two would spill)
        Blk ba;
        for (int j = j0; j < j1; ++j) {
            load_blk(j, ba);
            compute_blk(j, ba);
        }
    }
    c = xor_sum(c);

    // Output rows d = 16 sd + 4 (lane / 16) + r of head g.
    const int h = hk * G + g;
    if (splits == 1) {
        if (g >= G) return;
        const float inv = l > 0.f ? 1.f / l : 0.f;
        uint16_t *orow = O + ((size_t)b * Hq + h) * Du;
#pragma unroll
        for (int sd = 0; sd < VS; ++sd) {
            const f32x4_t v = (oacc[sd] - c) * inv;
            if (16 * sd + 4 * q4 < Du)
                *reinterpret_cast<u32x2_t *>(orow + 16 * sd + 4 * q4) = round4<ACT>(v);
        }
        return;
    }
    if (g >= G) return;
    // Partials, split-contiguous per output element: O at part[(bh D + d) SP + split],
    // then (max, sum) pairs at part[B Hq D SP + 2 (bh SP + split)] (SP: splits padded to 4).
    const int SP = (splits + 3) & ~3;
    const size_t bhq = (size_t)b * Hq + h;
    const size_t nbh = (size_t)(gridDim.x / splits) / Hkv * Hq;     // B * Hq
#pragma unroll
    for (int sd = 0; sd < VS; ++sd)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            part[(bhq * D + 16 * sd + 4 * q4 + r) * SP + split] = oacc[sd][r] - c;
    if (q4 == 0) {
        float *ml = part + nbh * D * SP + 2 * (bhq * SP + split);
        ml[0] = m;
        ml[1] = l;
    }
}

// out[b][h][d] = sum_i w_i O_i[d] / sum_i w_i l_i, w_i = 2^(m_i - max m); one thread per d.
// (splits <= kMaxSplits)
constexpr int kMaxSplits = 1024;
template <int ACT, int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(const float *__restrict__ part, int splits,
                                                         int nbh, uint16_t *__restrict__ O, int Du) {
    __shared__ float w[kMaxSplits];
    __shared__ float red[D / 64][2];
    const int bh = blockIdx.x, d = threadIdx.x;
    const int SP = (splits + 3) & ~3;
    const float *ml = part + (size_t)nbh * D * SP + 2 * (size_t)bh * SP;
    const f32x4_t *row = reinterpret_cast<const f32x4_t *>(part + ((size_t)bh * D + d) * SP);
    // The first 64 splits of this thread's row are requested first, so that their latency
    // overlaps the max and weight phases (a batch at a time afterwards).
    constexpr int kPre = 16, kBatch = 8;
    f32x4_t pre[kPre];
#pragma unroll
    for (int u = 0; u < kPre; ++u) pre[u] = u < SP / 4 ? row[u] : f32x4_t{0.f, 0.f, 0.f, 0.f};
    // This thread's first (max, sum) pair stays in registers for the weight phase.
    float mi = -INFINITY, li = 0.f;
    if (d < splits) {
        const f32x2_t p = *reinterpret_cast<const f32x2_t *>(ml + 2 * d);
        mi = p.x;
        li = p.y;
    }
    float mx = mi;
    for (int i = d + D; i < splits; i += D) mx = fmaxf(mx, ml[2 * i]);
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if ((d & 63) == 0) red[d >> 6][0] = mx;
    __syncthreads();
    mx = red[0][0];
#pragma unroll
    for (int k = 1; k < D / 64; ++k) mx = fmaxf(mx, red[k][0]);
    float ls = 0.f;
    if (d < splits) {
        const float wi = mx == -INFINITY ? 0.f : exp2f(mi - mx);
        w[d] = wi;
        ls = wi * li;
    }
    for (int i = d + D; i < splits; i += D) {
        const float wi = mx == -INFINITY ? 0.f : exp2f(ml[2 * i] - mx);
        w[i] = wi;
        ls += wi * ml[2 * i + 1];
    }
    for (int o = 32; o >= 1; o >>= 1) ls += __shfl_xor(ls, o, 64);
    if ((d & 63) == 0) red[d >> 6][1] = ls;
    __syncthreads();
    ls = 0.f;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) ls += red[k][1];
    float acc = 0.f;
    auto add = [&](int c, const f32x4_t &v) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 4 * c + e;
            if (i < splits && w[i] != 0.f) acc += w[i] * v[e];
        }
    };
#pragma unroll
    for (int u = 0; u < kPre; ++u) add(u, pre[u]);
    // Eight independent 16-byte loads in flight per batch (the loop would otherwise wait
    // out one memory latency per load).
    for (int i0 = kPre; i0 < SP / 4; i0 += kBatch) {
        f32x4_t v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            v[u] = i0 + u < SP / 4 ? row[i0 + u] : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < kBatch; ++u) add(i0 + u, v[u]);
    }
    if (d < Du) O[(size_t)bh * Du + d] = round_act<ACT>(ls > 0.f ? acc / ls : 0.f);
}

// One thread per (token, KV head): writes its K and V codes (zeros past the caller's head
// size D, up to the stored size Dp), scales and zeros.
__global__ void kv_pack_kernel(const uint8_t *__restrict__ kc, const uint16_t *__restrict__ ks,
                               const uint8_t *__restrict__ kz, const uint8_t *__restrict__ vc,
                               const uint16_t *__restrict__ vs, const uint8_t *__restrict__ vz,
                               int n, int t0, int Hkv, int D, int Dp, const int *__restrict__ table_row,
                               int table_len, int num_blocks, uint8_t *__restrict__ cache) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n * Hkv) return;
    const int tl = i / Hkv, h = i % Hkv;
    const int t = t0 + tl, slot = t % kKvTokens, jb = t / kKvTokens;
    if (jb >= table_len) return;
    const int pb = table_row[jb];
    if (pb < 0 || pb >= num_blocks) return;
    const size_t HB = 128 * (size_t)Dp + 384;
    uint8_t *hb = cache + (size_t)pb * HB * Hkv + (size_t)h * HB;
    const size_t row = (size_t)tl * Hkv + h;
    for (int d = 0; d < Dp; ++d) {
        // K^T: k = d, n = slot (16 x 64 tiles, K = Dp rows); V: k = slot, n = d (K = 64).
        const int kk = d % 64, vk = slot % 64;
        const size_t koff = ((size_t)(slot / 16) * (Dp / 64) + d / 64) * 1024 +
                            (size_t)(slot % 16 + 16 * ((kk % 32) / 8)) * 16 + (kk / 32) * 8 + kk % 8;
        const size_t voff = (size_t)(d / 16) * 1024 + (size_t)(d % 16 + 16 * ((vk % 32) / 8)) * 16 +
                            (vk / 32) * 8 + vk % 8;
        hb[koff] = d < D ? kc[row * D + d] : (uint8_t)0;
        hb[64 * (size_t)Dp + voff] = d < D ? vc[row * D + d] : (uint8_t)0;
    }
    uint16_t *sc = reinterpret_cast<uint16_t *>(hb + 128 * (size_t)Dp);
    sc[slot] = ks[row];
    sc[kKvTokens + slot] = vs[row];
    hb[128 * (size_t)Dp + 256 + slot] = kz ? kz[row] : (uint8_t)0;
    hb[128 * (size_t)Dp + 320 + slot] = vz ? vz[row] : (uint8_t)0;
}

template <int ACT, int D, int KVC>
void launch_attn(const AttnArgs &a, hipStream_t stream) {
    const dim3 grid((unsigned)(a.B * a.Hkv * a.splits));
    attn_decode_kv8_kernel<ACT, D, KVC><<<grid, dim3(64), 0, stream>>>(
        a.Q, a.cache, a.num_blocks, a.table, a.table_stride, a.lens, a.Hq, a.Hkv, a.bps,
        a.splits, a.scale_log2, a.O, a.part, a.D);
    if (a.splits > 1)
        attn_combine_kernel<ACT, D><<<dim3((unsigned)(a.B * a.Hq)), dim3(D), 0, stream>>>(
            a.part, a.splits, a.B * a.Hq, a.O, a.D);
}

template <int ACT, int KVC>
void launch_attn_kvc(const AttnArgs &a, hipStream_t stream) {
    switch (kv_padded_d(a.D)) {
        case 64: launch_attn<ACT, 64, KVC>(a, stream); break;
        case 192: launch_attn<ACT, 192, KVC>(a, stream); break;
        case 256: launch_attn<ACT, 256, KVC>(a, stream); break;
        default: launch_attn<ACT, 128, KVC>(a, stream); break;
    }
}

template <int ACT>
void launch_attn_act(const AttnArgs &a, hipStream_t stream) {
    switch (a.kv_code) {
        case kE4M3: launch_attn_kvc<ACT, kE4M3>(a, stream); break;
        case kE5M2: launch_attn_kvc<ACT, kE5M2>(a, stream); break;
        default: launch_attn_kvc<ACT, kU8>(a, stream); break;
    }
}

}  // namespace

size_t attn_part_bytes(int B, int Hq, int D, int splits) {
    const size_t sp = (size_t)((splits + 3) & ~3);
    return splits > 1 ? (size_t)B * Hq * sp * (kv_padded_d(D) + 2) * sizeof(float) : 0;
}

hipError_t launch_attention_kv8(const AttnArgs &a, hipStream_t stream) {
    a.act == kBF16 ? launch_attn_act<kBF16>(a, stream) : launch_attn_act<kF16>(a, stream);
    return hipGetLastError();
}

hipError_t launch_kv_pack(const uint8_t *kc, const uint16_t *ks, const uint8_t *kz,
                          const uint8_t *vc, const uint16_t *vs, const uint8_t *vz, int n, int t0,
                          int Hkv, int D, const int *table_row, int table_len, int num_blocks,
                          void *cache, hipStream_t stream) {
    const int threads = 128;
    const int items = n * Hkv;
    if (items > 0)
        kv_pack_kernel<<<(items + threads - 1) / threads, threads, 0, stream>>>(
            kc, ks, kz, vc, vs, vz, n, t0, Hkv, D, kv_padded_d(D), table_row, table_len,
            num_blocks, (uint8_t *)cache);
    return hipGetLastError();
}

}  // namespace mpgemm
