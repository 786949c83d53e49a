// Offline weight packing and its inverse (layout v1 for 4-bit codes and its 8-bit
// counterpart, both specified in include/mpgemm.h).
//
// [TurboMind, technique (i); Fig. 6 and Fig. 7 captions]: packing is done once, offline, and
// is a pure permutation of bits; it places every 4-bit code where the online kernel's
// 128-bit loads and MFMA operand registers want it.  Source: "LMDeploy Accelerates
// Mixed-Precision LLM Inference with TurboMind" (arXiv 2508.15601).
#include "kernels.hpp"

namespace mpgemm {

namespace {

// Position of element i (= k % 8) inside its 32-bit word: e0 e2 e4 e6 e1 e3 e5 e7 from the
// least significant nibble up ([TurboMind], interleave diagram beside Fig. 24).
__device__ __forceinline__ int nibble_pos(int i) { return (i >> 1) + ((i & 1) << 2); }

// Word index (32-bit units) of the word holding rows k0..k0+7 (k0 % 8 == 0) of column n.
__device__ __forceinline__ size_t code_word_index(int k0, int n, int K) {
    const size_t tile = (size_t)(n >> 4) * (size_t)(K >> 7) + (size_t)(k0 >> 7);
    const int kk = k0 & 127;
    const int lane = (n & 15) + 16 * ((kk & 31) >> 3);
    return tile * kTileWords + (size_t)lane * 4 + (kk >> 5);
}

// Ragged shapes ([TurboMind, Fig. 24]: a data matrix padded up to the hardware tile): the
// planes hold the matrix padded to Kp x Np (Shape), in which every padded weight
// dequantizes to zero.  Padded columns (n >= N) hold code 0, scale 0 and zero 0; padded
// rows (k >= K) of real columns hold the element's zero point as their code (the group's
// zero; 0 in groups past the user's ceil(K/g); 8 or 128 for symmetric codes).
struct Shape {
    int K, N;        // user matrix (K % 8 == 0)
    int Kp, Np;      // padded matrix
    int g, rows;     // group size, user group rows ceil(K/g)
    uint32_t zmask;  // bits of a zero that are read (4-bit meta plane)
};

// Code of padded-matrix element (k, n); `bits` = 4 or 8.
__device__ __forceinline__ uint32_t padded_code(const uint8_t *codes, const uint8_t *zeros,
                                                const Shape &sh, int k, int n, int bits) {
    if (n >= sh.N) return 0u;
    if (k < sh.K) return codes[(size_t)k * sh.N + n];
    const int r = k / sh.g;
    if (zeros == nullptr) return 1u << (bits - 1);
    return r < sh.rows ? zeros[(size_t)r * sh.N + n] : 0u;
}

// One thread per (8-row block, column) of the padded matrix: consecutive threads read
// consecutive columns.
__global__ void pack_codes_kernel(const uint8_t *__restrict__ codes,
                                  const uint8_t *__restrict__ zeros, Shape sh,
                                  uint32_t *__restrict__ out) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)(sh.Kp >> 3) * sh.Np;
    if (i >= total) return;
    const int n = (int)(i % sh.Np);
    const int k0 = (int)(i / sh.Np) * 8;
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        w |= (padded_code(codes, zeros, sh, k0 + e, n, 4) & 0xFu) << (4 * nibble_pos(e));
    out[code_word_index(k0, n, sh.Kp)] = w;
}

// One thread per (8-row block, column) of the user matrix.
__global__ void unpack_codes_kernel(const uint32_t *__restrict__ in, Shape sh,
                                    uint8_t *__restrict__ codes) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)(sh.K >> 3) * sh.N;
    if (i >= total) return;
    const int n = (int)(i % sh.N);
    const int k0 = (int)(i / sh.N) * 8;
    const uint32_t w = in[code_word_index(k0, n, sh.Kp)];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        codes[(size_t)(k0 + e) * sh.N + n] = (uint8_t)((w >> (4 * nibble_pos(e))) & 0xFu);
    }
}

// Meta element index e <-> (group r, column n) of the padded matrix:
// e = (n/16)*G*16 + r*16 + n%16, G = Kp/g.
__device__ __forceinline__ void meta_coords(size_t e, int groups, int *r, int *n) {
    const size_t row = e >> 4;                   // (strip, group) pair
    *r = (int)(row % groups);
    *n = (int)(row / groups) * 16 + (int)(e & 15);
}

__device__ __forceinline__ bool user_cell(const Shape &sh, int r, int n) {
    return r < sh.rows && n < sh.N;
}

// One thread per element of the padded meta plane: scale, and (4-bit) the zero nibble
// pair of even elements.
__global__ void pack_meta_kernel(const uint16_t *__restrict__ scales,
                                 const uint8_t *__restrict__ zeros, Shape sh,
                                 uint16_t *__restrict__ out_scales,
                                 uint8_t *__restrict__ out_zeros) {
    const int groups = sh.Kp / sh.g;
    const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t count = (size_t)groups * sh.Np;
    if (e >= count) return;
    int r, n;
    meta_coords(e, groups, &r, &n);
    const bool in = user_cell(sh, r, n);
    out_scales[e] = in ? scales[(size_t)r * sh.N + n] : (uint16_t)0;
    if (zeros != nullptr && (e & 1) == 0) {
        int r1, n1;
        meta_coords(e + 1, groups, &r1, &n1);
        const uint32_t z0 = in ? zeros[(size_t)r * sh.N + n] & sh.zmask : 0u;
        const uint32_t z1 = user_cell(sh, r1, n1) ? zeros[(size_t)r1 * sh.N + n1] & sh.zmask : 0u;
        out_zeros[e >> 1] = (uint8_t)(z0 | (z1 << 4));
    }
}

__global__ void unpack_meta_kernel(const uint16_t *__restrict__ in_scales,
                                   const uint8_t *__restrict__ in_zeros, Shape sh,
                                   uint16_t *__restrict__ scales, uint8_t *__restrict__ zeros) {
    const int groups = sh.Kp / sh.g;
    const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t count = (size_t)groups * sh.Np;
    if (e >= count) return;
    int r, n;
    meta_coords(e, groups, &r, &n);
    if (!user_cell(sh, r, n)) return;
    scales[(size_t)r * sh.N + n] = in_scales[e];
    if (in_zeros != nullptr) {
        const uint32_t b = in_zeros[e >> 1];
        zeros[(size_t)r * sh.N + n] = (uint8_t)((e & 1) ? (b >> 4) : (b & 0xFu));
    }
}

// ---- 2-bit and 3-bit codes: tiles of 16 columns x 128 k, 4 * b bytes per lane ----
//
// Pair register r = 4t + j of lane L holds elements 2j (low half) and 2j + 1 (high half)
// of MFMA step t: rows k = 32t + 8 (L / 16) + 2j (+1) of the tile, column L % 16.
//   2-bit: word r / 8, field at bit 16 h + 2 (r % 4) + 8 ((r % 8) / 4);
//   3-bit: r < 15: word r / 5, field at bit 16 h + 3 (r % 5); r = 15: bit c of the code in
//          word c at bit 16 h + 15.

// One thread per (tile, lane) of the padded matrix.
__global__ void pack_codes_low_kernel(const uint8_t *__restrict__ codes,
                                      const uint8_t *__restrict__ zeros, Shape sh, int bits,
                                      uint32_t *__restrict__ out) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int tiles_k = sh.Kp >> 7;
    if (i >= (size_t)(sh.Np >> 4) * tiles_k * 64) return;
    const int L = (int)(i & 63);
    const size_t T = i >> 6;
    const int strip = (int)(T / tiles_k), kt = (int)(T % tiles_k);
    const int n = strip * 16 + (L & 15);
    const uint32_t mask = (1u << bits) - 1;
    uint32_t w[3] = {0u, 0u, 0u};
    for (int r = 0; r < 16; ++r) {
        const int t = r >> 2, j = r & 3;
        for (int h = 0; h < 2; ++h) {
            const int k = kt * 128 + 32 * t + 8 * (L >> 4) + 2 * j + h;
            const uint32_t q = padded_code(codes, zeros, sh, k, n, bits) & mask;
            if (bits == 2) {
                w[r >> 3] |= q << (16 * h + 2 * (r & 3) + 8 * ((r & 7) >> 2));
            } else if (r < 15) {
                w[r / 5] |= q << (16 * h + 3 * (r % 5));
            } else {
                for (int c = 0; c < 3; ++c) w[c] |= ((q >> c) & 1u) << (16 * h + 15);
            }
        }
    }
    uint32_t *dst = out + (T * 256 * bits + (size_t)L * 4 * bits) / 4;
    for (int c = 0; c < bits; ++c) dst[c] = w[c];
}

// One thread per (tile, lane) of the padded matrix; writes the user part.
__global__ void unpack_codes_low_kernel(const uint32_t *__restrict__ in, Shape sh, int bits,
                                        uint8_t *__restrict__ codes) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int tiles_k = sh.Kp >> 7;
    if (i >= (size_t)(sh.Np >> 4) * tiles_k * 64) return;
    const int L = (int)(i & 63);
    const size_t T = i >> 6;
    const int strip = (int)(T / tiles_k), kt = (int)(T % tiles_k);
    const int n = strip * 16 + (L & 15);
    if (n >= sh.N) return;
    const uint32_t *src = in + (T * 256 * bits + (size_t)L * 4 * bits) / 4;
    uint32_t w[3] = {0u, 0u, 0u};
    for (int c = 0; c < bits; ++c) w[c] = src[c];
    for (int r = 0; r < 16; ++r) {
        const int t = r >> 2, j = r & 3;
        for (int h = 0; h < 2; ++h) {
            const int k = kt * 128 + 32 * t + 8 * (L >> 4) + 2 * j + h;
            if (k >= sh.K) continue;
            uint32_t q;
            if (bits == 2) {
                q = (w[r >> 3] >> (16 * h + 2 * (r & 3) + 8 * ((r & 7) >> 2))) & 3u;
            } else if (r < 15) {
                q = (w[r / 5] >> (16 * h + 3 * (r % 5))) & 7u;
            } else {
                q = 0;
                for (int c = 0; c < 3; ++c) q |= ((w[c] >> (16 * h + 15)) & 1u) << c;
            }
            codes[(size_t)k * sh.N + n] = (uint8_t)q;
        }
    }
}

// ---- 8-bit codes: tiles of 16 columns x 64 k, one byte per code ----

// Byte offset of the 8-byte run holding rows k0..k0+7 (k0 % 8 == 0) of column n.
__device__ __forceinline__ size_t code8_run_offset(int k0, int n, int K) {
    const size_t tile = (size_t)(n >> 4) * (size_t)(K >> 6) + (size_t)(k0 >> 6);
    const int kk = k0 & 63;
    const int lane = (n & 15) + 16 * ((kk & 31) >> 3);
    return tile * 1024 + (size_t)lane * 16 + (size_t)(kk >> 5) * 8;
}

// One thread per (8-row block, column) of the padded matrix, as for 4-bit codes.
__global__ void pack_codes8_kernel(const uint8_t *__restrict__ codes,
                                   const uint8_t *__restrict__ zeros, Shape sh,
                                   uint8_t *__restrict__ out) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)(sh.Kp >> 3) * sh.Np;
    if (i >= total) return;
    const int n = (int)(i % sh.Np);
    const int k0 = (int)(i / sh.Np) * 8;
    u32x2_t run = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e)
        run[e >> 2] |= (padded_code(codes, zeros, sh, k0 + e, n, 8) & 0xFFu) << (8 * (e & 3));
    *reinterpret_cast<u32x2_t *>(out + code8_run_offset(k0, n, sh.Kp)) = run;
}

__global__ void unpack_codes8_kernel(const uint8_t *__restrict__ in, Shape sh,
                                     uint8_t *__restrict__ codes) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)(sh.K >> 3) * sh.N;
    if (i >= total) return;
    const int n = (int)(i % sh.N);
    const int k0 = (int)(i / sh.N) * 8;
    const u32x2_t run =
        *reinterpret_cast<const u32x2_t *>(in + code8_run_offset(k0, n, sh.Kp));
#pragma unroll
    for (int e = 0; e < 8; ++e)
        codes[(size_t)(k0 + e) * sh.N + n] = (uint8_t)(run[e >> 2] >> (8 * (e & 3)));
}

// Meta for 8-bit codes: scales as above, one zero byte per element.
__global__ void pack_meta8_kernel(const uint16_t *__restrict__ scales,
                                  const uint8_t *__restrict__ zeros, Shape sh,
                                  uint16_t *__restrict__ out_scales,
                                  uint8_t *__restrict__ out_zeros) {
    const int groups = sh.Kp / sh.g;
    const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (size_t)groups * sh.Np) return;
    int r, n;
    meta_coords(e, groups, &r, &n);
    const bool in = user_cell(sh, r, n);
    out_scales[e] = in ? scales[(size_t)r * sh.N + n] : (uint16_t)0;
    if (zeros != nullptr) out_zeros[e] = in ? zeros[(size_t)r * sh.N + n] : (uint8_t)0;
}

__global__ void unpack_meta8_kernel(const uint16_t *__restrict__ in_scales,
                                    const uint8_t *__restrict__ in_zeros, Shape sh,
                                    uint16_t *__restrict__ scales, uint8_t *__restrict__ zeros) {
    const int groups = sh.Kp / sh.g;
    const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (size_t)groups * sh.Np) return;
    int r, n;
    meta_coords(e, groups, &r, &n);
    if (!user_cell(sh, r, n)) return;
    scales[(size_t)r * sh.N + n] = in_scales[e];
    if (in_zeros != nullptr) zeros[(size_t)r * sh.N + n] = in_zeros[e];
}

// Sub-4-bit packed codes -> the 4-bit packed layout of the same matrix (both layouts cut
// 16 x 128 tiles the same way and give lane L the same elements: element (t, i) of lane L
// is pair register r = 4t + i/2, half i%2, of the b-bit words, and nibble i/2 or 4 + i/2
// of 4-bit word t).  Every code gains `add`: 0 for asymmetric codes (their b-bit zeros are
// valid 4-bit zeros), 8 - 2^(b-1) for symmetric ones, whose zero point 2^(b-1) then
// becomes the 4-bit symmetric zero 8.  Each dequantized weight is unchanged bit for bit.
// One thread per (tile, lane); padding cells hold the zero point either way.
__global__ void repack_low_u4_kernel(const uint32_t *__restrict__ in, size_t lanes, int bits,
                                     uint32_t add, u32x4_t *__restrict__ out) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= lanes) return;
    const uint32_t *src = in + i * bits;      // tile T = i / 64 at word T*64*bits, lane at L*bits
    uint32_t w[3] = {0u, 0u, 0u};
    for (int c = 0; c < bits; ++c) w[c] = src[c];
    u32x4_t o = {0u, 0u, 0u, 0u};
    for (int r = 0; r < 16; ++r) {
        const int t = r >> 2, j = r & 3;
        for (int h = 0; h < 2; ++h) {
            uint32_t q;
            if (bits == 2) {
                q = (w[r >> 3] >> (16 * h + 2 * (r & 3) + 8 * ((r & 7) >> 2))) & 3u;
            } else if (r < 15) {
                q = (w[r / 5] >> (16 * h + 3 * (r % 5))) & 7u;
            } else {
                q = 0;
                for (int c = 0; c < 3; ++c) q |= ((w[c] >> (16 * h + 15)) & 1u) << c;
            }
            o[t] |= (q + add) << (4 * (j + 4 * h));
        }
    }
    out[i] = o;                               // 4-bit tile T at 1 KiB, lane L at 16 bytes
}

unsigned blocks_for(size_t total, unsigned threads) {
    return (unsigned)((total + threads - 1) / threads);
}

}  // namespace

namespace {

Shape shape_of(int K, int N, int group, int bits = 4) {
    Shape sh;
    sh.K = K;
    sh.N = N;
    sh.Kp = padded_k(K);
    sh.Np = padded_n(N);
    sh.g = group;
    sh.rows = (K + group - 1) / group;
    sh.zmask = bits < 4 ? (1u << bits) - 1 : 0xFu;
    return sh;
}

// Launches the code and meta kernels of one direction over `code_items` / `meta_items`.
template <typename CodeFn, typename MetaFn>
hipError_t launch_two(size_t code_items, size_t meta_items, CodeFn code, MetaFn meta) {
    const unsigned threads = 256;
    if (code_items) code(blocks_for(code_items, threads), threads);
    if (meta_items) meta(blocks_for(meta_items, threads), threads);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                       int K, int N, int group, void *packed_codes, void *packed_meta,
                       hipStream_t stream) {
    const Shape sh = shape_of(K, N, group);
    const size_t metas = (size_t)(sh.Kp / group) * sh.Np;
    uint16_t *ms = (uint16_t *)packed_meta;
    uint8_t *mz = zeros ? (uint8_t *)packed_meta + metas * 2 : nullptr;
    return launch_two(
        (size_t)(sh.Kp >> 3) * sh.Np, metas,
        [&](unsigned b, unsigned t) {
            pack_codes_kernel<<<b, t, 0, stream>>>(codes, zeros, sh, (uint32_t *)packed_codes);
        },
        [&](unsigned b, unsigned t) {
            pack_meta_kernel<<<b, t, 0, stream>>>(scales, zeros, sh, ms, mz);
        });
}

hipError_t launch_unpack(const void *packed_codes, const void *packed_meta, int K, int N,
                         int group, int symmetric, uint8_t *codes, uint16_t *scales,
                         uint8_t *zeros, hipStream_t stream) {
    const Shape sh = shape_of(K, N, group);
    const size_t metas = (size_t)(sh.Kp / group) * sh.Np;
    const uint16_t *ms = (const uint16_t *)packed_meta;
    const uint8_t *mz = symmetric ? nullptr : (const uint8_t *)packed_meta + metas * 2;
    return launch_two(
        (size_t)(K >> 3) * N, metas,
        [&](unsigned b, unsigned t) {
            unpack_codes_kernel<<<b, t, 0, stream>>>((const uint32_t *)packed_codes, sh, codes);
        },
        [&](unsigned b, unsigned t) {
            unpack_meta_kernel<<<b, t, 0, stream>>>(ms, mz, sh, scales,
                                                    symmetric ? nullptr : zeros);
        });
}

hipError_t launch_pack_lowbit(int bits, const uint8_t *codes, const uint16_t *scales,
                              const uint8_t *zeros, int K, int N, int group, void *packed_codes,
                              void *packed_meta, hipStream_t stream) {
    const Shape sh = shape_of(K, N, group, bits);
    const size_t metas = (size_t)(sh.Kp / group) * sh.Np;
    uint16_t *ms = (uint16_t *)packed_meta;
    uint8_t *mz = zeros ? (uint8_t *)packed_meta + metas * 2 : nullptr;
    return launch_two(
        (size_t)(sh.Np >> 4) * (sh.Kp >> 7) * 64, metas,
        [&](unsigned b, unsigned t) {
            pack_codes_low_kernel<<<b, t, 0, stream>>>(codes, zeros, sh, bits,
                                                       (uint32_t *)packed_codes);
        },
        [&](unsigned b, unsigned t) {
            pack_meta_kernel<<<b, t, 0, stream>>>(scales, zeros, sh, ms, mz);
        });
}

hipError_t launch_unpack_lowbit(int bits, const void *packed_codes, const void *packed_meta,
                                int K, int N, int group, int symmetric, uint8_t *codes,
                                uint16_t *scales, uint8_t *zeros, hipStream_t stream) {
    const Shape sh = shape_of(K, N, group, bits);
    const size_t metas = (size_t)(sh.Kp / group) * sh.Np;
    const uint16_t *ms = (const uint16_t *)packed_meta;
    const uint8_t *mz = symmetric ? nullptr : (const uint8_t *)packed_meta + metas * 2;
    return launch_two(
        (size_t)(sh.Np >> 4) * (sh.Kp >> 7) * 64, metas,
        [&](unsigned b, unsigned t) {
            unpack_codes_low_kernel<<<b, t, 0, stream>>>((const uint32_t *)packed_codes, sh, bits,
                                                         codes);
        },
        [&](unsigned b, unsigned t) {
            unpack_meta_kernel<<<b, t, 0, stream>>>(ms, mz, sh, scales,
                                                    symmetric ? nullptr : zeros);
        });
}

hipError_t launch_repack_lowbit_u4(int bits, bool symmetric, const void *packed_codes, int Kp,
                                   int Np, void *out, hipStream_t stream) {
    const size_t lanes = (size_t)(Np >> 4) * (Kp >> 7) * 64;
    const uint32_t add = symmetric ? 8u - (1u << (bits - 1)) : 0u;
    if (lanes)
        repack_low_u4_kernel<<<blocks_for(lanes, 256), 256, 0, stream>>>(
            (const uint32_t *)packed_codes, lanes, bits, add, (u32x4_t *)out);
    return hipGetLastError();
}

hipError_t launch_pack_w8(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                          int K, int N, int group, void *packed_codes, void *packed_meta,
                          hipStream_t stream) {
    const Shape sh = shape_of(K, N, group);
    const size_t metas = (size_t)(sh.Kp / group) * sh.Np;
    uint16_t *ms = (uint16_t *)packed_meta;
    uint8_t *mz = zeros ? (uint8_t *)packed_meta + metas * 2 : nullptr;
    return launch_two(
        (size_t)(sh.Kp >> 3) * sh.Np, metas,
        [&](unsigned b, unsigned t) {
            pack_codes8_kernel<<<b, t, 0, stream>>>(codes, zeros, sh, (uint8_t *)packed_codes);
        },
        [&](unsigned b, unsigned t) {
            pack_meta8_kernel<<<b, t, 0, stream>>>(scales, zeros, sh, ms, mz);
        });
}

hipError_t launch_unpack_w8(const void *packed_codes, const void *packed_meta, int K, int N,
                            int group, int symmetric, uint8_t *codes, uint16_t *scales,
                            uint8_t *zeros, hipStream_t stream) {
    const Shape sh = shape_of(K, N, group);
    const size_t metas = (size_t)(sh.Kp / group) * sh.Np;
    const uint16_t *ms = (const uint16_t *)packed_meta;
    const uint8_t *mz = symmetric ? nullptr : (const uint8_t *)packed_meta + metas * 2;
    return launch_two(
        (size_t)(K >> 3) * N, metas,
        [&](unsigned b, unsigned t) {
            unpack_codes8_kernel<<<b, t, 0, stream>>>((const uint8_t *)packed_codes, sh, codes);
        },
        [&](unsigned b, unsigned t) {
            unpack_meta8_kernel<<<b, t, 0, stream>>>(ms, mz, sh, scales,
                                                     symmetric ? nullptr : zeros);
        });
}

}  // namespace mpgemm
