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

// One thread per (8-row block, column): consecutive threads read consecutive columns.
__global__ void pack_codes_kernel(const uint8_t *__restrict__ codes, int K, int N,
                                  uint32_t *__restrict__ out) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)(K >> 3) * N;
    if (i >= total) return;
    const int n = (int)(i % N);
    const int k0 = (int)(i / N) * 8;
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t q = codes[(size_t)(k0 + e) * N + n] & 0xFu;
        w |= q << (4 * nibble_pos(e));
    }
    out[code_word_index(k0, n, K)] = w;
}

__global__ void unpack_codes_kernel(const uint32_t *__restrict__ in, int K, int N,
                                    uint8_t *__restrict__ codes) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)(K >> 3) * N;
    if (i >= total) return;
    const int n = (int)(i % N);
    const int k0 = (int)(i / N) * 8;
    const uint32_t w = in[code_word_index(k0, n, K)];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        codes[(size_t)(k0 + e) * N + n] = (uint8_t)((w >> (4 * nibble_pos(e))) & 0xFu);
    }
}

// Meta element index e <-> (group r, column n): e = (n/16)*G*16 + r*16 + n%16, G = K/g.
__device__ __forceinline__ void meta_coords(size_t e, int groups, int *r, int *n) {
    const size_t row = e >> 4;                   // (strip, group) pair
    *r = (int)(row % groups);
    *n = (int)(row / groups) * 16 + (int)(e & 15);
}

// One thread per output byte of the meta plane: scale bytes first, then zero bytes.
__global__ void pack_meta_kernel(const uint16_t *__restrict__ scales,
                                 const uint8_t *__restrict__ zeros, int groups, int N,
                                 uint16_t *__restrict__ out_scales,
                                 uint8_t *__restrict__ out_zeros) {
    const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t count = (size_t)groups * N;
    if (e >= count) return;
    int r, n;
    meta_coords(e, groups, &r, &n);
    out_scales[e] = scales[(size_t)r * N + n];
    if (zeros != nullptr && (e & 1) == 0) {
        int r1, n1;
        meta_coords(e + 1, groups, &r1, &n1);
        const uint32_t z0 = zeros[(size_t)r * N + n] & 0xFu;
        const uint32_t z1 = zeros[(size_t)r1 * N + n1] & 0xFu;
        out_zeros[e >> 1] = (uint8_t)(z0 | (z1 << 4));
    }
}

__global__ void unpack_meta_kernel(const uint16_t *__restrict__ in_scales,
                                   const uint8_t *__restrict__ in_zeros, int groups, int N,
                                   uint16_t *__restrict__ scales, uint8_t *__restrict__ zeros) {
    const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t count = (size_t)groups * N;
    if (e >= count) return;
    int r, n;
    meta_coords(e, groups, &r, &n);
    scales[(size_t)r * N + n] = in_scales[e];
    if (in_zeros != nullptr) {
        const uint32_t b = in_zeros[e >> 1];
        zeros[(size_t)r * N + n] = (uint8_t)((e & 1) ? (b >> 4) : (b & 0xFu));
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

// One thread per (8-row block, column), as for 4-bit codes.
__global__ void pack_codes8_kernel(const uint8_t *__restrict__ codes, int K, int N,
                                   uint8_t *__restrict__ out) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)(K >> 3) * N;
    if (i >= total) return;
    const int n = (int)(i % N);
    const int k0 = (int)(i / N) * 8;
    u32x2_t run = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e)
        run[e >> 2] |= (uint32_t)codes[(size_t)(k0 + e) * N + n] << (8 * (e & 3));
    *reinterpret_cast<u32x2_t *>(out + code8_run_offset(k0, n, K)) = run;
}

__global__ void unpack_codes8_kernel(const uint8_t *__restrict__ in, int K, int N,
                                     uint8_t *__restrict__ codes) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t total = (size_t)(K >> 3) * N;
    if (i >= total) return;
    const int n = (int)(i % N);
    const int k0 = (int)(i / N) * 8;
    const u32x2_t run = *reinterpret_cast<const u32x2_t *>(in + code8_run_offset(k0, n, K));
#pragma unroll
    for (int e = 0; e < 8; ++e)
        codes[(size_t)(k0 + e) * N + n] = (uint8_t)(run[e >> 2] >> (8 * (e & 3)));
}

// Meta for 8-bit codes: scales as above, one zero byte per element.
__global__ void pack_meta8_kernel(const uint16_t *__restrict__ scales,
                                  const uint8_t *__restrict__ zeros, int groups, int N,
                                  uint16_t *__restrict__ out_scales,
                                  uint8_t *__restrict__ out_zeros) {
    const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (size_t)groups * N) return;
    int r, n;
    meta_coords(e, groups, &r, &n);
    out_scales[e] = scales[(size_t)r * N + n];
    if (zeros != nullptr) out_zeros[e] = zeros[(size_t)r * N + n];
}

__global__ void unpack_meta8_kernel(const uint16_t *__restrict__ in_scales,
                                    const uint8_t *__restrict__ in_zeros, int groups, int N,
                                    uint16_t *__restrict__ scales, uint8_t *__restrict__ zeros) {
    const size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (size_t)groups * N) return;
    int r, n;
    meta_coords(e, groups, &r, &n);
    scales[(size_t)r * N + n] = in_scales[e];
    if (in_zeros != nullptr) zeros[(size_t)r * N + n] = in_zeros[e];
}

unsigned blocks_for(size_t total, unsigned threads) {
    return (unsigned)((total + threads - 1) / threads);
}

}  // namespace

hipError_t launch_pack(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                       int K, int N, int group, void *packed_codes, void *packed_meta,
                       hipStream_t stream) {
    const unsigned threads = 256;
    const size_t words = (size_t)(K >> 3) * N;
    const int groups = K / group;
    const size_t metas = (size_t)groups * N;
    uint16_t *ms = (uint16_t *)packed_meta;
    uint8_t *mz = zeros ? (uint8_t *)packed_meta + metas * 2 : nullptr;
    if (words) {
        pack_codes_kernel<<<blocks_for(words, threads), threads, 0, stream>>>(
            codes, K, N, (uint32_t *)packed_codes);
    }
    if (metas) {
        pack_meta_kernel<<<blocks_for(metas, threads), threads, 0, stream>>>(scales, zeros,
                                                                             groups, N, ms, mz);
    }
    return hipGetLastError();
}

hipError_t launch_unpack(const void *packed_codes, const void *packed_meta, int K, int N,
                         int group, int symmetric, uint8_t *codes, uint16_t *scales,
                         uint8_t *zeros, hipStream_t stream) {
    const unsigned threads = 256;
    const size_t words = (size_t)(K >> 3) * N;
    const int groups = K / group;
    const size_t metas = (size_t)groups * N;
    const uint16_t *ms = (const uint16_t *)packed_meta;
    const uint8_t *mz = symmetric ? nullptr : (const uint8_t *)packed_meta + metas * 2;
    if (words) {
        unpack_codes_kernel<<<blocks_for(words, threads), threads, 0, stream>>>(
            (const uint32_t *)packed_codes, K, N, codes);
    }
    if (metas) {
        unpack_meta_kernel<<<blocks_for(metas, threads), threads, 0, stream>>>(
            ms, mz, groups, N, scales, symmetric ? nullptr : zeros);
    }
    return hipGetLastError();
}

hipError_t launch_pack_w8(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                          int K, int N, int group, void *packed_codes, void *packed_meta,
                          hipStream_t stream) {
    const unsigned threads = 256;
    const size_t runs = (size_t)(K >> 3) * N;
    const int groups = K / group;
    const size_t metas = (size_t)groups * N;
    uint16_t *ms = (uint16_t *)packed_meta;
    uint8_t *mz = zeros ? (uint8_t *)packed_meta + metas * 2 : nullptr;
    if (runs) {
        pack_codes8_kernel<<<blocks_for(runs, threads), threads, 0, stream>>>(
            codes, K, N, (uint8_t *)packed_codes);
    }
    if (metas) {
        pack_meta8_kernel<<<blocks_for(metas, threads), threads, 0, stream>>>(scales, zeros,
                                                                              groups, N, ms, mz);
    }
    return hipGetLastError();
}

hipError_t launch_unpack_w8(const void *packed_codes, const void *packed_meta, int K, int N,
                            int group, int symmetric, uint8_t *codes, uint16_t *scales,
                            uint8_t *zeros, hipStream_t stream) {
    const unsigned threads = 256;
    const size_t runs = (size_t)(K >> 3) * N;
    const int groups = K / group;
    const size_t metas = (size_t)groups * N;
    const uint16_t *ms = (const uint16_t *)packed_meta;
    const uint8_t *mz = symmetric ? nullptr : (const uint8_t *)packed_meta + metas * 2;
    if (runs) {
        unpack_codes8_kernel<<<blocks_for(runs, threads), threads, 0, stream>>>(
            (const uint8_t *)packed_codes, K, N, codes);
    }
    if (metas) {
        unpack_meta8_kernel<<<blocks_for(metas, threads), threads, 0, stream>>>(
            ms, mz, groups, N, scales, symmetric ? nullptr : zeros);
    }
    return hipGetLastError();
}

}  // namespace mpgemm
