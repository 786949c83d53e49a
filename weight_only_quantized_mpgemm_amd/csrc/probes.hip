// Peak microkernels (include/mpgemm_probes.h): an HBM stream read and an MFMA loop, built
// into libmpgemm_probes.so, apart from the GEMM library.  They give the measured
// denominators against which the GEMM kernels' achieved bandwidth and flop rate are read,
// beside the published MI355X peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"
#include "mpgemm.h"
#include "mpgemm_probes.h"

namespace {

using namespace mpgemm;

constexpr uint32_t kNever = 0x9E3779B9u;     // a combined value no test buffer produces

// One workgroup reads one chunk: rounds of U 16-byte loads per lane, each load of a wave
// covering 1 KiB contiguously (lane l at 16 l, wave w at 1 KiB w, load u at 4 KiB u).  The
// chunk's descriptor is bounded to the chunk, so loads past its end read zeros without
// touching memory (a short last chunk needs no masking).
template <int U>
__global__ __launch_bounds__(256) void hbm_read_kernel(const uint8_t *__restrict__ buf,
                                                       uint64_t bytes, uint32_t chunk,
                                                       uint32_t *__restrict__ sink) {
    const uint64_t base = (uint64_t)blockIdx.x * chunk;
    const uint64_t left = bytes - base;
    const uint32_t mine = left < chunk ? (uint32_t)left : chunk;
    const rsrc_t r = make_rsrc(buf + base, mine);
    const uint32_t voff = threadIdx.x * 16u;
    constexpr uint32_t kRound = 256u * 16u * U;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (uint32_t off = 0; off < mine; off += kRound) {
        u32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = buf_load_b128(r, voff, off + u * 4096u);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == kNever) sink[blockIdx.x] = x;
}

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int KIND>
__device__ __forceinline__ void mfma_step(const u32x4_t &a, const u32x4_t &b, f32x16_t &c) {
    if constexpr (KIND == MPGEMM_PROBE_MFMA_32X32X16_F16)
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<half8_t>(a), bitcast<half8_t>(b), c,
                                                   0, 0, 0);
    else if constexpr (KIND == MPGEMM_PROBE_MFMA_32X32X16_BF16)
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8_t>(a), bitcast<bf16x8_t>(b),
                                                    c, 0, 0, 0);
    else {
        // Two 16x16x32 MFMAs (2 x 16384 flops) on the two halves of the accumulator.
        f32x4_t lo = {c[0], c[1], c[2], c[3]}, hi = {c[4], c[5], c[6], c[7]};
        if constexpr (KIND == MPGEMM_PROBE_MFMA_16X16X32_F16) {
            lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(a), bitcast<half8_t>(b),
                                                        lo, 0, 0, 0);
            hi = __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<half8_t>(b), bitcast<half8_t>(a),
                                                        hi, 0, 0, 0);
        } else {
            lo = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(a),
                                                         bitcast<bf16x8_t>(b), lo, 0, 0, 0);
            hi = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8_t>(b),
                                                         bitcast<bf16x8_t>(a), hi, 0, 0, 0);
        }
        c[0] = lo[0]; c[1] = lo[1]; c[2] = lo[2]; c[3] = lo[3];
        c[4] = hi[0]; c[5] = hi[1]; c[6] = hi[2]; c[7] = hi[3];
    }
}

// Four independent accumulator chains per wave keep the matrix unit busy across the
// dependent-issue latency of one chain.  Operands: 16-bit values of magnitude about 1/64
// to 1 drawn from the lane index, so the units toggle as on real data (all-zero operands
// draw less power and would overstate the reachable clock under load).
template <int KIND>
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float *__restrict__ sink) {
    const uint32_t h = (threadIdx.x + 1u) * 2654435761u;
    const bool bf = KIND == MPGEMM_PROBE_MFMA_32X32X16_BF16 ||
                    KIND == MPGEMM_PROBE_MFMA_16X16X32_BF16;
    // exponent field of 2^-6 .. 2^-1, random sign and mantissa bits
    const uint32_t e16 = bf ? 0x3C803C80u : 0x24002400u;
    u32x4_t a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t r1 = h * (2u * i + 3u), r2 = h * (2u * i + 5u);
        a[i] = e16 | (r1 & (bf ? 0x803F803Fu : 0x83FF83FFu)) | ((r1 >> 7) & 0x0C000C00u);
        b[i] = e16 | (r2 & (bf ? 0x803F803Fu : 0x83FF83FFu)) | ((r2 >> 7) & 0x0C000C00u);
    }
    f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        mfma_step<KIND>(a, b, c0);
        mfma_step<KIND>(b, a, c1);
        mfma_step<KIND>(a, a, c2);
        mfma_step<KIND>(b, b, c3);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    if (s == 1234.5f) sink[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int mpgemm_probe_hbm_read(const void *buf, size_t bytes, int chunk_kib, int unroll,
                          uint32_t *sink, void *stream) {
    if (buf == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0)
        return MPGEMM_ERR_INVALID_ARG;
    if (chunk_kib < 1 || chunk_kib > 65536) return MPGEMM_ERR_INVALID_ARG;
    if (((uintptr_t)buf & 15u) != 0) return MPGEMM_ERR_ALIGNMENT;
    const uint64_t chunk = (uint64_t)chunk_kib * 1024u;
    const uint64_t blocks = (bytes + chunk - 1) / chunk;
    if (blocks > 0x7FFFFFFFull) return MPGEMM_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)blocks), block(256);
    const uint8_t *p = (const uint8_t *)buf;
    switch (unroll) {
        case 4: hbm_read_kernel<4><<<grid, block, 0, s>>>(p, bytes, (uint32_t)chunk, sink); break;
        case 8: hbm_read_kernel<8><<<grid, block, 0, s>>>(p, bytes, (uint32_t)chunk, sink); break;
        case 16: hbm_read_kernel<16><<<grid, block, 0, s>>>(p, bytes, (uint32_t)chunk, sink); break;
        default: return MPGEMM_ERR_INVALID_ARG;
    }
    return hipGetLastError() == hipSuccess ? MPGEMM_OK : MPGEMM_ERR_HIP;
}

int mpgemm_probe_mfma(int kind, int iters, int blocks, float *sink, void *stream) {
    if (iters < 1 || blocks < 1 || sink == nullptr) return MPGEMM_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)blocks), block(256);
    switch (kind) {
        case MPGEMM_PROBE_MFMA_32X32X16_F16:
            mfma_kernel<MPGEMM_PROBE_MFMA_32X32X16_F16><<<grid, block, 0, s>>>(iters, sink);
            break;
        case MPGEMM_PROBE_MFMA_16X16X32_F16:
            mfma_kernel<MPGEMM_PROBE_MFMA_16X16X32_F16><<<grid, block, 0, s>>>(iters, sink);
            break;
        case MPGEMM_PROBE_MFMA_32X32X16_BF16:
            mfma_kernel<MPGEMM_PROBE_MFMA_32X32X16_BF16><<<grid, block, 0, s>>>(iters, sink);
            break;
        case MPGEMM_PROBE_MFMA_16X16X32_BF16:
            mfma_kernel<MPGEMM_PROBE_MFMA_16X16X32_BF16><<<grid, block, 0, s>>>(iters, sink);
            break;
        default: return MPGEMM_ERR_INVALID_ARG;
    }
    return hipGetLastError() == hipSuccess ? MPGEMM_OK : MPGEMM_ERR_HIP;
}

}  // extern "C"
