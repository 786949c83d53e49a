/*
 * mpgemm_probes.h -- peak microkernels of libmpgemm_probes.so (gfx950).
 *
 * These are measurement kernels, not part of the GEMM path: they measure the two
 * denominators the GEMM kernels are judged against on the machine at hand, beside the
 * published MI355X figures (8 TB/s HBM3E; 2.5 PFLOP/s dense fp16/bf16 MFMA):
 *   - a stream read of a device buffer through 128-bit buffer loads (the load the decode
 *     GEMM kernels issue for packed weights), whose time for a given byte count is the
 *     floor for any kernel that must read that many bytes;
 *   - a loop of in-place MFMAs (the instructions the GEMM kernels issue) on operands that
 *     are not zero, whose rate under the chip's power limit is the reachable matrix peak.
 *
 * Conventions as in mpgemm.h: device pointers owned by the caller, work enqueued on
 * `stream` (a hipStream_t), arguments checked before anything is enqueued, a negative
 * MPGEMM_ERR_* status on error (nothing enqueued), MPGEMM_OK (0) otherwise.
 */
#ifndef MPGEMM_PROBES_H
#define MPGEMM_PROBES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads `bytes` bytes of `buf` (16-byte aligned; bytes a positive multiple of 16): each
 * workgroup of 256 lanes reads a contiguous chunk of `chunk_kib` KiB (the last one may be
 * shorter) with `unroll` 16-byte loads per lane in flight (unroll in {4, 8, 16}); a wave's
 * loads cover 1 KiB contiguously.  The loaded words are combined and written to
 * sink[workgroup] only if they equal a value no realistic buffer produces, so the kernel
 * reads everything and writes (almost) nothing; `sink` must hold ceil(bytes / chunk)
 * 32-bit words.
 * Errors: MPGEMM_ERR_INVALID_ARG (null pointer, bytes == 0 or not a multiple of 16,
 * chunk_kib outside 1..65536, unroll not 4, 8 or 16, or more than 2^31 workgroups),
 * MPGEMM_ERR_ALIGNMENT, MPGEMM_ERR_HIP.
 */
int mpgemm_probe_hbm_read(const void *buf, size_t bytes, int chunk_kib, int unroll,
                          uint32_t *sink, void *stream);

/* MFMA kinds of mpgemm_probe_mfma. */
enum {
    MPGEMM_PROBE_MFMA_32X32X16_F16 = 0,
    MPGEMM_PROBE_MFMA_16X16X32_F16 = 1,
    MPGEMM_PROBE_MFMA_32X32X16_BF16 = 2,
    MPGEMM_PROBE_MFMA_16X16X32_BF16 = 3
};

/*
 * Runs `blocks` workgroups of four waves; each wave issues `iters` rounds of four
 * independent in-place steps of the given kind, a step being 32768 flops (one 32x32x16
 * MFMA, or two 16x16x32 MFMAs), on operands drawn from the lane index (finite, non-zero),
 * and writes one float per lane of its results to sink only if they equal a value the
 * loop cannot produce; `sink` must hold blocks * 256 floats.
 * Flops of one launch: blocks * 4 * iters * 4 * 32768.
 * Errors: MPGEMM_ERR_INVALID_ARG (unknown kind, iters < 1, blocks < 1, sink NULL),
 * MPGEMM_ERR_HIP.
 */
int mpgemm_probe_mfma(int kind, int iters, int blocks, float *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MPGEMM_PROBES_H */
