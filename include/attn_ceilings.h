/*
 * attn_ceilings.h -- measured throughput ceilings of the GPU, the second denominator next to the
 * published peaks in the roofline of the attention forward (libattn_ceilings.so).
 *
 * The attention kernels are bound by one of two resources: the dense 16-bit matrix rate (the
 * none and causal modes, whose arithmetic intensity is far above the ridge) or HBM streaming
 * (the block-diagonal mode, which reads Q, K and V once and writes O once).  The published peaks
 * of those resources assume the top clock; what a kernel can sustain depends on the clock the
 * chip holds under that load.  These two calls measure it with the simplest kernels that keep
 * one resource busy:
 *
 *   attn_ceiling_mfma_bf16  v_mfma_f32_32x32x16_bf16 issued back to back by two waves per SIMD
 *                           on every compute unit (four accumulator chains per wave), with
 *                           pseudo-random operands (uniform in [-2, 2)) that differ from one
 *                           MFMA to the next, so the matrix cores switch like they do on real
 *                           data.  Rate = FLOPs of the MFMAs issued (32*32*16*2 each) / time.
 *   attn_ceiling_hbm_3r1w   the block-diagonal traffic mix: three arrays of bytes_per_array
 *                           bytes read and one written, 16-byte non-temporal accesses.
 *                           Rate = 4 * bytes_per_array / time.
 *
 * Each call allocates its own device buffers, runs `warmup` untimed launches and then `launches`
 * timed ones back to back on the default stream, synchronises, frees its buffers and stores the
 * sustained rate of the timed launches in *out (TFLOP/s, resp. GB/s with 1 GB = 1e9 bytes).
 * It returns 0, or the failing hipError_t value (then *out is untouched); warmup < 0,
 * launches < 1, bytes_per_array not a positive multiple of 16, or a NULL out return
 * hipErrorInvalidValue.  Calibration only: the attention entry points never call these, and they
 * synchronise the device, so they must not run while other work is timed.
 */
#ifndef ATTN_CEILINGS_H
#define ATTN_CEILINGS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

int attn_ceiling_mfma_bf16(int warmup, int launches, double* tflops);
int attn_ceiling_hbm_3r1w(int warmup, int launches, size_t bytes_per_array, double* gbs);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_CEILINGS_H */
