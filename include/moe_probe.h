/*
 * moe_probe.h -- measurement aids beside the MoE ABI of moe.h, built into
 * the same library: plain HBM stream kernels (read, write, copy of one
 * contiguous device buffer) and a register-only matrix-core loop.  The
 * HBM-bound stages of the layer (route, permute, combine) are read against
 * the rates the stream kernels reach on the device, the copy is the
 * known-size transfer that calibrates the HBM byte counters of the profiler,
 * and the matrix-core loop gives the bf16 MFMA rate the device sustains with
 * no memory traffic at all, which the grouped GEMM is read against beside
 * the nominal peak.  Not part of the method the pages describe.
 */
#ifndef MOE_MI355X_PROBE_H
#define MOE_MI355X_PROBE_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* kind 0: read `bytes` of src (nothing is written unless the data XORs to a
 *         fixed improbable value; then one word goes to sink, which may be
 *         NULL);
 * kind 1: write `bytes` of a fixed pattern to dst;
 * kind 2: copy `bytes` from src to dst.
 * nontemporal != 0 uses non-temporal loads and stores.  bytes must be a
 * multiple of 16 and the buffers 16-byte aligned (else MOE_ERR_INVALID_ARG);
 * the call only enqueues the kernel on `stream`. */
moe_status moe_stream_probe(int32_t kind, int32_t nontemporal, const void *src, void *dst, size_t bytes,
                            void *sink, void *stream);

/* `blocks` workgroups of 4 waves; each wave loads its operands once from
 * `operands` (bf16, 4096 values = 8 KB per wave: 32 KB per workgroup, so the
 * buffer holds blocks * 32 KB; fill it with random values, since the
 * matrix core's power and so the clock depend on the data), then issues
 * `iters` rounds of 8 v_mfma_f32_32x32x16_bf16 into 8 independent
 * accumulators (a 128 x 64 block of 32 x 32 tiles; the B operands of
 * alternate rounds differ) and nothing else; iters is rounded up to an
 * even count.  Flops = blocks * 4 * iters * 8 * 32768.  The accumulators
 * are summed into one float per wave, which goes to sink[wave] (blocks * 4
 * floats) only if it equals a fixed improbable value (sink may be NULL).  blocks and iters
 * must be positive and operands 16-byte aligned (else MOE_ERR_INVALID_ARG);
 * the call only enqueues the kernel on `stream`. */
moe_status moe_mfma_probe(int32_t blocks, int32_t iters, const void *operands, void *sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_PROBE_H */
