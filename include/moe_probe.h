/*
 * moe_probe.h -- a measurement aid beside the MoE ABI of moe.h: plain HBM
 * stream kernels (read, write, copy of one contiguous device buffer) built
 * into the same library.  The HBM-bound stages of the layer (route, permute,
 * combine) are read against the rates these reach on the device, and the
 * copy is the known-size transfer that calibrates the HBM byte counters of
 * the profiler.  Not part of the method the pages describe.
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

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_PROBE_H */
