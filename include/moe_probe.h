/*
 * moe_probe.h - bandwidth probes of libmoe.so, for measurement only (not part of the hot path).
 *
 * The practical HBM ceilings of the three access patterns the path's kernels mix, measured on the
 * running GPU with the cache policies of those kernels (16-byte buffer loads with the nt policy of
 * data read once, 16-byte streaming stores): a write-only fill, a read-only stream and a copy. The bench
 * reports each kernel's bandwidth against the ceiling of its own read/write mix next to the
 * specification peak ("Ascend DeepEP MoE Dispatch Optimization", section "结论": the pages measure
 * dispatch against the hardware's theoretical bandwidth).
 *
 * Every pointer is a device pointer, 16-byte aligned; bytes > 0 and a multiple of 16. Each call
 * enqueues one kernel on `stream` and returns MOE_OK, MOE_ERR_ARG (bad pointer or size) or
 * MOE_ERR_HIP (launch failure).
 */
#ifndef MOE_PROBE_MI355X_H
#define MOE_PROBE_MI355X_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Writes every byte of dst[0, bytes) (the values are unspecified). */
int moe_probe_fill(void *dst, int64_t bytes, hipStream_t stream);

/* Reads every byte of src[0, bytes); sink (one uint32) is written only for one unlikely data
 * pattern, so that the loads are kept. */
int moe_probe_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream);

/* dst[0, bytes) = src[0, bytes); the ranges must not overlap. */
int moe_probe_copy(const void *src, void *dst, int64_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_MI355X_H */
