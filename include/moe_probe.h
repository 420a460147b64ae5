/*
 * moe_probe.h - measurement helper: a plain streaming read of device memory.
 *
 * Not part of the MoE method.  It gives the benchmark a reproducible
 * practical ceiling for kernels that stream weights from HBM: how fast a
 * kernel that does nothing but read can move bytes, as a function of how
 * many workgroups it runs (the FFN kernels run one 512-thread workgroup per
 * compute unit).
 */
#ifndef MOE_AMD_MOE_PROBE_H
#define MOE_AMD_MOE_PROBE_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes at `src` (device, 256-byte aligned, bytes a multiple
 * of 16384) once: n_workgroups workgroups of 512 threads take contiguous
 * equal parts (rounded to 16 KiB); every thread issues four 16-byte loads
 * before it waits, and folds what it read into one word of `sink` (device,
 * n_workgroups uint32), so the loads cannot be dropped.  n_workgroups in
 * [1, 65536].  Enqueued on `stream`. */
moe_status moe_read_probe(const void* src, uint64_t bytes, int32_t n_workgroups, uint32_t* sink,
                          moe_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_AMD_MOE_PROBE_H */
