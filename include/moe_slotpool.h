/*
 * moe_slotpool.h - bounded HBM slot pool for streamed routed experts.
 *
 * The pages keep only the dense core resident and stream routed experts on
 * demand into a bounded pool that evicts with "LFU plus recency" (page "Show
 * HN: Run an 80B Qwen in 4.3 GB of RAM on a Mac and a 35B on an iPhone",
 * how-it-works list and prior-art paragraph; creativeainews explainer, "How
 * Expert Streaming Works"), one read per fixed-stride expert blob.  Here the
 * backing store is pinned host memory and a miss is one host-to-device copy
 * on a side stream: by default one kernel per acquire that reads the missed
 * blobs straight from the pinned host memory over the host link (many
 * compute units keep more reads in flight than one copy engine does), or,
 * with MOE_POOL_DMA_COPY or when the host memory has no device mapping, one
 * hipMemcpyAsync per miss.  The pages give no formula; this pool's policy:
 *
 *  - per layer, slots_per_layer slots of blob_stride bytes in device_slab;
 *  - every resident expert carries (count, last_use); counts are halved
 *    (integer shift) once per aging_period steps (0 = never), applied lazily
 *    when the layer is next touched;
 *  - acquire: requested experts already resident are hits (count += 1,
 *    last_use = step, pinned); then each miss, in request order, takes the
 *    lowest-numbered free slot, else evicts the unpinned resident expert with
 *    the smallest (count, last_use, expert id); it enters with count 1,
 *    last_use = step, pinned, and its blob is copied into the slot;
 *  - release unpins every slot of the layer.
 *
 * Hazards (explicit, as the pages' what-was-built list says theirs are):
 *  - read-after-write: the compute stream waits on an event recorded on
 *    copy_stream after the acquire's copies;
 *  - write-after-read: a copy into a slot of layer l waits on the event that
 *    the last slotpool_release(l) recorded on the compute stream.
 * One compute stream per pool; a pool is not thread-safe.
 */
#ifndef MOE_AMD_MOE_SLOTPOOL_H
#define MOE_AMD_MOE_SLOTPOOL_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_slotpool moe_slotpool;

#define MOE_POOL_HOST_ONLY 1u /* policy only: no copies, no events, no device writes */
#define MOE_POOL_DMA_COPY 2u  /* copy misses with hipMemcpyAsync (a copy engine) instead of the copy kernel */

typedef struct {
  int32_t n_layers, n_experts, slots_per_layer, aging_period;
  uint64_t blob_stride;       /* bytes between blobs (host) and between slots (device); multiple of 256 */
  uint64_t blob_bytes;        /* bytes copied per miss, <= blob_stride */
  const uint8_t* host_blobs;  /* host, pinned: [n_layers][n_experts][blob_stride] */
  uint8_t* device_slab;       /* device: [n_layers][slots_per_layer][blob_stride] */
  uint64_t* device_offsets;   /* device: [n_layers][n_experts]; entry of a resident expert = slot * blob_stride,
                                 relative to device_slab + layer * slots_per_layer * blob_stride */
  moe_stream copy_stream;     /* side stream for host-to-device copies (not the NULL stream) */
  uint32_t flags;             /* MOE_POOL_* */
} moe_slotpool_config;

typedef struct {
  uint64_t hits, misses, evictions, bytes_h2d;
} moe_slotpool_stats;

moe_status slotpool_create(const moe_slotpool_config* cfg, moe_slotpool** out);

/* Make experts[0..n) of `layer` resident and pinned (host array, distinct
 * ids).  Enqueues the miss copies on copy_stream, the device-offset updates
 * and the wait for the copies on `compute`.  Optional host outputs per
 * request: slot_out[n], victim_out[n] (evicted expert or -1), hit_out[n].
 * MOE_EPOOLFULL when the misses outnumber free plus evictable slots; the pool
 * is then unchanged. */
moe_status slotpool_acquire(moe_slotpool* pool, int32_t layer, const int32_t* experts, int32_t n, uint64_t step,
                            moe_stream compute, int32_t* slot_out, int32_t* victim_out, uint8_t* hit_out);

/* Unpin every slot of `layer` and record its write-after-read event on compute. */
moe_status slotpool_release(moe_slotpool* pool, int32_t layer, moe_stream compute);

/* Drop an unpinned resident expert (no-op when not resident; MOE_EBUSY when pinned). */
moe_status slotpool_evict(moe_slotpool* pool, int32_t layer, int32_t expert);

moe_status slotpool_stats(const moe_slotpool* pool, moe_slotpool_stats* out);

void slotpool_destroy(moe_slotpool* pool);

#ifdef __cplusplus
}
#endif

#endif /* MOE_AMD_MOE_SLOTPOOL_H */
