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
 *  - release unpins every slot of the layer;
 *  - prefetch (pre-gating: experts predicted for a later acquire, e.g. the
 *    next layer's router applied to the current layer's input) is best
 *    effort: aging first; requested experts already resident are left as
 *    they are; each other one, in request order, takes the lowest-numbered
 *    free slot, else evicts the unpinned resident expert with the smallest
 *    (count, last_use, expert id) among those this call does not request,
 *    else is skipped; it enters unpinned with count 0 and last_use = step,
 *    so the acquire that then hits it leaves the entry a miss would have
 *    left.
 *
 * Hazards (explicit, as the pages' what-was-built list says theirs are):
 *  - read-after-write: the compute stream waits on an event recorded on
 *    copy_stream after the acquire's copies;
 *  - write-after-read: a copy into a slot of layer l waits on the event that
 *    the last slotpool_release(l) recorded on the compute stream;
 *  - prefetch copies run on copy_stream without making the compute stream
 *    wait; the next acquire of that layer does (also when it has no miss).
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
  uint64_t prefetches;   /* experts loaded by slotpool_prefetch */
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

/* Best-effort early load of experts[0..n) of `layer` (host array, distinct
 * ids; policy above).  Enqueues their copies on copy_stream and their
 * device-offset updates on `compute`, which does not wait for the copies.
 * Optional host outputs, capacity n: *n_loaded_out = number of experts
 * loaded; expert_out, slot_out, victim_out (evicted expert or -1) describe
 * them in request order.  Never fails for lack of slots. */
moe_status slotpool_prefetch(moe_slotpool* pool, int32_t layer, const int32_t* experts, int32_t n, uint64_t step,
                             moe_stream compute, int32_t* n_loaded_out, int32_t* expert_out, int32_t* slot_out,
                             int32_t* victim_out);

/* Unpin every slot of `layer` and record its write-after-read event on compute. */
moe_status slotpool_release(moe_slotpool* pool, int32_t layer, moe_stream compute);

/* Drop an unpinned resident expert (no-op when not resident; MOE_EBUSY when pinned). */
moe_status slotpool_evict(moe_slotpool* pool, int32_t layer, int32_t expert);

moe_status slotpool_stats(const moe_slotpool* pool, moe_slotpool_stats* out);

/* The configuration the pool was created with. */
moe_status slotpool_get_config(const moe_slotpool* pool, moe_slotpool_config* out);

/* One batch-1 decode token through n_layers MoE layers whose routed experts
 * stream through `pool` (the pages' expert streaming: Show HN page,
 * how-it-works list), driven natively: for layer l, route x_l; with
 * pregate > 0, also route x_l with layer l+1's router (pre-gating); copy both
 * index sets to idx_host and wait for them; slotpool_acquire(l);
 * slotpool_prefetch(l+1) of the pregate highest-ranked predictions; expert
 * FFN from the pool's slots; combine with the residual epilogue;
 * slotpool_release(l).  So the prefetch copies of layer l+1 run while layer
 * l computes, and no per-layer work waits on an interpreter.
 *   pregate:  number of predictions to prefetch per layer (0 = none, values
 *             above top_k mean top_k)
 *   desc:     layer shape; top_k <= 64
 *   layers:   [n_layers] weights; router_w, router_bias and shared are used,
 *             experts / expert_stride / expert_offset are taken from the pool
 *             (device_slab + l * slots_per_layer * blob_stride, blob_stride,
 *             device_offsets + l * n_experts)
 *   step:     the pool's step (one per token)
 *   x0:       device [H] act_dtype, the token's input
 *   r:        device [H] fp32 residual, x0 as fp32 on entry, the final
 *             residual on exit
 *   x_buf:    device [2][H] act_dtype; layer l's epilogue writes x_{l+1} to
 *             x_buf[l % 2]
 *   idx_host: host [2][top_k] int32 staging for the index copies (pinned
 *             memory keeps the copies asynchronous)
 *   idx_log:  host [n_layers][2][top_k] int32 or NULL: layer l's selection,
 *             then the predictions prefetched at layer l for layer l+1 (-1
 *             where none)
 *   ws:       workspace of moe_workspace_bytes(desc, 1) bytes
 * Returns after the last layer is enqueued on `compute` (the copy stream is
 * the pool's).  The pool must have been created for n_layers layers with
 * device copies (not MOE_POOL_HOST_ONLY). */
moe_status moe_pool_decode_step(const moe_layer_desc* desc, const moe_layer_weights* layers, int32_t n_layers,
                                moe_slotpool* pool, uint64_t step, const void* x0, float* r, void* x_buf,
                                int32_t* idx_host, int32_t* idx_log, int32_t pregate, void* ws, size_t ws_bytes,
                                moe_stream compute);

void slotpool_destroy(moe_slotpool* pool);

/* GPU-resident slot pool.  The same policy as slotpool_acquire (residency,
 * LFU counts with lazy aging, recency, lowest-id tie-break; the prefetch
 * form is not offered), run by a one-wave kernel on the device on expert ids
 * that are already on the device (the top-K output), with its misses copied
 * by a kernel that reads the miss list from device memory and the blobs
 * from mapped pinned host memory.  Nothing waits for the host, so a streamed
 * decode token needs no host round trip per layer and can be captured in a
 * graph.  Pins last for one acquire: the decode loop releases every layer
 * before it is acquired again.  All work is ordered on the caller's stream
 * (copies, then the FFN that reads the slots, then later copies into them),
 * so there are no separate copy-stream events.
 *   cfg:   as for slotpool_create; copy_stream is not used; flags must be 0;
 *          host_blobs must be pinned host memory with a device mapping;
 *          blob_bytes a multiple of 16; slots_per_layer <= min(n_experts,
 *          1024)
 *   state: caller-owned device memory of moe_devpool_state_bytes() bytes
 *          (256-byte aligned) holding the residency tables, counts, the step
 *          and the statistics; moe_devpool_reset gives the empty pool. */
typedef struct moe_devpool moe_devpool;
moe_status moe_devpool_state_bytes(const moe_slotpool_config* cfg, size_t* bytes);
moe_status moe_devpool_create(const moe_slotpool_config* cfg, void* state, size_t state_bytes, moe_devpool** out);
/* Enqueues the empty pool (no resident expert, step 0, statistics 0). */
moe_status moe_devpool_reset(moe_devpool* pool, moe_stream stream);
/* Enqueues one acquire of the n device expert ids at experts (distinct, in
 * [0, n_experts); 1 <= n <= min(64, slots_per_layer)) at the pool's step and
 * the copies of its misses; the device offsets of layer are updated for the
 * loaded experts.  trace (device, [n][3] int32 or NULL): slot, evicted
 * expert or -1, hit (0/1) per request.  bump_step != 0: the step advances by
 * one afterwards.  Invalid ids change nothing and set the pool's error word
 * (moe_devpool_stats). */
moe_status moe_devpool_acquire(moe_devpool* pool, int32_t layer, const int32_t* experts, int32_t n,
                               int32_t bump_step, int32_t* trace, moe_stream stream);
/* Synchronous read of the statistics (prefetches = 0), the step and the
 * error word (0 = none) after the work enqueued on stream. */
moe_status moe_devpool_stats(const moe_devpool* pool, moe_slotpool_stats* out, uint64_t* step_out,
                             int32_t* error_out, moe_stream stream);
void moe_devpool_destroy(moe_devpool* pool);

/* One batch-1 decode token through n_layers layers streamed through a
 * GPU-resident pool, enqueued on stream with no host synchronisation:
 * per layer, the router (that of layers after the first also combines the
 * previous layer, as in moe_stack_forward); the pool's acquire, whose kernel
 * first selects the token's top-K experts from the router's logits (the
 * same selection as moe_route) and then applies the policy of
 * moe_devpool_acquire to them (the last layer's advances the step); the
 * expert FFN from the pool's slots, whose gate/up kernel also copies the
 * misses (the gate/up sections of every missed blob first: a missed
 * expert's products wait for its sections, the others do not; then the
 * down sections, complete before down runs; a desc that forces the grouped
 * family copies with the copy kernel after the acquire); then the last
 * combine.  A
 * wait that gives up sets MOE_FLAG_STREAM_WAIT in the call's status word
 * (moe.h).  Arguments as for
 * moe_pool_decode_step (layers' experts / stride / offsets come from the
 * pool); trace (device, [n_layers][top_k][3] int32 or NULL) receives every
 * layer's acquire trace.  The call can be captured (moe_pool_graph_create). */
moe_status moe_pool_decode_step_dev(const moe_layer_desc* desc, const moe_layer_weights* layers, int32_t n_layers,
                                    moe_devpool* pool, const void* x0, float* r, void* x_buf, int32_t* trace,
                                    void* ws, size_t ws_bytes, moe_stream stream);
/* moe_pool_decode_step_dev captured as a HIP graph (arguments fixed at
 * capture; the pool's step lives on the device, so every launch is the next
 * token).  capture_stream must not be the NULL stream. */
moe_status moe_pool_graph_create(const moe_layer_desc* desc, const moe_layer_weights* layers, int32_t n_layers,
                                 moe_devpool* pool, const void* x0, float* r, void* x_buf, int32_t* trace,
                                 void* ws, size_t ws_bytes, moe_stream capture_stream, moe_graph** out);

#ifdef __cplusplus
}
#endif

#endif /* MOE_AMD_MOE_SLOTPOOL_H */
