// Internal interface of the GPU-resident slot pool (devpool.hip) for the
// decode driver (moe_api.cpp).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "blob_copy.h"
#include "moe_slotpool.h"

namespace moe {

// Layout of the pool's device state (byte offsets): a header (step, hits,
// misses, evictions, error word), per layer the aging epoch, per layer and
// expert its slot (-1: not resident), per layer and slot the resident expert
// (-1: free), its count and last use, and the miss list of the last acquire
// ([0] = n, then n experts, from [1 + 64] their slots, from [1 + 128] each
// request's list entry (-1: a hit)), and the copy counters of a streamed FFN
// (one per list entry, kReadyStride words apart, cleared by the acquire).
struct DevPoolGeom {
  int L, E, S, P;
  uint64_t stride;
  size_t o_epoch, o_slot_of, o_expert_in, o_count, o_last_use, o_miss, o_ready, bytes;
};
DevPoolGeom devpool_geom(int L, int E, int S, int P, uint64_t stride);

// The token's routing for an acquire that selects the experts itself: the
// router's logit slices (n_part slices of [1][E+1], bias when the slices do
// not hold it) and where the selection's weights and shared gate go.
struct DevRoute {
  const float* part;
  int n_part;
  const float* bias;
  float* w;
  float* gamma;
};

// The miss copy of `layer`'s last acquire (list, source and destination
// set; no byte ranges).
BlobCopy devpool_miss_copy(const moe_devpool* p, int layer);
// The same as a streamed FFN's copy (both parts without ranges), with the
// acquire's per-request list entries and the copy counters it cleared.
StreamCopy devpool_stream_copy(const moe_devpool* p, int layer);
// The acquire kernel for K device expert ids of `layer`, then (copy) the
// copy kernel of its misses, on s.  bump_step: the pool's step advances
// after it.  With route, the acquire kernel first runs the top-K selection
// of the token from route's logits and writes it to idx (and the weights
// and gate to route's buffers); without it, idx holds the request.  Without
// copy the caller copies the misses (devpool_stream_copy) before they are
// read.
hipError_t devpool_enqueue_acquire(moe_devpool* p, int layer, int32_t* idx, int K, bool bump_step, int32_t* trace,
                                   hipStream_t s, const DevRoute* route = nullptr, bool copy = true);
const moe_slotpool_config& devpool_config(const moe_devpool* p);

}  // namespace moe
