// Slot pool C ABI: the host policy (slotpool_core.h) plus the HIP side -
// host-to-device miss copies on a side stream, device offset-table updates
// on the compute stream, and the RAW / WAR events between the two.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <new>
#include <vector>

#include "moe_slotpool.h"
#include "slotpool_core.h"

namespace moe {
// moe_api.cpp owns the thread-local error string; this file reports through it.
moe_status set_error(moe_status code, const char* fmt, ...);
}  // namespace moe

namespace {

constexpr int kOffsetBatch = 32;
struct OffsetBatch {
  int32_t n;
  int32_t expert[kOffsetBatch];
  uint64_t offset[kOffsetBatch];
};

__global__ void k_set_offsets(uint64_t* table, OffsetBatch b) {
  const int i = threadIdx.x;
  if (i < b.n) table[b.expert[i]] = b.offset[i];
}

// Copy of up to kOffsetBatch missed blobs from mapped pinned host memory into
// their slots: blockIdx.y = miss, blockIdx.x = contiguous slice of the blob.
// Each thread keeps kCopyDepth 16-byte host reads in flight.
constexpr int kCopySlices = 64;
constexpr int kCopyDepth = 4;
struct CopyBatch {
  int32_t n;
  uint64_t src[kOffsetBatch];   // byte offsets from the host base
  uint64_t dst[kOffsetBatch];   // byte offsets from the device slab base
};
__global__ __launch_bounds__(256) void k_copy_blobs(const uint8_t* __restrict__ host, uint8_t* __restrict__ dev,
                                                    uint64_t bytes, CopyBatch b) {
  const int i = blockIdx.y;
  if (i >= b.n) return;
  const uint4* src = reinterpret_cast<const uint4*>(host + b.src[i]);
  uint4* dst = reinterpret_cast<uint4*>(dev + b.dst[i]);
  const uint64_t n16 = bytes / 16;
  const uint64_t per = (n16 + kCopySlices - 1) / kCopySlices;
  const uint64_t k0 = blockIdx.x * per;
  const uint64_t k1 = k0 + per < n16 ? k0 + per : n16;
  // kCopyDepth = 4 reads in flight, in named registers (an array here is
  // placed in LDS by the compiler)
  static_assert(kCopyDepth == 4, "four named registers");
  for (uint64_t k = k0 + threadIdx.x; k < k1; k += kCopyDepth * 256) {
    const bool m0 = k < k1, m1 = k + 256 < k1, m2 = k + 512 < k1, m3 = k + 768 < k1;
    uint4 v0, v1, v2, v3;
    if (m0) v0 = src[k];
    if (m1) v1 = src[k + 256];
    if (m2) v2 = src[k + 512];
    if (m3) v3 = src[k + 768];
    if (m0) dst[k] = v0;
    if (m1) dst[k + 256] = v1;
    if (m2) dst[k + 512] = v2;
    if (m3) dst[k + 768] = v3;
  }
  // a tail of fewer than 16 bytes, by one thread
  if (blockIdx.x == 0 && threadIdx.x == 0)
    for (uint64_t t = n16 * 16; t < bytes; ++t) (dev + b.dst[i])[t] = (host + b.src[i])[t];
}

}  // namespace

struct moe_slotpool;
static hipError_t enqueue_loads(moe_slotpool* p, int layer, const std::vector<moe::PoolEvent>& ev, hipStream_t ks);

struct moe_slotpool {
  moe_slotpool_config cfg{};
  moe::PoolCore core;
  std::vector<hipEvent_t> ready, released;  // per layer
  std::vector<uint8_t> released_recorded;
  std::vector<uint8_t> pending;   // per layer: prefetch copies whose wait no acquire has enqueued yet
  uint64_t bytes_h2d = 0;
  std::vector<moe::PoolEvent> events, loaded;
  const uint8_t* host_dev = nullptr;   // device mapping of host_blobs (copy kernel), or null (copy engine)
  moe_slotpool(const moe_slotpool_config& c)
      : cfg(c), core(c.n_layers, c.n_experts, c.slots_per_layer, c.aging_period) {}
  bool host_only() const { return (cfg.flags & MOE_POOL_HOST_ONLY) != 0; }
};

using moe::set_error;

// Copies of the loaded (non-hit) entries of ev into their slots on the copy
// stream, after the layer's write-after-read event, and their device offset
// updates on ks; then records the layer's ready event on the copy stream.
static hipError_t enqueue_loads(moe_slotpool* p, int layer, const std::vector<moe::PoolEvent>& ev, hipStream_t ks) {
  hipStream_t cs = reinterpret_cast<hipStream_t>(p->cfg.copy_stream);
  const uint64_t stride = p->cfg.blob_stride;
  const uint64_t S = static_cast<uint64_t>(p->cfg.slots_per_layer), E = static_cast<uint64_t>(p->cfg.n_experts);
  hipError_t e = hipSuccess;
  if (p->released_recorded[layer]) e = hipStreamWaitEvent(cs, p->released[layer], 0);  // WAR
  uint8_t* slab = p->cfg.device_slab + static_cast<uint64_t>(layer) * S * stride;
  const uint64_t host_off = static_cast<uint64_t>(layer) * E * stride;
  const uint8_t* host = p->cfg.host_blobs + host_off;
  OffsetBatch batch{};
  CopyBatch copies{};
  auto flush_copies = [&]() {
    if (copies.n == 0) return;
    hipLaunchKernelGGL(k_copy_blobs, dim3(kCopySlices, copies.n), dim3(256), 0, cs, p->host_dev + host_off, slab,
                       p->cfg.blob_bytes, copies);
    copies.n = 0;
    if (e == hipSuccess) e = hipGetLastError();
  };
  for (size_t i = 0; i < ev.size() && e == hipSuccess; ++i) {
    if (ev[i].hit) continue;
    if (p->host_dev) {
      copies.src[copies.n] = static_cast<uint64_t>(ev[i].expert) * stride;
      copies.dst[copies.n] = static_cast<uint64_t>(ev[i].slot) * stride;
      if (++copies.n == kOffsetBatch) flush_copies();
    } else {
      e = hipMemcpyAsync(slab + static_cast<uint64_t>(ev[i].slot) * stride,
                         host + static_cast<uint64_t>(ev[i].expert) * stride, p->cfg.blob_bytes,
                         hipMemcpyHostToDevice, cs);
    }
    p->bytes_h2d += p->cfg.blob_bytes;
    batch.expert[batch.n] = ev[i].expert;
    batch.offset[batch.n] = static_cast<uint64_t>(ev[i].slot) * stride;
    if (++batch.n == kOffsetBatch) {
      hipLaunchKernelGGL(k_set_offsets, dim3(1), dim3(kOffsetBatch), 0, ks,
                         p->cfg.device_offsets + static_cast<uint64_t>(layer) * E, batch);
      batch.n = 0;
      if (e == hipSuccess) e = hipGetLastError();
    }
  }
  if (e == hipSuccess) flush_copies();
  if (e == hipSuccess && batch.n > 0) {
    hipLaunchKernelGGL(k_set_offsets, dim3(1), dim3(kOffsetBatch), 0, ks,
                       p->cfg.device_offsets + static_cast<uint64_t>(layer) * E, batch);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(p->ready[layer], cs);
  return e;
}

extern "C" {

moe_status slotpool_create(const moe_slotpool_config* c, moe_slotpool** out) {
  if (!c || !out) return set_error(MOE_EINVAL, "NULL config or out");
  *out = nullptr;
  if (c->n_layers <= 0 || c->n_experts <= 0 || c->slots_per_layer <= 0 || c->aging_period < 0)
    return set_error(MOE_ESHAPE, "bad pool geometry (layers=%d experts=%d slots=%d aging=%d)", c->n_layers,
                     c->n_experts, c->slots_per_layer, c->aging_period);
  if (c->slots_per_layer > c->n_experts)
    return set_error(MOE_ESHAPE, "slots_per_layer=%d exceeds n_experts=%d", c->slots_per_layer, c->n_experts);
  if (c->flags & ~(MOE_POOL_HOST_ONLY | MOE_POOL_DMA_COPY)) return set_error(MOE_EINVAL, "unknown flags 0x%x", c->flags);
  const bool host_only = (c->flags & MOE_POOL_HOST_ONLY) != 0;
  if (!host_only) {
    if (c->blob_stride == 0 || c->blob_stride % 256 || c->blob_bytes == 0 || c->blob_bytes > c->blob_stride)
      return set_error(MOE_EINVAL, "blob_stride must be a positive multiple of 256 and >= blob_bytes");
    if (!c->host_blobs || !c->device_slab || !c->device_offsets || !c->copy_stream)
      return set_error(MOE_EINVAL, "host_blobs, device_slab, device_offsets and copy_stream are required");
    if (reinterpret_cast<uintptr_t>(c->device_slab) % 256)
      return set_error(MOE_EINVAL, "device_slab must be 256-byte aligned");
  }
  moe_slotpool* p = new (std::nothrow) moe_slotpool(*c);
  if (!p) return set_error(MOE_ENOMEM, "pool metadata allocation");
  if (!host_only) {
    p->ready.assign(c->n_layers, nullptr);
    p->released.assign(c->n_layers, nullptr);
    p->released_recorded.assign(c->n_layers, 0);
    p->pending.assign(c->n_layers, 0);
    if (!(c->flags & MOE_POOL_DMA_COPY)) {
      void* dev = nullptr;
      if (hipHostGetDevicePointer(&dev, const_cast<uint8_t*>(c->host_blobs), 0) == hipSuccess && dev != nullptr)
        p->host_dev = static_cast<const uint8_t*>(dev);
      else
        (void)hipGetLastError();   // not mapped: the copy engine path is used
    }
    for (int l = 0; l < c->n_layers; ++l) {
      hipError_t e1 = hipEventCreateWithFlags(&p->ready[l], hipEventDisableTiming);
      hipError_t e2 = hipEventCreateWithFlags(&p->released[l], hipEventDisableTiming);
      if (e1 != hipSuccess || e2 != hipSuccess) {
        slotpool_destroy(p);
        return set_error(MOE_EHIP, "hipEventCreate: %s", hipGetErrorString(e1 != hipSuccess ? e1 : e2));
      }
    }
  }
  *out = p;
  return set_error(MOE_OK, "");
}

moe_status slotpool_acquire(moe_slotpool* p, int32_t layer, const int32_t* experts, int32_t n, uint64_t step,
                            moe_stream compute, int32_t* slot_out, int32_t* victim_out, uint8_t* hit_out) {
  if (!p) return set_error(MOE_EINVAL, "pool is NULL");
  if (layer < 0 || layer >= p->cfg.n_layers) return set_error(MOE_EINVAL, "layer %d out of range", layer);
  if (n < 0 || (n > 0 && !experts)) return set_error(MOE_EINVAL, "bad expert list");
  const moe::PoolCore::Result r = p->core.acquire(layer, experts, n, step, p->events);
  if (r == moe::PoolCore::kBadInput) return set_error(MOE_EINVAL, "expert ids must be distinct and in [0, %d)", p->cfg.n_experts);
  if (r == moe::PoolCore::kFull)
    return set_error(MOE_EPOOLFULL, "layer %d: more misses than free or evictable slots", layer);
  int n_miss = 0;
  for (int i = 0; i < n; ++i) {
    if (slot_out) slot_out[i] = p->events[i].slot;
    if (victim_out) victim_out[i] = p->events[i].victim;
    if (hit_out) hit_out[i] = p->events[i].hit ? 1 : 0;
    if (!p->events[i].hit) ++n_miss;
  }
  if (p->host_only()) {
    p->bytes_h2d += static_cast<uint64_t>(n_miss) * p->cfg.blob_bytes;
    return set_error(MOE_OK, "");
  }
  hipStream_t ks = reinterpret_cast<hipStream_t>(compute);
  hipError_t e = hipSuccess;
  if (n_miss > 0) e = enqueue_loads(p, layer, p->events, ks);
  // RAW: the compute stream waits for this acquire's copies and for any
  // earlier prefetch copies of the layer (the copy stream is in order, so
  // the ready event recorded last covers both)
  if (e == hipSuccess && (n_miss > 0 || p->pending[layer])) e = hipStreamWaitEvent(ks, p->ready[layer], 0);
  if (e != hipSuccess) return set_error(MOE_EHIP, "slot pool copy/offset enqueue: %s", hipGetErrorString(e));
  p->pending[layer] = 0;
  return set_error(MOE_OK, "");
}

moe_status slotpool_prefetch(moe_slotpool* p, int32_t layer, const int32_t* experts, int32_t n, uint64_t step,
                             moe_stream compute, int32_t* n_loaded_out, int32_t* expert_out, int32_t* slot_out,
                             int32_t* victim_out) {
  if (!p) return set_error(MOE_EINVAL, "pool is NULL");
  if (layer < 0 || layer >= p->cfg.n_layers) return set_error(MOE_EINVAL, "layer %d out of range", layer);
  if (n < 0 || (n > 0 && !experts)) return set_error(MOE_EINVAL, "bad expert list");
  const moe::PoolCore::Result r = p->core.prefetch(layer, experts, n, step, p->loaded);
  if (r == moe::PoolCore::kBadInput) return set_error(MOE_EINVAL, "expert ids must be distinct and in [0, %d)", p->cfg.n_experts);
  const int nl = static_cast<int>(p->loaded.size());
  if (n_loaded_out) *n_loaded_out = nl;
  for (int i = 0; i < nl; ++i) {
    if (expert_out) expert_out[i] = p->loaded[i].expert;
    if (slot_out) slot_out[i] = p->loaded[i].slot;
    if (victim_out) victim_out[i] = p->loaded[i].victim;
  }
  if (p->host_only()) {
    p->bytes_h2d += static_cast<uint64_t>(nl) * p->cfg.blob_bytes;
    return set_error(MOE_OK, "");
  }
  if (nl == 0) return set_error(MOE_OK, "");
  const hipError_t e = enqueue_loads(p, layer, p->loaded, reinterpret_cast<hipStream_t>(compute));
  if (e != hipSuccess) return set_error(MOE_EHIP, "slot pool prefetch enqueue: %s", hipGetErrorString(e));
  p->pending[layer] = 1;
  return set_error(MOE_OK, "");
}

moe_status slotpool_release(moe_slotpool* p, int32_t layer, moe_stream compute) {
  if (!p) return set_error(MOE_EINVAL, "pool is NULL");
  if (layer < 0 || layer >= p->cfg.n_layers) return set_error(MOE_EINVAL, "layer %d out of range", layer);
  p->core.release(layer);
  if (!p->host_only()) {
    hipError_t e = hipEventRecord(p->released[layer], reinterpret_cast<hipStream_t>(compute));
    if (e != hipSuccess) return set_error(MOE_EHIP, "release event: %s", hipGetErrorString(e));
    p->released_recorded[layer] = 1;
  }
  return set_error(MOE_OK, "");
}

moe_status slotpool_evict(moe_slotpool* p, int32_t layer, int32_t expert) {
  if (!p) return set_error(MOE_EINVAL, "pool is NULL");
  const moe::PoolCore::Result r = p->core.evict(layer, expert);
  if (r == moe::PoolCore::kBadInput) return set_error(MOE_EINVAL, "layer/expert out of range");
  if (r == moe::PoolCore::kBusy) return set_error(MOE_EBUSY, "layer %d expert %d is pinned", layer, expert);
  return set_error(MOE_OK, "");
}

moe_status slotpool_get_config(const moe_slotpool* p, moe_slotpool_config* out) {
  if (!p || !out) return set_error(MOE_EINVAL, "NULL pool or out");
  *out = p->cfg;
  return set_error(MOE_OK, "");
}

moe_status slotpool_stats(const moe_slotpool* p, moe_slotpool_stats* out) {
  if (!p || !out) return set_error(MOE_EINVAL, "NULL pool or out");
  out->hits = p->core.hits();
  out->misses = p->core.misses();
  out->evictions = p->core.evictions();
  out->bytes_h2d = p->bytes_h2d;
  out->prefetches = p->core.prefetches();
  return set_error(MOE_OK, "");
}

void slotpool_destroy(moe_slotpool* p) {
  if (!p) return;
  for (hipEvent_t ev : p->ready)
    if (ev) hipEventDestroy(ev);
  for (hipEvent_t ev : p->released)
    if (ev) hipEventDestroy(ev);
  delete p;
}

}  // extern "C"
