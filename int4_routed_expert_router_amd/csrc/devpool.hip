// GPU-resident slot pool: the slot pool's replacement policy (include/
// moe_slotpool.h) run by a one-wave kernel, with the miss copies read from
// a device-side miss list, so that a streamed decode token needs no host
// round trip per layer and can be captured in a HIP graph.
#include <hip/hip_runtime.h>

#include <new>

#include "blob_copy.h"
#include "moe_common.h"
#include "moe_slotpool.h"
#include "moe_topk.h"
#include "devpool.h"

namespace moe {
moe_status set_error(moe_status code, const char* fmt, ...);
}  // namespace moe

namespace {

using moe::DevPoolGeom;
using moe::DevRoute;
using moe::TopkIn;
using moe::load_bias;
using moe::topk_finish;
using moe::topk_issue;

constexpr int kMaxSlotsPerLane = 16;   // slots_per_layer <= 1024 (the kernel is instantiated per slots per lane)
constexpr int kMissCap = 64;           // top_k <= 64

__device__ __forceinline__ uint64_t* hdr(uint8_t* st) { return reinterpret_cast<uint64_t*>(st); }

// Empty pool: no resident experts, step 0, statistics 0.
__global__ void k_devpool_reset(uint8_t* st, DevPoolGeom g) {
  const size_t tid = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const size_t nth = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = tid; i < 8; i += nth) hdr(st)[i] = 0;
  for (size_t i = tid; i < static_cast<size_t>(g.L); i += nth) reinterpret_cast<uint64_t*>(st + g.o_epoch)[i] = 0;
  for (size_t i = tid; i < static_cast<size_t>(g.L) * g.E; i += nth) reinterpret_cast<int32_t*>(st + g.o_slot_of)[i] = -1;
  const size_t ls = static_cast<size_t>(g.L) * g.S;
  for (size_t i = tid; i < ls; i += nth) {
    reinterpret_cast<int32_t*>(st + g.o_expert_in)[i] = -1;
    reinterpret_cast<uint32_t*>(st + g.o_count)[i] = 0;
    reinterpret_cast<uint64_t*>(st + g.o_last_use)[i] = 0;
  }
  for (size_t i = tid; i < 1 + 3 * kMissCap; i += nth)
    reinterpret_cast<int32_t*>(st + g.o_miss)[i] = (i >= 1 + 2 * kMissCap && i < 1 + 3 * kMissCap) ? -1 : 0;
  for (size_t i = tid; i < static_cast<size_t>(kMissCap) * moe::kReadyStride; i += nth)
    reinterpret_cast<uint32_t*>(st + g.o_ready)[i] = 0u;
}

// One acquire of `layer` for the K experts at idx (device), at the pool's
// step: aging, hits, then each miss in request order into the lowest free
// slot or in place of the unpinned resident expert with the smallest
// (count, last_use, expert id).  Lane i owns slots i, i + 64, ... (SPL slots
// per lane: S <= 64 SPL); every choice is a wave reduction, so the result is
// the host policy's, exactly.  Writes the layer's device offsets of the
// loaded experts, the miss list for the copy kernel, the statistics and,
// when trace is set, [K][3] = (slot, victim or -1, hit).  Ids that are not
// distinct or not in [0, E) change nothing and set the error word.
// bump_step: advance the step afterwards.
//
// KJ > 0: the kernel first selects the token's experts itself from the
// router's logit slices (the top-K kernel's code, KJ logits per lane) and
// writes the selection, weights and shared gate to rt (rt.idx == idx).
template <int SPL, int KJ>
__global__ __launch_bounds__(64) void k_devpool_acquire(uint8_t* st, DevPoolGeom g, int layer,
                                                        int32_t* __restrict__ idx, int K, int bump_step,
                                                        uint64_t* __restrict__ offsets, int32_t* __restrict__ trace,
                                                        DevRoute rt) {
  const int lane = threadIdx.x;
  const int S = g.S, E = g.E;
  uint64_t* h = hdr(st);
  int32_t* slot_of = reinterpret_cast<int32_t*>(st + g.o_slot_of) + static_cast<size_t>(layer) * E;
  int32_t* ein_g = reinterpret_cast<int32_t*>(st + g.o_expert_in) + static_cast<size_t>(layer) * S;
  uint32_t* cnt_g = reinterpret_cast<uint32_t*>(st + g.o_count) + static_cast<size_t>(layer) * S;
  uint64_t* lu_g = reinterpret_cast<uint64_t*>(st + g.o_last_use) + static_cast<size_t>(layer) * S;
  int32_t* miss = reinterpret_cast<int32_t*>(st + g.o_miss);
  int32_t* entry_of = miss + 1 + 2 * kMissCap;
  uint32_t* ready = reinterpret_cast<uint32_t*>(st + g.o_ready);
  uint64_t* epoch = reinterpret_cast<uint64_t*>(st + g.o_epoch) + layer;
  // an empty miss list until this acquire has placed its misses (so an
  // error return copies nothing), no request waiting, no copy counted
  if (lane == 0) miss[0] = 0;
  entry_of[lane] = -1;
  ready[lane * moe::kReadyStride] = 0u;
  // this layer's slots in registers, and the step and aging epoch: loaded
  // first, they do not depend on the request
  const uint64_t step = h[0];
  const uint64_t e0 = g.P > 0 ? *epoch : 0;
  int ein[SPL];
  uint32_t cnt[SPL];
  uint64_t lu[SPL];
  bool pin[SPL];
#pragma unroll
  for (int j = 0; j < SPL; ++j) {
    const int s = lane + 64 * j;
    ein[j] = s < S ? ein_g[s] : -2;   // -2: no slot
    cnt[j] = s < S ? cnt_g[s] : 0;
    lu[j] = s < S ? lu_g[s] : 0;
    pin[j] = false;
  }
  int e;
  if constexpr (KJ > 0) {
    __shared__ int32_t ssel[kMissCap];
    TopkIn<KJ> in;
    topk_issue(rt.part, rt.n_part, 1, E, 0, lane, in);
    float bj[KJ];
    load_bias(rt.bias, E, lane, bj);
    topk_finish(in, bj, rt.bias != nullptr, rt.n_part, E, K, 0, lane, idx, rt.w, rt.gamma, nullptr, ssel, K);
    __syncthreads();
    e = lane < K ? ssel[lane] : -1;
  } else {
    // the request: lane k < K holds expert k
    e = lane < K ? idx[lane] : -1;
  }
  bool bad = lane < K && (e < 0 || e >= E);
  for (int k = 0; k < K; ++k) {
    const int ek = __builtin_amdgcn_readlane(e, k);
    if (lane < K && lane != k && ek == e) bad = true;
  }
  if (__ballot(bad) != 0) {
    if (lane == 0) h[4] = 1;   // error word
    return;
  }
  // lazy aging: counts halved once per elapsed aging period
  if (g.P > 0) {
    const uint64_t ep = step / static_cast<uint64_t>(g.P);
    if (ep > e0) {
      const uint64_t d = ep - e0;
#pragma unroll
      for (int j = 0; j < SPL; ++j) cnt[j] = d >= 32 ? 0u : (cnt[j] >> d);
      if (lane == 0) *epoch = ep;
    }
  }
  // hits: the slot holding each requested expert, found in the slot
  // registers (the same answer as the expert -> slot table, which the
  // misses below keep up to date); count + 1, last use, pinned
  int hs = -1;
  for (int k = 0; k < K; ++k) {
    const int ek = __builtin_amdgcn_readlane(e, k);
    uint32_t found = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < SPL; ++j)
      if (ein[j] == ek) found = static_cast<uint32_t>(lane + 64 * j);
    const unsigned long long at = __ballot(found != 0xFFFFFFFFu);
    const int sk = at == 0ull ? -1 : __builtin_amdgcn_readlane(static_cast<int>(found), __ffsll(at) - 1);
    if (lane == k) hs = sk;
  }
  const bool hit = hs >= 0;
  for (int k = 0; k < K; ++k) {
    const int sk = __builtin_amdgcn_readlane(hs, k);
    if (sk < 0) continue;   // uniform
#pragma unroll
    for (int j = 0; j < SPL; ++j)
      if (lane + 64 * j == sk) {
        cnt[j] += 1;
        lu[j] = step;
        pin[j] = true;
      }
  }
  // misses in request order
  int my_slot = hs, my_victim = -1, my_entry = -1;
  int n_miss = 0, n_evict = 0;
  for (int k = 0; k < K; ++k) {
    if (__builtin_amdgcn_readlane(hs, k) >= 0) continue;   // a hit (uniform)
    const int ek = __builtin_amdgcn_readlane(e, k);
    // lowest free slot
    uint32_t free_s = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < SPL; ++j)
      if (ein[j] == -1) free_s = min(free_s, static_cast<uint32_t>(lane + 64 * j));
    free_s = moe::wave_min_u32_s(free_s);
    int s = static_cast<int>(free_s), victim = -1;
    if (free_s == 0xFFFFFFFFu) {
      // the unpinned resident expert with the smallest (count, last_use, id)
      uint32_t mc = 0xFFFFFFFFu;
#pragma unroll
      for (int j = 0; j < SPL; ++j)
        if (ein[j] >= 0 && !pin[j]) mc = min(mc, cnt[j]);
      mc = moe::wave_min_u32_s(mc);
      uint32_t mh = 0xFFFFFFFFu;
#pragma unroll
      for (int j = 0; j < SPL; ++j)
        if (ein[j] >= 0 && !pin[j] && cnt[j] == mc) mh = min(mh, static_cast<uint32_t>(lu[j] >> 32));
      mh = moe::wave_min_u32_s(mh);
      uint32_t ml = 0xFFFFFFFFu;
#pragma unroll
      for (int j = 0; j < SPL; ++j)
        if (ein[j] >= 0 && !pin[j] && cnt[j] == mc && static_cast<uint32_t>(lu[j] >> 32) == mh)
          ml = min(ml, static_cast<uint32_t>(lu[j]));
      ml = moe::wave_min_u32_s(ml);
      uint32_t me = 0xFFFFFFFFu;
      const uint64_t mlu = (static_cast<uint64_t>(mh) << 32) | ml;
#pragma unroll
      for (int j = 0; j < SPL; ++j)
        if (ein[j] >= 0 && !pin[j] && cnt[j] == mc && lu[j] == mlu) me = min(me, static_cast<uint32_t>(ein[j]));
      me = moe::wave_min_u32_s(me);   // K <= S, so an unpinned resident expert exists
      if (me == 0xFFFFFFFFu) {       // cannot happen: the launcher checks K <= S
        if (lane == 0) h[4] = 2;
        return;
      }
      victim = static_cast<int>(me);
      uint32_t vs = 0xFFFFFFFFu;
#pragma unroll
      for (int j = 0; j < SPL; ++j)
        if (ein[j] == victim) vs = static_cast<uint32_t>(lane + 64 * j);
      s = static_cast<int>(moe::wave_min_u32_s(vs));
      if (lane == 0) slot_of[victim] = -1;
      ++n_evict;
    }
#pragma unroll
    for (int j = 0; j < SPL; ++j)
      if (lane + 64 * j == s) {
        ein[j] = ek;
        cnt[j] = 1;
        lu[j] = step;
        pin[j] = true;
      }
    if (lane == 0) {
      slot_of[ek] = s;
      offsets[ek] = static_cast<uint64_t>(s) * g.stride;
      miss[1 + n_miss] = ek;
      miss[1 + kMissCap + n_miss] = s;
    }
    if (lane == k) {
      my_slot = s;
      my_victim = victim;
      my_entry = n_miss;
    }
    ++n_miss;
  }
#pragma unroll
  for (int j = 0; j < SPL; ++j) {
    const int s = lane + 64 * j;
    if (s < S) {
      ein_g[s] = ein[j];
      cnt_g[s] = cnt[j];
      lu_g[s] = lu[j];
    }
  }
  if (lane < K) entry_of[lane] = my_entry;
  if (trace != nullptr && lane < K) {
    trace[3 * lane] = my_slot;
    trace[3 * lane + 1] = my_victim;
    trace[3 * lane + 2] = hit ? 1 : 0;
  }
  if (lane == 0) {
    miss[0] = n_miss;
    h[1] += static_cast<uint64_t>(K - n_miss);
    h[2] += static_cast<uint64_t>(n_miss);
    h[3] += static_cast<uint64_t>(n_evict);
    if (bump_step) h[0] = step + 1;
  }
}

// The miss copies: the listed blobs' byte ranges, cut into equal pieces over
// the grid (entries past the list's length take no piece).
constexpr int kCopyWgs = 256;
__global__ __launch_bounds__(256) void k_copy_listed(moe::BlobCopy c) {
  uint64_t k0, k1;
  moe::blob_copy_part<256>(c, blockIdx.x, gridDim.x, k0, k1);
}

}  // namespace

struct moe_devpool {
  moe_slotpool_config cfg{};
  DevPoolGeom g{};
  uint8_t* state = nullptr;
  const uint8_t* host_dev = nullptr;   // device mapping of cfg.host_blobs
};

namespace moe {

DevPoolGeom devpool_geom(int L, int E, int S, int P, uint64_t stride) {
  auto al = [](size_t v) { return (v + 255) & ~size_t(255); };
  DevPoolGeom g{};
  g.L = L;
  g.E = E;
  g.S = S;
  g.P = P;
  g.stride = stride;
  size_t o = al(64);   // header: step, hits, misses, evictions, error word
  g.o_epoch = o; o += al(static_cast<size_t>(L) * 8);
  g.o_slot_of = o; o += al(static_cast<size_t>(L) * E * 4);
  g.o_expert_in = o; o += al(static_cast<size_t>(L) * S * 4);
  g.o_count = o; o += al(static_cast<size_t>(L) * S * 4);
  g.o_last_use = o; o += al(static_cast<size_t>(L) * S * 8);
  g.o_miss = o; o += al((1 + 3 * kMissCap) * 4);
  g.o_ready = o; o += al(static_cast<size_t>(kMissCap) * moe::kReadyStride * 4);
  g.bytes = o;
  return g;
}

template <int SPL>
static void launch_acquire(moe_devpool* p, int layer, int32_t* idx, int K, bool bump_step, int32_t* trace,
                           const DevRoute& rt, hipStream_t s) {
  const moe_slotpool_config& c = p->cfg;
  const uint64_t E = static_cast<uint64_t>(c.n_experts);
  uint64_t* off = c.device_offsets + layer * E;
  const int b = bump_step ? 1 : 0;
#define ACQ_LAUNCH(J) \
  hipLaunchKernelGGL((k_devpool_acquire<SPL, J>), dim3(1), dim3(64), 0, s, p->state, p->g, layer, idx, K, b, off, trace, rt)
  if (rt.part == nullptr) ACQ_LAUNCH(0);
  else if (E <= 64) ACQ_LAUNCH(1);
  else if (E <= 128) ACQ_LAUNCH(2);
  else if (E <= 256) ACQ_LAUNCH(4);
  else if (E <= 512) ACQ_LAUNCH(8);
  else ACQ_LAUNCH(16);
#undef ACQ_LAUNCH
}

BlobCopy devpool_miss_copy(const moe_devpool* p, int layer) {
  const moe_slotpool_config& c = p->cfg;
  const uint64_t S = static_cast<uint64_t>(c.slots_per_layer), E = static_cast<uint64_t>(c.n_experts);
  BlobCopy b{};
  b.host = p->host_dev + layer * E * c.blob_stride;
  b.dev = c.device_slab + layer * S * c.blob_stride;
  b.stride = c.blob_stride;
  b.list = reinterpret_cast<const int32_t*>(p->state + p->g.o_miss);
  b.cap = kMissCap;
  return b;
}

StreamCopy devpool_stream_copy(const moe_devpool* p, int layer) {
  StreamCopy c{};
  c.first = c.second = devpool_miss_copy(p, layer);
  int32_t* miss = reinterpret_cast<int32_t*>(p->state + p->g.o_miss);
  c.entry_of = miss + 1 + 2 * kMissCap;
  c.ready = reinterpret_cast<uint32_t*>(p->state + p->g.o_ready);
  return c;
}

hipError_t devpool_enqueue_acquire(moe_devpool* p, int layer, int32_t* idx, int K, bool bump_step, int32_t* trace,
                                   hipStream_t s, const DevRoute* route, bool copy) {
  const moe_slotpool_config& c = p->cfg;
  const uint64_t S = static_cast<uint64_t>(c.slots_per_layer);
  const DevRoute rt = route != nullptr ? *route : DevRoute{};
  if (rt.part != nullptr && (c.n_experts > moe::kMaxExperts || rt.w == nullptr || rt.gamma == nullptr))
    return hipErrorInvalidValue;
  const int spl = static_cast<int>((S + 63) / 64);
  if (spl <= 1) launch_acquire<1>(p, layer, idx, K, bump_step, trace, rt, s);
  else if (spl <= 2) launch_acquire<2>(p, layer, idx, K, bump_step, trace, rt, s);
  else if (spl <= 4) launch_acquire<4>(p, layer, idx, K, bump_step, trace, rt, s);
  else if (spl <= 8) launch_acquire<8>(p, layer, idx, K, bump_step, trace, rt, s);
  else launch_acquire<kMaxSlotsPerLane>(p, layer, idx, K, bump_step, trace, rt, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !copy) return e;
  BlobCopy b = devpool_miss_copy(p, layer);
  b.len[0] = c.blob_bytes;   // a multiple of 16 (checked at creation)
  hipLaunchKernelGGL(k_copy_listed, dim3(kCopyWgs), dim3(256), 0, s, b);
  return hipGetLastError();
}

const moe_slotpool_config& devpool_config(const moe_devpool* p) { return p->cfg; }

}  // namespace moe

using moe::set_error;

extern "C" {

moe_status moe_devpool_state_bytes(const moe_slotpool_config* c, size_t* bytes) {
  if (!c || !bytes) return set_error(MOE_EINVAL, "NULL config or bytes");
  if (c->n_layers <= 0 || c->n_experts <= 0 || c->slots_per_layer <= 0 || c->aging_period < 0)
    return set_error(MOE_ESHAPE, "bad pool geometry (layers=%d experts=%d slots=%d aging=%d)", c->n_layers,
                     c->n_experts, c->slots_per_layer, c->aging_period);
  *bytes = moe::devpool_geom(c->n_layers, c->n_experts, c->slots_per_layer, c->aging_period, c->blob_stride).bytes;
  return set_error(MOE_OK, "");
}

moe_status moe_devpool_create(const moe_slotpool_config* c, void* state, size_t state_bytes, moe_devpool** out) {
  if (!c || !out) return set_error(MOE_EINVAL, "NULL config or out");
  *out = nullptr;
  size_t need = 0;
  moe_status st = moe_devpool_state_bytes(c, &need);
  if (st) return st;
  if (c->slots_per_layer > c->n_experts || c->slots_per_layer > 64 * kMaxSlotsPerLane)
    return set_error(MOE_ESHAPE, "slots_per_layer=%d must be <= n_experts=%d and <= %d", c->slots_per_layer,
                     c->n_experts, 64 * kMaxSlotsPerLane);
  if (c->flags != 0) return set_error(MOE_EINVAL, "flags must be 0 (the device pool copies with its copy kernel)");
  if (c->blob_stride == 0 || c->blob_stride % 256 || c->blob_bytes == 0 || c->blob_bytes % 16 ||
      c->blob_bytes > c->blob_stride)
    return set_error(MOE_EINVAL, "blob_stride must be a positive multiple of 256 and >= blob_bytes, a multiple of 16");
  if (!c->host_blobs || !c->device_slab || !c->device_offsets)
    return set_error(MOE_EINVAL, "host_blobs, device_slab and device_offsets are required");
  if (reinterpret_cast<uintptr_t>(c->device_slab) % 256) return set_error(MOE_EINVAL, "device_slab must be 256-byte aligned");
  if (!state || reinterpret_cast<uintptr_t>(state) % 256 || state_bytes < need)
    return set_error(MOE_EINVAL, "state must be a 256-byte aligned device buffer of >= %zu bytes", need);
  void* dev = nullptr;
  if (hipHostGetDevicePointer(&dev, const_cast<uint8_t*>(c->host_blobs), 0) != hipSuccess || dev == nullptr) {
    (void)hipGetLastError();
    return set_error(MOE_EINVAL, "host_blobs must be pinned host memory mapped for the device");
  }
  moe_devpool* p = new (std::nothrow) moe_devpool;
  if (!p) return set_error(MOE_ENOMEM, "pool metadata allocation");
  p->cfg = *c;
  p->g = moe::devpool_geom(c->n_layers, c->n_experts, c->slots_per_layer, c->aging_period, c->blob_stride);
  p->state = static_cast<uint8_t*>(state);
  p->host_dev = static_cast<const uint8_t*>(dev);
  *out = p;
  return set_error(MOE_OK, "");
}

moe_status moe_devpool_reset(moe_devpool* p, moe_stream stream) {
  if (!p) return set_error(MOE_EINVAL, "pool is NULL");
  hipLaunchKernelGGL(k_devpool_reset, dim3(64), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), p->state, p->g);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(MOE_EHIP, "pool reset launch: %s", hipGetErrorString(e));
  return set_error(MOE_OK, "");
}

moe_status moe_devpool_acquire(moe_devpool* p, int32_t layer, const int32_t* experts, int32_t n, int32_t bump_step,
                               int32_t* trace, moe_stream stream) {
  if (!p) return set_error(MOE_EINVAL, "pool is NULL");
  if (layer < 0 || layer >= p->cfg.n_layers) return set_error(MOE_EINVAL, "layer %d out of range", layer);
  if (n < 1 || n > kMissCap || n > p->cfg.slots_per_layer || !experts)
    return set_error(MOE_EINVAL, "need 1 <= n <= min(64, slots_per_layer) device expert ids");
  const hipError_t e = moe::devpool_enqueue_acquire(p, layer, const_cast<int32_t*>(experts), n, bump_step != 0, trace,
                                                   reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return set_error(MOE_EHIP, "pool acquire launch: %s", hipGetErrorString(e));
  return set_error(MOE_OK, "");
}

moe_status moe_devpool_stats(const moe_devpool* p, moe_slotpool_stats* out, uint64_t* step_out, int32_t* error_out,
                             moe_stream stream) {
  if (!p || !out) return set_error(MOE_EINVAL, "NULL pool or out");
  uint64_t h[8] = {};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(h, p->state, sizeof(h), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return set_error(MOE_EHIP, "pool statistics read: %s", hipGetErrorString(e));
  out->hits = h[1];
  out->misses = h[2];
  out->evictions = h[3];
  out->bytes_h2d = h[2] * p->cfg.blob_bytes;
  out->prefetches = 0;
  if (step_out) *step_out = h[0];
  if (error_out) *error_out = static_cast<int32_t>(h[4]);
  return set_error(MOE_OK, "");
}

void moe_devpool_destroy(moe_devpool* p) { delete p; }

}  // extern "C"
