// Host-to-device copies of listed expert blobs (the slot pool's miss copies),
// shared by the standalone copy kernel and the copy workgroups that the
// gate/up GEMV kernel runs beside its own for a streamed FFN.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Two byte ranges of every listed blob: list[0] = n, list[1 + i] = the source
// blob, list[1 + cap + i] = the destination slot.  Offsets and lengths are
// multiples of 16; a zero length skips a range.
struct BlobCopy {
  const uint8_t* host;   // source blob b at host + b * stride (device mapping of pinned host memory)
  uint8_t* dev;          // destination slot s at dev + s * stride
  uint64_t stride;
  const int32_t* list;   // nullptr: nothing to copy
  int cap;
  uint64_t off[2];
  uint64_t len[2];
};

constexpr int kCopyDepth = 4;   // 16-byte reads in flight per thread

// Workgroup wg of n_wg (NT threads) copies its share: the n x 2 ranges,
// concatenated as 16-byte words, are cut into n_wg contiguous pieces.  The
// piece's word range [k0, k1) is returned (k0 >= k1: nothing to copy).
// COH: every store is an agent-scope atomic store (written through to
// memory, so a later load from any compute unit that misses its caches sees
// it once the store has completed).
__device__ __forceinline__ void store16_coherent(uint4* p, const uint4 v) {
  uint64_t* q = reinterpret_cast<uint64_t*>(p);
  __hip_atomic_store(q, static_cast<uint64_t>(v.x) | (static_cast<uint64_t>(v.y) << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, static_cast<uint64_t>(v.z) | (static_cast<uint64_t>(v.w) << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
template <int NT, bool COH = false>
__device__ __forceinline__ void blob_copy_part(const BlobCopy& c, int wg, int n_wg, uint64_t& k0, uint64_t& k1) {
  const int n = __builtin_amdgcn_readfirstlane(c.list[0]);
  const uint64_t w0 = c.len[0] / 16, w1 = c.len[1] / 16, per = w0 + w1;
  const uint64_t total = per * static_cast<uint64_t>(n);
  k0 = k1 = 0;
  if (total == 0) return;
  const uint64_t piece = (total + n_wg - 1) / n_wg;
  k0 = piece * wg;
  k1 = k0 + piece < total ? k0 + piece : total;
  if (k0 >= k1) return;
  const int i0 = static_cast<int>(k0 / per), i1 = static_cast<int>((k1 - 1) / per);
  for (int i = i0; i <= i1; ++i) {
    const uint64_t b = static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(c.list[1 + i]));
    const uint64_t sl = static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(c.list[1 + c.cap + i]));
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const uint64_t s0 = per * i + (r ? w0 : 0);
      const uint64_t s1 = s0 + (r ? w1 : w0);
      const uint64_t lo = k0 > s0 ? k0 : s0;
      const uint64_t hi = k1 < s1 ? k1 : s1;
      if (lo >= hi) continue;
      const uint4* src = reinterpret_cast<const uint4*>(c.host + b * c.stride + c.off[r]) + (lo - s0);
      uint4* dst = reinterpret_cast<uint4*>(c.dev + sl * c.stride + c.off[r]) + (lo - s0);
      const int64_t cnt = static_cast<int64_t>(hi - lo);
      // kCopyDepth = 4 reads in flight, in named registers (an array here
      // is placed in LDS or scratch memory by the compiler)
      for (int64_t k = threadIdx.x; k < cnt; k += kCopyDepth * NT) {
        const bool m0 = k < cnt, m1 = k + NT < cnt, m2 = k + 2 * NT < cnt, m3 = k + 3 * NT < cnt;
        uint4 v0, v1, v2, v3;
        if (m0) v0 = src[k];
        if (m1) v1 = src[k + NT];
        if (m2) v2 = src[k + 2 * NT];
        if (m3) v3 = src[k + 3 * NT];
        if constexpr (COH) {
          if (m0) store16_coherent(dst + k, v0);
          if (m1) store16_coherent(dst + k + NT, v1);
          if (m2) store16_coherent(dst + k + 2 * NT, v2);
          if (m3) store16_coherent(dst + k + 3 * NT, v3);
        } else {
          if (m0) dst[k] = v0;
          if (m1) dst[k + NT] = v1;
          if (m2) dst[k + 2 * NT] = v2;
          if (m3) dst[k + 3 * NT] = v3;
        }
      }
    }
  }
}

// The copies of a streamed FFN (the slot pool's misses of one layer), run by
// the first kStreamCopyWgs workgroups of the gate/up GEMV beside its
// products: first the sections that gate/up reads, counted per list entry in
// `ready` once they are in memory, then the sections that the kernels after
// gate/up read.  A gate/up workgroup whose row is a miss waits for its
// entry's count before it loads weights.  Those loads find nothing stale in
// the caches: the caches start the kernel clean, and nothing in the kernel
// reads a missed slot before its wait.  The handoff uses no cache-wide
// write-back or invalidation (those cost tens of microseconds per kernel
// here): the first sections are written through with agent-scope atomic
// stores, and their completion is awaited before the count is raised.
struct StreamCopy {
  BlobCopy first;            // list == nullptr: no streamed copy
  BlobCopy second;           // same list, source and destination; other ranges
  const int32_t* entry_of;   // [T*K]: list entry of routed row j, -1: resident (no wait)
  uint32_t* ready;           // entry i's counter at ready[i * kReadyStride]: 16-byte words of its first
                             // ranges copied (zero at launch)
};
// each counter on a 256-byte line of its own: polls of one line serialise
// (and load the memory channel that holds it)
constexpr int kReadyStride = 64;
// the copy workgroups come first in the grid, so in-order dispatch puts them
// on the chip before any workgroup that waits for them
constexpr int kStreamCopyWgs = 64;
// a wait gives up after this many polls (each a memory round trip and a
// short sleep: well over 0.1 s) and flags the call
constexpr int kStreamSpinLimit = 1 << 17;

template <int NT>
__device__ __forceinline__ void stream_copy(const StreamCopy& c, int wg) {
  uint64_t k0, k1;
  blob_copy_part<NT, true>(c.first, wg, kStreamCopyWgs, k0, k1);
  // every thread's stores have completed before the count is raised
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0 && k0 < k1) {
    const uint64_t per = (c.first.len[0] + c.first.len[1]) / 16;
    for (uint64_t i = k0 / per; i <= (k1 - 1) / per; ++i) {
      const uint64_t lo = k0 > per * i ? k0 : per * i;
      const uint64_t hi = k1 < per * (i + 1) ? k1 : per * (i + 1);
      __hip_atomic_fetch_add(c.ready + i * kReadyStride, static_cast<uint32_t>(hi - lo), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  blob_copy_part<NT>(c.second, wg, kStreamCopyWgs, k0, k1);
}

// Wait (thread 0 polls, the workgroup waits at a barrier) until entry ent's
// first ranges are complete; returns false if the wait gave up.
__device__ __forceinline__ bool stream_wait(const StreamCopy& c, int ent) {
  __shared__ int ok;
  if (threadIdx.x == 0) {
    const uint32_t target = static_cast<uint32_t>((c.first.len[0] + c.first.len[1]) / 16);
    int it = 0;
    while (__hip_atomic_load(c.ready + static_cast<size_t>(ent) * kReadyStride, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT) < target &&
           it < kStreamSpinLimit) {
      __builtin_amdgcn_s_sleep(8);
      ++it;
    }
    ok = it < kStreamSpinLimit;
  }
  __syncthreads();
  return ok != 0;
}

}  // namespace moe
