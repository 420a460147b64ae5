// Top-K selection of one token on one wave (used by the top-K kernel and,
// fused, by the batch-1 gate/up GEMV).  Selection order is (logit desc,
// expert index asc); the weights are the softmax restricted to the selected
// set; the shared gate is the sigmoid of the gate logit.
#pragma once
#include <utility>

#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

// Order-preserving map of a float onto uint32 (larger float, larger key).
// NaN is read as -inf (maxNum drops it), so a selection always exists, and
// -0 as +0, so the two zeros tie as they do under float comparison.  The key
// of -inf is 0x007FFFFF; key 0 is left free to mark "no entry".
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(fmaxf(f, -INFINITY) + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Batcher's odd-even merge sorting network over N (a power of two) entries
// held in registers: cas(a, b) with a < b must leave the pair in order.  All
// loop bounds are compile-time constants, so the network unrolls into
// straight-line code on constant register indices.
template <int N, class Cas>
__device__ __forceinline__ void oddeven_merge_sort(Cas cas) {
#pragma unroll
  for (int p = 1; p < N; p <<= 1) {
#pragma unroll
    for (int k = p; k >= 1; k >>= 1) {
#pragma unroll
      for (int j = k % p; j + k < N; j += 2 * k) {
#pragma unroll
        for (int i = 0; i < k; ++i) {
          if (i + j + k < N && (i + j) / (2 * p) == (i + j + k) / (2 * p)) cas(i + j, i + j + k);
        }
      }
    }
  }
}

// a[i] = a[i + 1] for i < N-1 where take is set.  Written over constant
// indices (not a loop) so that the list stays in registers as plain values:
// a select between two neighbouring array loads inside a loop would become
// one load at a selected index, i.e. a gather over the whole list.
template <int N, int... I>
__device__ __forceinline__ void shift_up(uint32_t (&a)[N], bool take, std::integer_sequence<int, I...>) {
  ((a[I] = take ? a[I + 1] : a[I]), ...);
}

// Top-K of one token on one wave.  Lane l holds experts l, l+64, ... (kJ of
// them).  Each lane first sorts its own entries by (logit desc, expert index
// asc), as a 64-bit key (order_key(logit), kJ-1-j).  Then K rounds, each of
// which takes the largest remaining entry of the wave (ties to the lower
// expert index) from the head of its lane's list.  The shared-gate logit is
// column E of the slices.
//
// topk_issue issues every load of a token (all slices of the lane's kJ
// logits and of the gate column; indices clamped to valid memory) without
// using them, so a wave can fetch its next token while it selects this one.
template <int kJ>
struct TopkIn {
  float raw[kRouterMaxParts][kJ];
  float zg[kRouterMaxParts];
};
template <int kJ>
__device__ __forceinline__ void topk_issue(const float* __restrict__ part, int n_part, int T, int E, int t, int lane,
                                           TopkIn<kJ>& in) {
  const size_t pstride = static_cast<size_t>(T) * (E + 1);
  const float* z = part + static_cast<size_t>(t) * (E + 1);
#pragma unroll
  for (int p = 0; p < kRouterMaxParts; ++p) {
    const float* zp = z + min(p, n_part - 1) * pstride;
#pragma unroll
    for (int j = 0; j < kJ; ++j) in.raw[p][j] = zp[min(lane + 64 * j, E)];
    in.zg[p] = zp[E];
  }
}

// A lane's entries after the sort, by (logit desc, expert index asc): the
// keys, and the matching fields kJ-1-j packed 4 bits each (list positions
// 0..7 in lo, 8..15 in lo_hi8), so that a pop is one shift; head is the
// expert index of the lane's first entry.
template <int kJ>
struct TopkList {
  uint32_t hi[kJ];
  uint32_t lo, lo_hi8;
  int head;
};

// z = slice 0 + slice 1 + ... (in order) + bias, written to logits when
// non-null; returns the gate logit in zg and the lane's sorted list.
template <int kJ>
__device__ __forceinline__ TopkList<kJ> topk_sorted(TopkIn<kJ>& in, const float (&bj)[kJ], bool has_bias, int n_part,
                                                    int E, int t, int lane, float* __restrict__ logits, float& zg) {
  // opaque to the optimiser, so no load is sunk into a branch
#pragma unroll
  for (int p = 0; p < kRouterMaxParts; ++p) {
#pragma unroll
    for (int j = 0; j < kJ; ++j) asm volatile("" : "+v"(in.raw[p][j]));
    asm volatile("" : "+v"(in.zg[p]));
  }
  zg = in.zg[0];
#pragma unroll
  for (int p = 1; p < kRouterMaxParts; ++p) {
    if (p < n_part) {   // uniform
      zg += in.zg[p];
#pragma unroll
      for (int j = 0; j < kJ; ++j) in.raw[0][j] += in.raw[p][j];
    }
  }
  if (has_bias) {
#pragma unroll
    for (int j = 0; j < kJ; ++j) in.raw[0][j] += bj[j];
  }
  if (logits != nullptr) {
    float* lo_out = logits + static_cast<size_t>(t) * (E + 1);
#pragma unroll
    for (int j = 0; j < kJ; ++j)
      if (lane + 64 * j < E) lo_out[lane + 64 * j] = in.raw[0][j];
    if (lane == 0) lo_out[E] = zg;
  }
  // sorted as plain local arrays (a member array of the result, captured by
  // the compare-and-swap, would be lowered to branches and moves)
  uint32_t hi[kJ], lo[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    hi[j] = (lane + 64 * j < E) ? order_key(in.raw[0][j]) : 0u;
    lo[j] = kJ - 1 - j;
  }
  oddeven_merge_sort<kJ>([&](int a, int b) {
    const bool swap = hi[b] > hi[a] || (hi[b] == hi[a] && lo[b] > lo[a]);
    const uint32_t ha = hi[a], la = lo[a];
    hi[a] = swap ? hi[b] : ha;
    lo[a] = swap ? lo[b] : la;
    hi[b] = swap ? ha : hi[b];
    lo[b] = swap ? la : lo[b];
  });
  TopkList<kJ> L;
#pragma unroll
  for (int j = 0; j < kJ; ++j) L.hi[j] = hi[j];
  L.lo = 0;
#pragma unroll
  for (int i = 0; i < kJ && i < 8; ++i) L.lo |= lo[i] << (4 * i);
  L.lo_hi8 = 0;
#pragma unroll
  for (int i = 8; i < kJ; ++i) L.lo_hi8 |= lo[i] << (4 * (i - 8));
  L.head = (kJ - 1 - static_cast<int>(L.lo & 0xFu)) * 64 + lane;
  return L;
}

// One round: the wave maximum of the lanes' head keys picks the logit key m;
// among the lanes whose head holds it (one, unless logits tie across lanes)
// the lowest expert index wins, and the winning lane pops its head.  Returns
// the winner's expert index (uniform).  Some lane must still hold an entry.
template <int kJ>
__device__ __forceinline__ int topk_round(TopkList<kJ>& L, int lane, uint32_t& m) {
  m = wave_max_u32_s(L.hi[0]);
  const unsigned long long cand = __ballot(L.hi[0] == m);
  int wl = __ffsll(cand) - 1;
  if (__builtin_expect(__popcll(cand) != 1, 0)) {
    const uint32_t idx = (L.hi[0] == m) ? static_cast<uint32_t>(L.head) : 0xFFFFFFFFu;
    wl = static_cast<int>(wave_min_u32_s(idx) & 63u);
  }
  const int e = __builtin_amdgcn_readlane(L.head, wl);
  // the winning lane drops its head: its list moves up one position
  const bool pop = lane == wl;
  shift_up(L.hi, pop, std::make_integer_sequence<int, kJ - 1>{});
  L.hi[kJ - 1] = pop ? 0u : L.hi[kJ - 1];
  if constexpr (kJ > 8) {
    L.lo = pop ? (L.lo >> 4) | (L.lo_hi8 << 28) : L.lo;
    L.lo_hi8 = pop ? L.lo_hi8 >> 4 : L.lo_hi8;
  } else {
    L.lo = pop ? L.lo >> 4 : L.lo;
  }
  L.head = (kJ - 1 - static_cast<int>(L.lo & 0xFu)) * 64 + lane;
  return e;
}

// The selection: K rounds (K <= E), softmax weights of the selected set,
// sigmoid gate.  Writes idx/w when topk_idx is non-null, the token's K
// indices in rank order to sidx[0..K) when sidx is non-null, gamma when
// non-null, logits when non-null.  With rounds < K (uniform) only the first
// `rounds` ranks are selected, into sidx[0..rounds) (the same experts those
// ranks get from the whole selection), and nothing else is written.
template <int kJ>
__device__ __forceinline__ void topk_finish(TopkIn<kJ>& in, const float (&bj)[kJ], bool has_bias, int n_part, int E,
                                            int K, int t, int lane, int32_t* __restrict__ topk_idx,
                                            float* __restrict__ topk_w, float* __restrict__ gamma,
                                            float* __restrict__ logits, int32_t* sidx, int rounds) {
  float zg;
  TopkList<kJ> L = topk_sorted(in, bj, has_bias, n_part, E, t, lane, logits, zg);
  uint32_t my_key = 0, key0 = 0;
  int my_i = 0;
  for (int k = 0; k < rounds; ++k) {
    uint32_t m;
    const int e = topk_round(L, lane, m);
    if (k == 0) key0 = m;
    if (lane == k) {
      my_key = m;
      my_i = e;
    }
  }
  if (sidx != nullptr && lane < rounds) sidx[lane] = my_i;
  if (rounds < K) return;
  const float ex = (lane < K) ? expf(key_value(my_key) - key_value(key0)) : 0.0f;
  const float s = wave_sum(ex);
  if (lane < K && topk_idx != nullptr) {
    topk_idx[static_cast<size_t>(t) * K + lane] = my_i;
    topk_w[static_cast<size_t>(t) * K + lane] = ex / s;
  }
  if (lane == 0 && gamma != nullptr) gamma[t] = 1.0f / (1.0f + expf(-zg));
}

template <int kJ>
__device__ __forceinline__ void load_bias(const float* __restrict__ bias, int E, int lane, float (&bj)[kJ]) {
#pragma unroll
  for (int j = 0; j < kJ; ++j) bj[j] = bias != nullptr ? bias[min(lane + 64 * j, E - 1)] : 0.0f;
}

}  // namespace moe
