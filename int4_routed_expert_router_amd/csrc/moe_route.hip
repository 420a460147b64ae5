// Router GEMV, top-K selection, token-to-expert bucketing.
//
// Routing step of the block (the how-it-works list of the page "Show HN: Run
// an 80B Qwen in 4.3 GB of RAM on a Mac and a 35B on an iPhone": every token
// goes to 10 of 512 or 8 of 256 experts).  Selection order is (logit desc,
// expert index asc); weights are the softmax restricted to the selected set,
// which equals a softmax over all experts followed by renormalisation.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

// z[t][row] = sum_h x[t][h] * Wr[row][h] (+ bias[row] for row < E).
// One wave per router row; each lane owns 8 consecutive columns per 512-column
// stride, so every 16-byte load of the wave is one coalesced 1 KiB run.  Lane
// partials are sequential fp32 FMAs of exact products (16-bit x times fp16 w),
// then a fixed butterfly: the summation tree has depth 8*ceil(H/512) + 6.
template <int ACT>
__global__ __launch_bounds__(64) void k_router_logits(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ wr,
                                                      const float* __restrict__ bias,
                                                      float* __restrict__ logits, int T, int H, int E,
                                                      int tok_per_block) {
  const int lane = threadIdx.x;
  const int row = blockIdx.x;
  const int t0 = blockIdx.y * tok_per_block;
  const int t1 = min(T, t0 + tok_per_block);
  const int nit = (H + 511) / 512;
  uint4 wv[kMaxH / 512];
#pragma unroll
  for (int it = 0; it < kMaxH / 512; ++it) {
    const int col = it * 512 + lane * 8;
    wv[it] = (it < nit && col < H) ? *reinterpret_cast<const uint4*>(wr + static_cast<size_t>(row) * H + col)
                                   : make_uint4(0, 0, 0, 0);
  }
  const float b = (row < E && bias != nullptr) ? bias[row] : 0.0f;
  for (int t = t0; t < t1; ++t) {
    const uint16_t* xr = x + static_cast<size_t>(t) * H;
    float acc = 0.0f;
#pragma unroll
    for (int it = 0; it < kMaxH / 512; ++it) {
      const int col = it * 512 + lane * 8;
      if (it < nit && col < H) {
        const uint4 xv = *reinterpret_cast<const uint4*>(xr + col);
        const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
        const uint32_t ws[4] = {wv[it].x, wv[it].y, wv[it].z, wv[it].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc = fmaf(act_to_f32<ACT>(xs[i] & 0xFFFFu), f16_bits_to_f32(ws[i] & 0xFFFFu), acc);
          acc = fmaf(act_to_f32<ACT>(xs[i] >> 16), f16_bits_to_f32(ws[i] >> 16), acc);
        }
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) logits[static_cast<size_t>(t) * (E + 1) + row] = (row < E) ? acc + b : acc;
  }
}

// One wave per token: K rounds of a wave-wide arg-max over E/64 values per
// lane (lane l holds experts l, l+64, ...).  Each round takes the wave maximum
// of the lanes' best remaining logits, then the lowest expert index among the
// lanes holding that maximum, so ties resolve to the lower expert index.  Both
// reductions run on DPP/row-swap permutes (no LDS round trips).
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int K,
                                              int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                              float* __restrict__ gamma) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* z = logits + static_cast<size_t>(t) * (E + 1);
  constexpr int kJ = kMaxExperts / 64;
  float v[kJ];
  uint32_t avail = 0;
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      // NaN orders as -inf, so a selection always exists (indices stay in [0, E))
      const float zv = z[e];
      v[j] = zv == zv ? zv : -INFINITY;
      avail |= 1u << j;
    } else {
      v[j] = 0.0f;
    }
  }
  float my_v = 0.0f, v0 = 0.0f;
  int my_i = 0;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int bj = -1;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      // j ascending = index ascending, so a strict '>' keeps the lower index on ties
      if (((avail >> j) & 1u) && (bj < 0 || v[j] > bv)) {
        bv = v[j];
        bj = j;
      }
    }
    const float m = wave_max(bv);
    const uint32_t key = (bj >= 0 && bv == m) ? static_cast<uint32_t>(lane + 64 * bj) : 0xFFFFFFFFu;
    const int e = static_cast<int>(wave_min_u32(key));
    if (k == 0) v0 = m;
    if (lane == k) {
      my_v = m;
      my_i = e;
    }
    if ((e & 63) == lane) avail &= ~(1u << (e >> 6));
  }
  const float ex = (lane < K) ? expf(my_v - v0) : 0.0f;
  const float s = wave_sum(ex);
  if (lane < K) {
    topk_idx[static_cast<size_t>(t) * K + lane] = my_i;
    topk_w[static_cast<size_t>(t) * K + lane] = ex / s;
  }
  if (lane == 0 && gamma != nullptr) gamma[t] = 1.0f / (1.0f + expf(-z[E]));
}

// Inclusive scan over a 1024-thread block (wave shuffles + one LDS pass).
__device__ __forceinline__ int block_incl_scan_1024(int v, int* lds16, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  if (lane == 63) lds16[wave] = v;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    const int s = lds16[w];
    if (w < wave) base += s;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return v + base;
}

// Stable counting sort of the n = T*K routed rows by expert, one 1024-thread
// workgroup: histogram (LDS integer atomics), exclusive prefix sum over the
// experts, then a scatter.  The rank of a row among earlier rows of the same
// expert is: rows of earlier 1024-row chunks (a running count), plus rows of
// earlier waves of this chunk (per-wave counts in LDS), plus earlier lanes of
// its own wave (ballot of the lanes holding the same expert).  Rows of one
// expert therefore keep their (t, k) order.  With a unit plan it also writes
// the unit records of the grouped family (see UnitPlan): the unit of a row is
// ubase[e] + rank / 16, where ubase is a prefix sum of ceil(count / 16).
__global__ __launch_bounds__(1024) void k_permute(const int32_t* __restrict__ topk_idx, int n, int E,
                                                  int32_t* __restrict__ expert_off, int32_t* __restrict__ perm,
                                                  int32_t* __restrict__ inv, UnitPlan plan) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int start[kMaxExperts];
  __shared__ int run[kMaxExperts];
  __shared__ int ubase[kMaxExperts];
  __shared__ unsigned short wcnt[16][kMaxExperts];
  __shared__ int scan_tmp[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  if (tid < E) {
    cnt[tid] = 0;
    run[tid] = 0;
  }
  __syncthreads();
  // rows whose expert index lies outside [0, E) are dropped: not counted,
  // not placed (inv = -1), so they contribute nothing
  for (int i = tid; i < n; i += 1024) {
    const int e = topk_idx[i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  const int c = (tid < E) ? cnt[tid] : 0;
  int total = 0;
  const int incl = block_incl_scan_1024(c, scan_tmp, total);
  if (tid < E) {
    start[tid] = incl - c;
    expert_off[tid] = incl - c;
  }
  if (tid == 0) expert_off[E] = total;
  const int n_su = (plan.units != nullptr && plan.shared) ? (plan.T + kSubTokens - 1) / kSubTokens : 0;
  int n_ru = 0;
  if (plan.units != nullptr) {
    const int nu = (c + kSubTokens - 1) / kSubTokens;
    const int uincl = block_incl_scan_1024(nu, scan_tmp, n_ru);
    if (tid < E) ubase[tid] = n_su + uincl - nu;
    if (tid == 0) {
      plan.n_units[0] = n_su;
      plan.n_units[1] = n_ru;
    }
    // the shared expert's units: every token, in order
    for (int u = tid; u < n_su; u += 1024) {
      int32_t* rec = plan.units + static_cast<size_t>(u) * kUnitInts;
      const int mc = min(kSubTokens, plan.T - kSubTokens * u);
      *reinterpret_cast<int4*>(rec) = make_int4(n + kSubTokens * u, mc, -1, 0);
      for (int m = 0; m < mc; ++m) rec[4 + m] = kSubTokens * u + m;
    }
  }
  for (int base = 0; base < n; base += 1024) {
    const int i = base + tid;
    const int ei = i < n ? topk_idx[i] : -1;
    const bool valid = ei >= 0 && ei < E;
    const int e = valid ? ei : -1;
    if (i < n && !valid && inv != nullptr) inv[i] = -1;
    unsigned long long peers = 0;
    unsigned long long todo = __ballot(valid);
    while (todo) {
      const int leader = __ffsll(static_cast<long long>(todo)) - 1;
      const int le = __builtin_amdgcn_readlane(e, leader);
      const unsigned long long m = __ballot(valid && e == le);
      if (valid && e == le) peers = m;
      todo &= ~m;
    }
    const int rank = __popcll(peers & ((1ull << lane) - 1ull));
    const bool first_peer = valid && rank == 0;
    for (int k = tid; k < 16 * E; k += 1024) wcnt[k / E][k % E] = 0;
    __syncthreads();
    if (first_peer) wcnt[wave][e] = static_cast<unsigned short>(__popcll(peers));
    __syncthreads();
    if (valid) {
      int before = 0;
      for (int w = 0; w < wave; ++w) before += wcnt[w][e];
      const int r = run[e] + before + rank;   // rank among all rows of expert e
      const int pos = start[e] + r;
      perm[pos] = i;
      if (inv != nullptr) inv[i] = pos;
      if (plan.units != nullptr) {
        int32_t* rec = plan.units + static_cast<size_t>(ubase[e] + r / kSubTokens) * kUnitInts;
        rec[4 + r % kSubTokens] = i / plan.K;
        if (r % kSubTokens == 0) *reinterpret_cast<int4*>(rec) = make_int4(pos, min(kSubTokens, cnt[e] - r), e, 0);
      }
    }
    __syncthreads();
    if (first_peer) atomicAdd(&run[e], __popcll(peers));
    __syncthreads();
  }
}

// Router logits on the matrix cores for batches of 16+ tokens.  One workgroup
// = 16 router rows x 16 tokens; its waves split H into 32-column steps and
// their fp32 partial tiles are summed in a fixed order.  The fp16 router
// weights enter bf16 MFMAs as an exact hi + lo pair (fp16 has 11 significant
// bits); with fp16 activations they enter as they are.
template <int ACT>
__global__ __launch_bounds__(1024) void k_router_mfma(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                                      const float* __restrict__ bias, float* __restrict__ logits,
                                                      int T, int H, int E) {
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  __shared__ float part[16][16][17];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int n = lane & 15, kb = lane >> 4;
  const int row = blockIdx.x * 16 + n;      // router row this lane loads (B operand column)
  const int tok = blockIdx.y * 16 + n;      // token this lane loads (A operand row)
  const int nsteps = H / 32;
  f32x4_t acc = {0, 0, 0, 0};
  for (int st = wave; st < nsteps; st += nw) {
    const int col = 32 * st + 8 * kb;
    const uint4 av = (tok < T) ? *reinterpret_cast<const uint4*>(x + static_cast<size_t>(tok) * H + col)
                               : make_uint4(0, 0, 0, 0);
    const uint4 bv = (row <= E) ? *reinterpret_cast<const uint4*>(wr + static_cast<size_t>(row) * H + col)
                                : make_uint4(0, 0, 0, 0);
    if constexpr (ACT == 2) {
      const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w};
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float f0 = f16_bits_to_f32(bw[i] & 0xFFFFu), f1 = f16_bits_to_f32(bw[i] >> 16);
        const uint32_t h0 = __float_as_uint(f0) & 0xFFFF0000u, h1 = __float_as_uint(f1) & 0xFFFF0000u;
        const uint32_t l0 = f32_to_act<2>(f0 - __uint_as_float(h0)), l1 = f32_to_act<2>(f1 - __uint_as_float(h1));
        hi[i] = (h0 >> 16) | h1;
        lo[i] = l0 | (l1 << 16);
      }
      const uint4 bh = make_uint4(hi[0], hi[1], hi[2], hi[3]), bl = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bh),
                                                    acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bl),
                                                    acc, 0, 0, 0);
    } else {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, av), __builtin_bit_cast(f16x8_t, bv),
                                                   acc, 0, 0, 0);
    }
  }
  // lane holds tokens 4kb..4kb+3 (tile rows) of router row n (tile column)
#pragma unroll
  for (int i = 0; i < 4; ++i) part[wave][4 * kb + i][n] = acc[i];
  __syncthreads();
  if (threadIdx.x < 256) {
    const int m = threadIdx.x >> 4, c = threadIdx.x & 15;
    const int t = blockIdx.y * 16 + m, r = blockIdx.x * 16 + c;
    float sum = 0.0f;
    for (int w = 0; w < nw; ++w) sum += part[w][m][c];
    if (t < T && r <= E) {
      if (r < E && bias != nullptr) sum += bias[r];
      logits[static_cast<size_t>(t) * (E + 1) + r] = sum;
    }
  }
}

template <int ACT>
static hipError_t launch_router_t(const uint16_t* x, const uint16_t* wr, const float* bias, float* logits, int T,
                                  int H, int E, hipStream_t s) {
  if (T >= kRouterMfmaMinTokens) {
    const int steps = H / 32;
    const int nw = steps < 16 ? steps : 16;
    dim3 grid((E + 1 + 15) / 16, (T + 15) / 16);
    hipLaunchKernelGGL(k_router_mfma<ACT>, grid, dim3(64 * nw), 0, s, x, wr, bias, logits, T, H, E);
  } else {
    const int tpb = (T <= 8) ? T : 8;
    dim3 grid(E + 1, (T + tpb - 1) / tpb);
    hipLaunchKernelGGL(k_router_logits<ACT>, grid, dim3(64), 0, s, x, wr, bias, logits, T, H, E, tpb);
  }
  return hipGetLastError();
}

hipError_t launch_router_logits(int act, const uint16_t* x, const uint16_t* wr, const float* bias, float* logits,
                                int T, int H, int E, hipStream_t s) {
  return act == 2 ? launch_router_t<2>(x, wr, bias, logits, T, H, E, s)
                  : launch_router_t<1>(x, wr, bias, logits, T, H, E, s);
}

hipError_t launch_topk(const float* logits, int T, int E, int K, int32_t* idx, float* w, float* gamma,
                       hipStream_t s) {
  hipLaunchKernelGGL(k_topk, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, K, idx, w, gamma);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int n, int E, int32_t* off, int32_t* perm, int32_t* inv,
                          const UnitPlan* plan, hipStream_t s) {
  UnitPlan p{};
  if (plan != nullptr) p = *plan;
  hipLaunchKernelGGL(k_permute, dim3(1), dim3(1024), 0, s, idx, n, E, off, perm, inv, p);
  return hipGetLastError();
}

}  // namespace moe
