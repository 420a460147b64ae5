// Router GEMV, top-K selection, token-to-expert bucketing.
//
// Routing step of the block (the how-it-works list of the page "Show HN: Run
// an 80B Qwen in 4.3 GB of RAM on a Mac and a 35B on an iPhone": every token
// goes to 10 of 512 or 8 of 256 experts).  Selection order is (logit desc,
// expert index asc); weights are the softmax restricted to the selected set,
// which equals a softmax over all experts followed by renormalisation.
#include "moe_common.h"
#include "moe_kernels.h"
#include "moe_topk.h"

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

// Router of a layer after the first in a decode-sized stack, with the
// previous layer's combine and residual folded in:
//   y_t  = sum_k w[t,k] yrow[tK+k] + gamma[t] yrow[TK+t]   (rank order, shared last)
//   r'_t = r_src_t + y_t,   x_t = rne(r'_t / sqrt(mean(r'_t^2) + 1e-6))
//   z[t][row] = sum_h x[t][h] Wr[row][h] (+ bias[row] for row < E)
// Four router rows per 256-thread workgroup (one per wave).  Every workgroup
// forms y, r' and x of every token itself, with the same code in the same
// order, so all of them hold the same bits; workgroup 0 stores r' (r_dst,
// a different buffer from r_src), x (x_out) and y (y_out, when non-null).
// The router rows' loads are issued first (they do not depend on x); the
// dot products follow k_router_logits' order exactly (lane-sequential over
// the lane's columns, then the wave butterfly, then the bias).  Thread u
// owns columns 2048 m + 8 u + i (i < 8) of the combine.  Dynamic LDS: x of
// all tokens, T * H 16-bit values.
template <int ACT>
__global__ __launch_bounds__(256) void k_router_combine(const uint16_t* __restrict__ wr,
                                                        const float* __restrict__ bias, float* __restrict__ logits,
                                                        int T, int H, int E, int K, int has_shared,
                                                        const float* __restrict__ yrow, const float* __restrict__ w,
                                                        const float* __restrict__ gamma,
                                                        const float* __restrict__ r_src, float* __restrict__ r_dst,
                                                        uint16_t* __restrict__ x_out, float* __restrict__ y_out) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];   // [T][H]
  __shared__ float red[4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = 4 * blockIdx.x + wave;
  const bool row_ok = row <= E;
  const int nit = (H + 511) / 512;
  uint4 wv[kMaxH / 512];
#pragma unroll
  for (int it = 0; it < kMaxH / 512; ++it) {
    const int col = it * 512 + lane * 8;
    wv[it] = (row_ok && it < nit && col < H)
                 ? *reinterpret_cast<const uint4*>(wr + static_cast<size_t>(row) * H + col)
                 : make_uint4(0, 0, 0, 0);
  }
  const float b = (row < E && bias != nullptr) ? bias[row] : 0.0f;
  const int ns = K + has_shared;
  constexpr int kCh = kMaxH / 2048;   // 8-column chunks per thread
  for (int t = 0; t < T; ++t) {
    float ss = 0.0f;
    float rv[kCh][8];
#pragma unroll
    for (int m = 0; m < kCh; ++m) {
      const int c = 2048 * m + 8 * tid;
      if (c < H) {
        // every source row's loads of the chunk are issued before the sums
        constexpr int kB = 12;
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int k0 = 0; k0 < ns; k0 += kB) {
          float4 v[kB][2];
#pragma unroll
          for (int q = 0; q < kB; ++q) {
            const int k = min(k0 + q, ns - 1);
            const float* src = yrow + static_cast<size_t>(k < K ? t * K + k : T * K + t) * H + c;
            v[q][0] = *reinterpret_cast<const float4*>(src);
            v[q][1] = *reinterpret_cast<const float4*>(src + 4);
          }
#pragma unroll
          for (int q = 0; q < kB; ++q) {
            if (k0 + q < ns) {   // uniform
              const int k = k0 + q;
              const float wk = k < K ? w[t * K + k] : gamma[t];
              acc[0] = fmaf(wk, v[q][0].x, acc[0]);
              acc[1] = fmaf(wk, v[q][0].y, acc[1]);
              acc[2] = fmaf(wk, v[q][0].z, acc[2]);
              acc[3] = fmaf(wk, v[q][0].w, acc[3]);
              acc[4] = fmaf(wk, v[q][1].x, acc[4]);
              acc[5] = fmaf(wk, v[q][1].y, acc[5]);
              acc[6] = fmaf(wk, v[q][1].z, acc[6]);
              acc[7] = fmaf(wk, v[q][1].w, acc[7]);
            }
          }
        }
        const float4 r0 = *reinterpret_cast<const float4*>(r_src + static_cast<size_t>(t) * H + c);
        const float4 r1 = *reinterpret_cast<const float4*>(r_src + static_cast<size_t>(t) * H + c + 4);
        const float rin[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          rv[m][i] = rin[i] + acc[i];
          ss = fmaf(rv[m][i], rv[m][i], ss);
        }
        if (blockIdx.x == 0) {
          float* rd = r_dst + static_cast<size_t>(t) * H + c;
          *reinterpret_cast<float4*>(rd) = make_float4(rv[m][0], rv[m][1], rv[m][2], rv[m][3]);
          *reinterpret_cast<float4*>(rd + 4) = make_float4(rv[m][4], rv[m][5], rv[m][6], rv[m][7]);
          if (y_out != nullptr) {
            float* yd = y_out + static_cast<size_t>(t) * H + c;
            *reinterpret_cast<float4*>(yd) = make_float4(acc[0], acc[1], acc[2], acc[3]);
            *reinterpret_cast<float4*>(yd + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
          }
        }
      }
    }
    // block sum of the squares: the wave butterfly, then the 4 waves in order
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    const float tot = ((red[0] + red[1]) + red[2]) + red[3];
    __syncthreads();
    const float inv_rms = 1.0f / sqrtf(tot / static_cast<float>(H) + 1e-6f);
#pragma unroll
    for (int m = 0; m < kCh; ++m) {
      const int c = 2048 * m + 8 * tid;
      if (c < H) {
        uint4 xv;
        xv.x = f32_to_act<ACT>(rv[m][0] * inv_rms) | (static_cast<uint32_t>(f32_to_act<ACT>(rv[m][1] * inv_rms)) << 16);
        xv.y = f32_to_act<ACT>(rv[m][2] * inv_rms) | (static_cast<uint32_t>(f32_to_act<ACT>(rv[m][3] * inv_rms)) << 16);
        xv.z = f32_to_act<ACT>(rv[m][4] * inv_rms) | (static_cast<uint32_t>(f32_to_act<ACT>(rv[m][5] * inv_rms)) << 16);
        xv.w = f32_to_act<ACT>(rv[m][6] * inv_rms) | (static_cast<uint32_t>(f32_to_act<ACT>(rv[m][7] * inv_rms)) << 16);
        *reinterpret_cast<uint4*>(xs + static_cast<size_t>(t) * H + c) = xv;
        if (blockIdx.x == 0) *reinterpret_cast<uint4*>(x_out + static_cast<size_t>(t) * H + c) = xv;
      }
    }
  }
  __syncthreads();
  if (!row_ok) return;
  for (int t = 0; t < T; ++t) {
    float acc = 0.0f;
#pragma unroll
    for (int it = 0; it < kMaxH / 512; ++it) {
      const int col = it * 512 + lane * 8;
      if (it < nit && col < H) {
        const uint4 xv = *reinterpret_cast<const uint4*>(xs + static_cast<size_t>(t) * H + col);
        const uint32_t xq[4] = {xv.x, xv.y, xv.z, xv.w};
        const uint32_t wq[4] = {wv[it].x, wv[it].y, wv[it].z, wv[it].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc = fmaf(act_to_f32<ACT>(xq[i] & 0xFFFFu), f16_bits_to_f32(wq[i] & 0xFFFFu), acc);
          acc = fmaf(act_to_f32<ACT>(xq[i] >> 16), f16_bits_to_f32(wq[i] >> 16), acc);
        }
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) logits[static_cast<size_t>(t) * (E + 1) + row] = (row < E) ? acc + b : acc;
  }
}

hipError_t launch_router_combine(int act, const uint16_t* wr, const float* bias, float* logits, int T, int H, int E,
                                 int K, bool has_shared, const float* yrow, const float* w, const float* gamma,
                                 const float* r_src, float* r_dst, uint16_t* x_out, float* y_out, hipStream_t s,
                                 RouterParts* out) {
  if (!router_combine_fits(T, H)) return hipErrorInvalidValue;
  const dim3 grid((E + 1 + 3) / 4), block(256);
  const size_t lds = static_cast<size_t>(T) * H * 2;
  const int hs = has_shared ? 1 : 0;
  if (act == 2)
    hipLaunchKernelGGL(k_router_combine<2>, grid, block, lds, s, wr, bias, logits, T, H, E, K, hs, yrow, w, gamma,
                       r_src, r_dst, x_out, y_out);
  else
    hipLaunchKernelGGL(k_router_combine<1>, grid, block, lds, s, wr, bias, logits, T, H, E, K, hs, yrow, w, gamma,
                       r_src, r_dst, x_out, y_out);
  out->n_part = 1;
  out->biased = true;
  return hipGetLastError();
}

// One token per 64-lane workgroup: spreads the loads over the compute units.
template <int kJ>
__global__ __launch_bounds__(64) void k_topk(const float* __restrict__ part, int n_part,
                                              const float* __restrict__ bias, int T, int E, int K,
                                              int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                              float* __restrict__ gamma, float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x;
  if (t >= T) return;
  TopkIn<kJ> in;
  topk_issue(part, n_part, T, E, t, lane, in);
  float bj[kJ];
  load_bias(bias, E, lane, bj);
  topk_finish(in, bj, bias != nullptr, n_part, E, K, t, lane, topk_idx, topk_w, gamma, logits, nullptr, K);
}

// Inclusive prefix sums of two values at once over a 1024-thread block.
// Within a wave: a Hillis-Steele scan inside each row of 16 lanes on DPP
// row shifts (lanes without a source add 0), then each row adds the totals
// of the rows before it (read from lanes 15, 31, 47).  Across the 16 waves:
// one LDS pass over the wave totals.  Integer sums, so the order is moot.
__device__ __forceinline__ int dpp_row_shr_or0(int v, int shift_ctrl) {
  switch (shift_ctrl) {   // the control must be a literal
    case 1: return __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);
    case 2: return __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);
    case 4: return __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);
    default: return __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);
  }
}
__device__ __forceinline__ int wave_incl_scan(int v) {
#pragma unroll
  for (int sh = 1; sh < 16; sh <<= 1) v += dpp_row_shr_or0(v, sh);
  const int lane = threadIdx.x & 63;
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
            r2 = __builtin_amdgcn_readlane(v, 47);
  return v + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
}
__device__ __forceinline__ void block_incl_scan2_1024(int& a, int& b, int2* lds16, int& total_a, int& total_b) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  a = wave_incl_scan(a);
  b = wave_incl_scan(b);
  if (lane == 63) lds16[wave] = make_int2(a, b);
  __syncthreads();
  int base_a = 0, base_b = 0, tot_a = 0, tot_b = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int2 s = lds16[w];
    if (w < wave) {
      base_a += s.x;
      base_b += s.y;
    }
    tot_a += s.x;
    tot_b += s.y;
  }
  a += base_a;
  b += base_b;
  total_a = tot_a;
  total_b = tot_b;
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
  __shared__ __attribute__((aligned(16))) unsigned short wcnt[kMaxExperts][16];   // rows of expert e in wave w of a chunk
  __shared__ int2 scan_tmp[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid < E) {
    cnt[tid] = 0;
    run[tid] = 0;
  }
  if (tid == 0 && plan.status_reset != nullptr) *plan.status_reset = 0u;
  __syncthreads();
  // rows whose expert index lies outside [0, E) are dropped: not counted,
  // not placed (inv = -1), so they contribute nothing
  // the first chunk's indices stay in a register for the scatter below
  const int first_e = tid < n ? topk_idx[tid] : -1;
  if (first_e >= 0 && first_e < E) atomicAdd(&cnt[first_e], 1);
  for (int i = tid + 1024; i < n; i += 1024) {
    const int e = topk_idx[i];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  const int c = (tid < E) ? cnt[tid] : 0;
  const int nu = (c + kSubTokens - 1) / kSubTokens;   // units of expert tid
  int incl = c, uincl = nu, total = 0, n_ru = 0;
  block_incl_scan2_1024(incl, uincl, scan_tmp, total, n_ru);
  if (tid < E) {
    start[tid] = incl - c;
    expert_off[tid] = incl - c;
  }
  if (tid == 0) expert_off[E] = total;
  const int n_su = (plan.units != nullptr && plan.shared) ? (plan.T + kSubTokens - 1) / kSubTokens : 0;
  if (plan.units != nullptr) {
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
    const int ei = base == 0 ? first_e : (i < n ? topk_idx[i] : -1);
    const bool valid = ei >= 0 && ei < E;
    const int e = valid ? ei : 0;
    if (i < n && !valid && inv != nullptr) inv[i] = -1;
    // lanes of this wave holding the same expert: intersect, bit by bit of
    // the expert index, the ballots of lanes that agree with this lane
    unsigned long long peers = __ballot(valid);
    for (int b = 0; (1 << b) < E; ++b) {
      const bool bit = (e >> b) & 1;
      const unsigned long long on = __ballot(bit);
      peers &= bit ? on : ~on;
    }
    const int rank = __popcll(peers & ((1ull << lane) - 1ull));
    const bool first_peer = valid && rank == 0;
    for (int k = tid; k < 8 * E; k += 1024) reinterpret_cast<uint32_t*>(&wcnt[0][0])[k] = 0u;
    __syncthreads();
    if (first_peer) wcnt[e][wave] = static_cast<unsigned short>(__popcll(peers));
    __syncthreads();
    if (valid) {
      // rows of expert e in the waves before this one: the 16 counts of the
      // expert are read as two 16-byte words and the first `wave` added
      const uint4 c_lo = *reinterpret_cast<const uint4*>(&wcnt[e][0]);
      const uint4 c_hi = *reinterpret_cast<const uint4*>(&wcnt[e][8]);
      const uint32_t cw[8] = {c_lo.x, c_lo.y, c_lo.z, c_lo.w, c_hi.x, c_hi.y, c_hi.z, c_hi.w};
      int before = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        before += 2 * q < wave ? static_cast<int>(cw[q] & 0xFFFFu) : 0;
        before += 2 * q + 1 < wave ? static_cast<int>(cw[q] >> 16) : 0;
      }
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
// = 16 router rows x 16 tokens x one slice of the hidden dimension
// (blockIdx.z; `steps` 32-column steps per slice); its waves split the slice
// into 32-column steps and their fp32 partial tiles are summed in a fixed
// order.  The slice sums go to part[z] (no bias); top-K adds the slices in
// order and the bias.  Slicing spreads a small batch over all compute units.
// The fp16 router weights enter bf16 MFMAs as an exact hi + lo pair (fp16 has
// 11 significant bits); with fp16 activations they enter as they are.  The
// shared-gate row E is not a matrix-core row (the grid stays a whole number
// of 16-row blocks): the workgroups of row block 0 also form its slice sums
// with exact fp32 products on the vector units and write them to column E.
template <int ACT>
__global__ __launch_bounds__(1024) void k_router_mfma(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                                      float* __restrict__ part, int T, int H, int E, int steps) {
  typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
  typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  __shared__ float wpart[16][16][17];   // per-wave partial tiles
  __shared__ float wgate[16][16];       // per-wave shared-gate partials
  const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, kb = lane >> 4;
  const int row = blockIdx.x * 16 + n;      // router row this lane loads (B operand column)
  const int tok = blockIdx.y * 16 + n;      // token this lane loads (A operand row)
  const int nsteps = steps;
  const int col0 = blockIdx.z * steps * 32;
  float* logits = part + static_cast<size_t>(blockIdx.z) * T * (E + 1);
  // out-of-range lanes load a clamped (valid) row and zero it, so every load
  // is unconditional and a wave's loads for up to kBatch steps go out together
  constexpr int kBatch = kRouterBatch;
  const bool tok_ok = tok < T, row_ok = row < E;   // row E (shared gate) is left to top-k
  const uint16_t* xrow = x + static_cast<size_t>(tok_ok ? tok : T - 1) * H + col0;
  const uint16_t* wrow = wr + static_cast<size_t>(row_ok ? row : E - 1) * H + col0;
  const uint16_t* grow = wr + static_cast<size_t>(E) * H + col0;   // shared-gate row
  const bool do_gate = blockIdx.x == 0;   // uniform
  f32x4_t acc = {0, 0, 0, 0};
  float gacc = 0.0f;
  for (int st0 = wave; st0 < nsteps; st0 += kBatch * nw) {
    uint4 av[kBatch], bv[kBatch], gv[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int col = 32 * min(st0 + u * nw, nsteps - 1) + 8 * kb;
      av[u] = *reinterpret_cast<const uint4*>(xrow + col);
      bv[u] = *reinterpret_cast<const uint4*>(wrow + col);
      if (do_gate) gv[u] = *reinterpret_cast<const uint4*>(grow + col);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (st0 + u * nw >= nsteps) break;   // wave-uniform
      if (!tok_ok) av[u] = make_uint4(0, 0, 0, 0);
      if (!row_ok) bv[u] = make_uint4(0, 0, 0, 0);
      if (do_gate) {
        const uint32_t xs[4] = {av[u].x, av[u].y, av[u].z, av[u].w};
        const uint32_t gs[4] = {gv[u].x, gv[u].y, gv[u].z, gv[u].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          gacc = fmaf(act_to_f32<ACT>(xs[i] & 0xFFFFu), f16_bits_to_f32(gs[i] & 0xFFFFu), gacc);
          gacc = fmaf(act_to_f32<ACT>(xs[i] >> 16), f16_bits_to_f32(gs[i] >> 16), gacc);
        }
      }
      if constexpr (ACT == 2) {
        const uint32_t bw[4] = {bv[u].x, bv[u].y, bv[u].z, bv[u].w};
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
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[u]),
                                                      __builtin_bit_cast(bf16x8_t, bh), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[u]),
                                                      __builtin_bit_cast(bf16x8_t, bl), acc, 0, 0, 0);
      } else {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, av[u]),
                                                     __builtin_bit_cast(f16x8_t, bv[u]), acc, 0, 0, 0);
      }
    }
  }
  // lane holds tokens 4kb..4kb+3 (tile rows) of router row n (tile column)
#pragma unroll
  for (int i = 0; i < 4; ++i) wpart[wave][4 * kb + i][n] = acc[i];
  if (do_gate) {
    // lanes n, n+16, n+32, n+48 hold token n's four column groups
    gacc += __shfl_xor(gacc, 16, kWave);
    gacc += __shfl_xor(gacc, 32, kWave);
    if (kb == 0) wgate[wave][n] = gacc;
  }
  __syncthreads();
  if (do_gate && threadIdx.x < 16) {
    const int t = blockIdx.y * 16 + static_cast<int>(threadIdx.x);
    float sum = 0.0f;
    for (int w = 0; w < nw; ++w) sum += wgate[w][threadIdx.x];
    if (t < T) logits[static_cast<size_t>(t) * (E + 1) + E] = sum;
  }
  // 256 outputs per tile; a block may have as few as 2 waves (H = 64)
  for (int q = threadIdx.x; q < 256; q += blockDim.x) {
    const int m = q >> 4, c = q & 15;
    const int t = blockIdx.y * 16 + m, r = blockIdx.x * 16 + c;
    float sum = 0.0f;
    for (int w = 0; w < nw; ++w) sum += wpart[w][m][c];
    if (t < T && r < E) logits[static_cast<size_t>(t) * (E + 1) + r] = sum;
  }
}

template <int ACT>
static hipError_t launch_router_t(const uint16_t* x, const uint16_t* wr, const float* bias, float* part, int T, int H,
                                  int E, hipStream_t s, RouterParts* out) {
  if (T >= kRouterMfmaMinTokens) {
    // slices: double while the grid stays within one workgroup per compute
    // unit and the slice stays a whole number of 32-column steps
    const int tiles = ((E + 15) / 16) * ((T + 15) / 16);
    int S = 1;
    while (S < kRouterMaxParts && tiles * 2 * S <= kGridTiles && (H / 32) % (2 * S) == 0) S *= 2;
    const int steps = H / 32 / S;
    const int nw = steps < kRouterWaves ? steps : kRouterWaves;
    dim3 grid((E + 15) / 16, (T + 15) / 16, S);
    hipLaunchKernelGGL(k_router_mfma<ACT>, grid, dim3(64 * nw), 0, s, x, wr, part, T, H, E, steps);
    out->n_part = S;
    out->biased = false;
  } else {
    const int tpb = (T <= 8) ? T : 8;
    dim3 grid(E + 1, (T + tpb - 1) / tpb);
    hipLaunchKernelGGL(k_router_logits<ACT>, grid, dim3(64), 0, s, x, wr, bias, part, T, H, E, tpb);
    out->n_part = 1;
    out->biased = true;
  }
  return hipGetLastError();
}

hipError_t launch_router_logits(int act, const uint16_t* x, const uint16_t* wr, const float* bias, float* part,
                                int T, int H, int E, hipStream_t s, RouterParts* out) {
  return act == 2 ? launch_router_t<2>(x, wr, bias, part, T, H, E, s, out)
                  : launch_router_t<1>(x, wr, bias, part, T, H, E, s, out);
}

#define MOE_TOPK_DISPATCH(LAUNCH)                                       \
  do {                                                                  \
    static_assert(kMaxExperts == 1024, "dispatch covers up to 16 logits per lane"); \
    if (E <= 64) LAUNCH(1);                                             \
    else if (E <= 128) LAUNCH(2);                                       \
    else if (E <= 256) LAUNCH(4);                                       \
    else if (E <= 512) LAUNCH(8);                                       \
    else LAUNCH(16);                                                    \
  } while (0)

hipError_t launch_topk(const float* part, int n_part, const float* bias, int T, int E, int K, int32_t* idx, float* w,
                       float* gamma, float* logits, hipStream_t s) {
#define TOPK_LAUNCH(J) \
  hipLaunchKernelGGL((k_topk<J>), dim3(T), dim3(64), 0, s, part, n_part, bias, T, E, K, idx, w, gamma, logits)
  MOE_TOPK_DISPATCH(TOPK_LAUNCH);
#undef TOPK_LAUNCH
  return hipGetLastError();
}

#undef MOE_TOPK_DISPATCH

hipError_t launch_permute(const int32_t* idx, int n, int E, int32_t* off, int32_t* perm, int32_t* inv,
                          const UnitPlan* plan, hipStream_t s) {
  UnitPlan p{};
  if (plan != nullptr) p = *plan;
  hipLaunchKernelGGL(k_permute, dim3(1), dim3(1024), 0, s, idx, n, E, off, perm, inv, p);
  return hipGetLastError();
}

}  // namespace moe
