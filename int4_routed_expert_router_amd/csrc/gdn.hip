// Gated DeltaNet single-token recurrence (see include/moe_gdn.h for the
// formula and its source).  The step is bound by the state's HBM traffic:
// every value head reads and writes its [d_v][128] fp32 state once.
#include <hip/hip_runtime.h>

#include "moe_common.h"
#include "moe_gdn.h"

namespace moe {
// moe_api.cpp owns the thread-local error string; this file reports through it.
moe_status set_error(moe_status code, const char* fmt, ...);

namespace {
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
}  // namespace

constexpr int kDK = 128;
constexpr int kRowsPerPass = 16;   // 256 threads, one row of 16 lanes per state row
constexpr int kPassBatch = 8;      // passes whose state loads a thread issues together

__device__ __forceinline__ float row_sum(float x) { return __uint_as_float(dpp_row_sum(__float_as_uint(x))); }

// One workgroup per (sequence, value head).  A row of 16 lanes owns one state
// row per pass; lane l16 of it holds columns 4 l16 .. 4 l16 + 3 and
// 64 + 4 l16 .. 64 + 4 l16 + 3, so each 16-byte load of a wave reads four
// rows' 256 contiguous bytes.  All state loads of a batch of passes are
// issued before the first is used; q and k of the key head are read by
// every row of lanes, normalised with row sums, and kept in registers.
// S k^ and S q^ are row dot products of the old state; then
// S' = alpha S + d k^T with d = beta (v - alpha S k^), and
// o = S' q^ = alpha (S q^) + d (k^ . q^).
template <int ACT>
__global__ __launch_bounds__(256) void k_gdn_step(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                  const uint16_t* __restrict__ v, const float* __restrict__ g,
                                                  const float* __restrict__ beta, float q_scale,
                                                  float* __restrict__ state, float* __restrict__ o, int Hk, int Hv,
                                                  int dv) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int hk = h / (Hv / Hk);
  const int l16 = threadIdx.x & 15, grp = threadIdx.x >> 4;
  const int c0 = 4 * l16, c1 = 64 + 4 * l16;
  const size_t head = static_cast<size_t>(b) * Hv + h;
  float* S = state + head * static_cast<size_t>(dv) * kDK;
  const uint16_t* vh = v + head * dv;
  const int npass = dv / kRowsPerPass;
  float4 sa[kPassBatch], sb[kPassBatch];
  uint32_t vr[kPassBatch];
  auto issue = [&](int p0) {
#pragma unroll
    for (int i = 0; i < kPassBatch; ++i) {
      if (p0 + i < npass) {   // uniform
        const int row = (p0 + i) * kRowsPerPass + grp;
        sa[i] = *reinterpret_cast<const float4*>(S + row * kDK + c0);
        sb[i] = *reinterpret_cast<const float4*>(S + row * kDK + c1);
        vr[i] = vh[row];
      }
    }
  };
  issue(0);
  const uint16_t* qh = q + (static_cast<size_t>(b) * Hk + hk) * kDK;
  const uint16_t* kh = k + (static_cast<size_t>(b) * Hk + hk) * kDK;
  const uint2 qa = *reinterpret_cast<const uint2*>(qh + c0), qb = *reinterpret_cast<const uint2*>(qh + c1);
  const uint2 ka = *reinterpret_cast<const uint2*>(kh + c0), kb = *reinterpret_cast<const uint2*>(kh + c1);
  const float alpha = expf(g[head]), bt = beta[head];
  const uint32_t qw[4] = {qa.x, qa.y, qb.x, qb.y}, kw[4] = {ka.x, ka.y, kb.x, kb.y};
  float qn[8], kn[8];
  float qq = 0.0f, kk = 0.0f, kq = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    qn[2 * j] = act_to_f32<ACT>(qw[j] & 0xFFFFu);
    qn[2 * j + 1] = act_to_f32<ACT>(qw[j] >> 16);
    kn[2 * j] = act_to_f32<ACT>(kw[j] & 0xFFFFu);
    kn[2 * j + 1] = act_to_f32<ACT>(kw[j] >> 16);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    qq = fmaf(qn[j], qn[j], qq);
    kk = fmaf(kn[j], kn[j], kk);
    kq = fmaf(kn[j], qn[j], kq);
  }
  qq = row_sum(qq);
  kk = row_sum(kk);
  kq = row_sum(kq);
  const float rq = q_scale / sqrtf(qq + 1e-6f), rk = 1.0f / sqrtf(kk + 1e-6f);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    qn[j] *= rq;
    kn[j] *= rk;
  }
  const float kdq = kq * rk * rq;   // k^ . q^
  float* oh = o + head * dv;
  for (int p0 = 0; p0 < npass; p0 += kPassBatch) {
    if (p0 != 0) issue(p0);
#pragma unroll
    for (int i = 0; i < kPassBatch; ++i) {
      if (p0 + i < npass) {   // uniform
        const int row = (p0 + i) * kRowsPerPass + grp;
        const float s[8] = {sa[i].x, sa[i].y, sa[i].z, sa[i].w, sb[i].x, sb[i].y, sb[i].z, sb[i].w};
        float u = 0.0f, w = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          u = fmaf(s[j], kn[j], u);
          w = fmaf(s[j], qn[j], w);
        }
        u = row_sum(u);
        w = row_sum(w);
        const float d = bt * (act_to_f32<ACT>(vr[i]) - alpha * u);
        float ns[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) ns[j] = fmaf(d, kn[j], alpha * s[j]);
        *reinterpret_cast<float4*>(S + row * kDK + c0) = make_float4(ns[0], ns[1], ns[2], ns[3]);
        *reinterpret_cast<float4*>(S + row * kDK + c1) = make_float4(ns[4], ns[5], ns[6], ns[7]);
        if (l16 == 0) oh[row] = fmaf(d, kdq, alpha * w);
      }
    }
  }
}

}  // namespace moe

extern "C" moe_status moe_gdn_step(const moe_gdn_desc* d, const void* q, const void* k, const void* v,
                                   const float* g, const float* beta, float q_scale, float* state, float* o,
                                   moe_stream stream) {
  using moe::aligned;
  using moe::kDK;
  using moe::kRowsPerPass;
  using moe::set_error;
  if (!d) return set_error(MOE_EINVAL, "desc is NULL");
  if (d->batch < 0 || d->batch > 65535) return set_error(MOE_ESHAPE, "batch=%d must be in [0, 65535]", d->batch);
  if (d->head_k_dim != kDK) return set_error(MOE_ESHAPE, "head_k_dim=%d must be %d", d->head_k_dim, kDK);
  if (d->head_v_dim < 16 || d->head_v_dim > 256 || d->head_v_dim % kRowsPerPass)
    return set_error(MOE_ESHAPE, "head_v_dim=%d must be a multiple of 16 in [16, 256]", d->head_v_dim);
  if (d->k_heads < 1 || d->v_heads < d->k_heads || d->v_heads > 1024 || d->v_heads % d->k_heads)
    return set_error(MOE_ESHAPE, "v_heads=%d must be a multiple of k_heads=%d, at most 1024", d->v_heads, d->k_heads);
  if (d->act_dtype != MOE_F16 && d->act_dtype != MOE_BF16)
    return set_error(MOE_EINVAL, "act_dtype=%d is not MOE_F16/MOE_BF16", d->act_dtype);
  if (d->batch == 0) return set_error(MOE_OK, "");
  if (!q || !k || !v || !g || !beta || !state || !o) return set_error(MOE_EINVAL, "NULL buffer");
  if (!aligned(q, 8) || !aligned(k, 8) || !aligned(v, 2) || !aligned(state, 16))
    return set_error(MOE_EINVAL, "q and k must be 8-byte, v 2-byte and state 16-byte aligned");
  const dim3 grid(d->v_heads, d->batch);
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const auto* qb = static_cast<const uint16_t*>(q);
  const auto* kb = static_cast<const uint16_t*>(k);
  const auto* vb = static_cast<const uint16_t*>(v);
  if (d->act_dtype == MOE_BF16)
    hipLaunchKernelGGL(moe::k_gdn_step<2>, grid, dim3(256), 0, s, qb, kb, vb, g, beta, q_scale, state, o, d->k_heads,
                       d->v_heads, d->head_v_dim);
  else
    hipLaunchKernelGGL(moe::k_gdn_step<1>, grid, dim3(256), 0, s, qb, kb, vb, g, beta, q_scale, state, o, d->k_heads,
                       d->v_heads, d->head_v_dim);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(MOE_EHIP, "Gated DeltaNet kernel launch: %s", hipGetErrorString(e));
  return set_error(MOE_OK, "");
}
