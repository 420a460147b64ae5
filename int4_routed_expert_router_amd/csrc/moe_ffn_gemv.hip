// Per-row int4 / int8 expert GEMVs (decode-sized batches) and the combine.
//
// The pages run a cooperative GEMV fast path over MLX-style affine int4/int8
// group-quantised weights (what-was-built list of the page "Show HN: Run an
// 80B Qwen in 4.3 GB of RAM on a Mac and a 35B on an iPhone").  Here a
// 64-lane wavefront reads one 1 KiB block of packed values per 16-byte load
// (int4: one block per 64-column chunk; int8: two, one per tile of the
// pair-tile), so every weight byte moves in fully coalesced 128-bit loads,
// and the activations are staged once per workgroup in LDS.
//
// Affine group identity used by every kernel: for a group of G input columns
// with scale s and bias b,  sum_c (s q_c + b) x_c = s sum_c q_c x_c + b sum_c x_c,
// so the per-column work is an integer-weight dot product and the bias costs
// one FMA per (row, group) with the group sum of x computed once per row.
#include "moe_common.h"
#include "moe_kernels.h"
#include "moe_topk.h"

namespace moe {

__device__ __forceinline__ void row_source(const FfnArgs& a, int j, const uint8_t*& blob, int& t, int& inter) {
  const int nr = a.T * a.K;
  if (j < nr) {
    const int e = a.topk_idx[j];
    // an index outside [0, E) selects no weights: the row contributes zero
    blob = (e < 0 || e >= a.E) ? nullptr
                               : a.experts + (a.offsets ? a.offsets[e] : static_cast<uint64_t>(e) * a.stride);
    t = j / a.K;
    inter = a.I;
  } else {
    blob = a.shared;
    t = j - nr;
    inter = a.Is;
  }
}

// Sums of G consecutive values of an LDS row (G in {32, 64, 128}): thread u
// adds `per` consecutive values, then the G/per partials of a group (adjacent
// lanes of one wave) are combined by a butterfly; a fixed order either way.
template <class LoadSum>
__device__ __forceinline__ void group_sums(int n_vals, int G, int per, float* out, LoadSum load_sum) {
  const int lanes_per_group = G / per;   // 4 .. 32, a power of two dividing 64
  for (int u0 = 0; u0 < n_vals / per; u0 += blockDim.x) {
    const int u = u0 + static_cast<int>(threadIdx.x);
    float v = u < n_vals / per ? load_sum(u * per) : 0.0f;
    for (int off = 1; off < lanes_per_group; off <<= 1) v += __shfl_xor(v, off, kWave);
    if (u < n_vals / per && (u & (lanes_per_group - 1)) == 0) out[u / lanes_per_group] = v;
  }
}

// Waves per workgroup of the GEMV kernels: at batch 1 the per-wave decode
// work, not the weight bytes, sets the time, so it is spread thin.
constexpr int kGemvWaves = 16;
constexpr int kGemvBatch = 4;   // chunks whose loads a wave issues together
// gate/up splits the hidden dimension over kGemvSplit workgroups per
// pair-tile (more, smaller workgroups even out the bytes per compute unit);
// each writes its partial gate and up sums to h as
// [kGemvSplit][rows][hstride][2], and the down kernel adds the splits in
// order and applies SwiGLU while it stages h.
constexpr int kGemvGateUpWaves = 8;

// gate/up partial sums.  Grid (rows, max(I,Is)/16, kGemvSplit); one
// workgroup = one row j, one gate/up pair-tile p (16 gate rows + the 16
// matching up rows) and one split z of the 64-column chunks of H (chunks
// z, z + S, ...); its 8 waves take every 8th chunk of the split.  Per lane and
// chunk: 8 gate + 8 up values for each of two 32-column halves, in one
// 16-byte load (int4) or two (int8: the gate plane, then the up plane).  The
// weight and scale loads of a wave's first chunks are issued before the row's
// activations are staged: they do not depend on them.  int4 products run as
// packed 16-bit dot products of re-based nibbles with the raw activations;
// int8 bytes multiply activations staged as fp32.
//
// KJ > 0 (batch-1 decode): top-K runs here instead of in its own kernel.
// Wave 0 of a routed row's workgroup selects from the router's logit slices
// (KJ logits per lane, the top-K kernel's code) and passes its rank's expert
// through LDS; the other rows skip it.  A workgroup of rank k runs only the
// first k + 1 selection rounds, so the early ranks start their weight loads
// while the later ranks still select.  The weight loads then follow as usual.
//
// STREAMED (a streamed decode through the GPU-resident slot pool): a 1-D
// grid whose first kStreamCopyWgs workgroups copy the layer's missed blobs
// from host memory (stream_copy), followed by the (j, p, z) workgroups in
// the order above.  A row whose expert is being copied waits for its gate/up
// sections before its first weight load; resident rows do not wait.
template <int ACT, int BITS, int KJ, bool STREAMED = false>
__global__ __launch_bounds__(64 * kGemvGateUpWaves) void k_gateup_gemv(FfnArgs a) {
  constexpr int NW = kGemvGateUpWaves;
  constexpr int NQ = BITS / 4;   // 16-byte loads per lane and chunk
  __shared__ __attribute__((aligned(16))) uint8_t xraw[(BITS == 8 ? 4 : 2) * kMaxH];
  __shared__ float sx[kMaxH / 32];
  uint16_t* xs = reinterpret_cast<uint16_t*>(xraw);   // int4: activations as given
  float* xf = reinterpret_cast<float*>(xraw);          // int8: activations as fp32
  __shared__ float red[NW][2][16];
  const uint8_t* blob;
  int t, inter;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rows = a.T * a.K + (a.Is > 0 ? a.T : 0);
  // a streamed FFN runs a 1-D grid: the copy workgroups, then (j, p, z)
  constexpr bool streamed = STREAMED;
  static_assert(!STREAMED || KJ == 0, "a streamed FFN has its selection before gate/up");
  if (streamed && static_cast<int>(blockIdx.x) < kStreamCopyWgs) {
    stream_copy<64 * NW>(a.stream, blockIdx.x);
    return;
  }
  int j = blockIdx.x, p = blockIdx.y, z = blockIdx.z;
  if constexpr (streamed) {
    const int lin = static_cast<int>(blockIdx.x) - kStreamCopyWgs;
    const int np = (a.hstride + 15) / 16;
    j = lin % rows;
    p = (lin / rows) % np;
    z = lin / (rows * np);
  }
  // a streamed row's copy entry (-1: resident, nothing to wait for), loaded
  // first as a vector load (a scalar one would be waited for before the
  // expert lookup), so that its latency overlaps the lookup's
  int ent_v = -1;
  if (streamed && j < a.T * a.K) {
    int jv = j;
    asm volatile("" : "+v"(jv));
    ent_v = a.stream.entry_of[jv];
  }
  if (a.status_reset && j == 0 && p == 0 && z == 0 && threadIdx.x == 0) *a.status = 0u;
  if constexpr (KJ > 0) {
    __shared__ int32_t ssel[kMaxTopK];
    if (j < a.T * a.K) {   // uniform: a routed row
      if (p * 16 >= a.I) return;
      t = j / a.K;
      const int k = j - t * a.K;
      if (wave == 0) {
        TopkIn<KJ> in;
        topk_issue(a.route_part, a.route_nparts, a.T, a.E, t, lane, in);
        float bj[KJ];
        load_bias(a.route_bias, a.E, lane, bj);
        // one workgroup per token (of the last rank: it runs every round
        // anyway) writes the selection for the down and combine kernels; the
        // others stop at their own rank
        const bool writer = p == 0 && z == 0 && k == a.K - 1;
        topk_finish(in, bj, a.route_bias != nullptr, a.route_nparts, a.E, a.K, t, lane, writer ? a.sel_idx : nullptr,
                    writer ? a.sel_w : nullptr, writer ? a.sel_gamma : nullptr, nullptr, ssel, writer ? a.K : k + 1);
      }
      __syncthreads();
      const int e = ssel[k];
      blob = a.experts + (a.offsets ? a.offsets[e] : static_cast<uint64_t>(e) * a.stride);
      inter = a.I;
    } else {
      row_source(a, j, blob, t, inter);
    }
  } else {
    row_source(a, j, blob, t, inter);
  }
  if (p * 16 >= inter) return;
  float* part = a.h + ((static_cast<size_t>(z) * rows + j) * a.hstride + 16 * p) * 2;
  if (blob == nullptr) {
    if (threadIdx.x < 32) part[threadIdx.x] = 0.0f;
    return;
  }
  const int H = a.H, G = a.G;
  const int ng = H / G;
  const int n = lane & 15, kb = lane >> 4;
  const int nc = H / 64;
  const uint4* qblk = reinterpret_cast<const uint4*>(blob) + static_cast<size_t>(p) * nc * 64 * NQ;
  const uint8_t* ssec = blob + blob_gu_s(H, inter, BITS);
  uint4 q[kGemvBatch][NQ];
  uint2 sv[kGemvBatch][2];
  // a streamed row whose expert is being copied waits for its gate/up sections
  const int ent = __builtin_amdgcn_readfirstlane(ent_v);
  if (ent >= 0 && !stream_wait(a.stream, ent) && threadIdx.x == 0) atomicOr(a.status, kStatusStreamWait);
  // chunk of the wave's i-th step: z + S (wave + NW i)
  auto chunk = [&](int i) { return z + kGemvSplit * (wave + NW * i); };
  auto issue = [&](int i0) {
#pragma unroll
    for (int b = 0; b < kGemvBatch; ++b) {
      const int c = chunk(i0 + b);
      if (c < nc) {   // uniform
#pragma unroll
        for (int h = 0; h < NQ; ++h) q[b][h] = qblk[(static_cast<size_t>(c) * NQ + h) * 64 + lane];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int g = (64 * c + 32 * ks) / G;
          sv[b][ks] = *reinterpret_cast<const uint2*>(ssec + ((static_cast<uint64_t>(p) * ng + g) * 16 + n) * 8);
        }
      }
    }
  };
  issue(0);
  const uint16_t* xr = a.x + static_cast<size_t>(t) * H;
  for (int c = threadIdx.x * 8; c < H; c += 64 * NW * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(xr + c);
    if constexpr (BITS == 8) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      float f[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        f[2 * d] = act_to_f32<ACT>(w[d] & 0xFFFFu);
        f[2 * d + 1] = act_to_f32<ACT>(w[d] >> 16);
      }
      *reinterpret_cast<float4*>(xf + c) = make_float4(f[0], f[1], f[2], f[3]);
      *reinterpret_cast<float4*>(xf + c + 4) = make_float4(f[4], f[5], f[6], f[7]);
    } else {
      *reinterpret_cast<uint4*>(xs + c) = v;
    }
  }
  __syncthreads();
  group_sums(H, G, 8, sx, [&](int i) {
    float s = 0.0f;
    if constexpr (BITS == 8) {
      const float4 u = *reinterpret_cast<const float4*>(xf + i);
      const float4 v = *reinterpret_cast<const float4*>(xf + i + 4);
      s = ((u.x + u.y) + (u.z + u.w)) + ((v.x + v.y) + (v.z + v.w));
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(xs + i);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int d = 0; d < 4; ++d) s += act_to_f32<ACT>(w[d] & 0xFFFFu) + act_to_f32<ACT>(w[d] >> 16);
    }
    return s;
  });
  __syncthreads();

  float accA = 0.0f, accB = 0.0f;
  for (int i0 = 0; chunk(i0) < nc; i0 += kGemvBatch) {
    if (i0 != 0) issue(i0);
#pragma unroll
    for (int b = 0; b < kGemvBatch; ++b) {
      const int c = chunk(i0 + b);
      if (c < nc) {   // uniform
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int col = 64 * c + 32 * ks + 8 * kb;
          const int g = (64 * c + 32 * ks) / G;
          const uint2 v = sv[b][ks];
          const float sA = f16_bits_to_f32(v.x & 0xFFFFu), bA = f16_bits_to_f32(v.x >> 16);
          const float sB = f16_bits_to_f32(v.y & 0xFFFFu), bB = f16_bits_to_f32(v.y >> 16);
          if constexpr (BITS == 8) {
            // plane 0 = gate, plane 1 = up; words 0, 1 = half 0, words 2, 3 = half 1
            const float pA = ks ? bytes8_dot(q[b][0].z, q[b][0].w, xf + col) : bytes8_dot(q[b][0].x, q[b][0].y, xf + col);
            const float pB = ks ? bytes8_dot(q[b][1].z, q[b][1].w, xf + col) : bytes8_dot(q[b][1].x, q[b][1].y, xf + col);
            accA = fmaf(sA, pA, accA);
            accB = fmaf(sB, pB, accB);
            if (kb == 0 && ((64 * c + 32 * ks) % G) == 0) {
              accA = fmaf(bA, sx[g], accA);
              accB = fmaf(bB, sx[g], accB);
            }
          } else {
            const uint4 xv = *reinterpret_cast<const uint4*>(xs + col);
            const float pA = word_dot_v<ACT>(ks ? q[b][0].y : q[b][0].x, xv);
            const float pB = word_dot_v<ACT>(ks ? q[b][0].w : q[b][0].z, xv);
            accA = fmaf(16.0f * sA, pA, accA);
            accB = fmaf(16.0f * sB, pB, accB);
            if (kb == 0 && ((64 * c + 32 * ks) % G) == 0) {
              accA = fmaf(bA - 16.0f * sA, sx[g], accA);
              accB = fmaf(bB - 16.0f * sB, sx[g], accB);
            }
          }
        }
      }
    }
  }
  accA += __shfl_xor(accA, 16, kWave);
  accA += __shfl_xor(accA, 32, kWave);
  accB += __shfl_xor(accB, 16, kWave);
  accB += __shfl_xor(accB, 32, kWave);
  if (kb == 0) {
    red[wave][0][n] = accA;
    red[wave][1][n] = accB;
  }
  __syncthreads();
  if (threadIdx.x < 32) {
    const int i = threadIdx.x & 15, gu = threadIdx.x >> 4;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[w][gu][i];
    part[2 * i + gu] = v;
  }
}

// down projection.  Grid (rows, ceil(H/128)); four 32-row down pair-tiles
// per workgroup, four waves on each (wave w: pair-tile w % 4, chunks
// w / 4 + 4 i of the inter dimension).  After the weight and scale loads are
// issued, the row's h = silu(gate) * up is formed in LDS from the gate/up
// splits (added in split order), with its group sums.
template <int BITS>
__global__ __launch_bounds__(64 * kGemvWaves) void k_down_gemv(FfnArgs a) {
  constexpr int NQ = BITS / 4;
  __shared__ __attribute__((aligned(16))) float hs[kMaxInter];
  __shared__ float sh[kMaxInter / 32];
  __shared__ float red[4][4][2][16];   // K quarter, pair-tile, A / B, row
  const uint8_t* blob;
  int t, inter;
  const int j = blockIdx.x;
  row_source(a, j, blob, t, inter);
  const int H = a.H, G = a.G;
  if (blob == nullptr) {
    for (int n = threadIdx.x; n < H; n += 64 * kGemvWaves) a.yrow[static_cast<size_t>(j) * H + n] = 0.0f;
    return;
  }
  const int ng = inter / G;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pt4 = wave & 3, kq = wave >> 2;
  const int p = blockIdx.y * 4 + pt4;
  const int pc = min(p, H / 32 - 1);   // loads of a wave past the last pair-tile stay in range
  const int n = lane & 15, kb = lane >> 4;
  const int nc = inter / 64;
  const uint4* qblk =
      reinterpret_cast<const uint4*>(blob + blob_d_q(H, inter, BITS)) + static_cast<size_t>(pc) * nc * 64 * NQ;
  const uint8_t* ssec = blob + blob_d_s(H, inter, G, BITS);
  uint4 q[kGemvBatch][NQ];
  uint2 sv[kGemvBatch][2];
  auto issue = [&](int c0) {
#pragma unroll
    for (int b = 0; b < kGemvBatch; ++b) {
      const int c = c0 + 4 * b;
      if (c < nc) {   // uniform
#pragma unroll
        for (int h = 0; h < NQ; ++h) q[b][h] = qblk[(static_cast<size_t>(c) * NQ + h) * 64 + lane];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int g = (64 * c + 32 * ks) / G;
          sv[b][ks] = *reinterpret_cast<const uint2*>(ssec + ((static_cast<uint64_t>(pc) * ng + g) * 16 + n) * 8);
        }
      }
    }
  };
  issue(kq);
  const int rows = gridDim.x;
  for (int i = threadIdx.x; i < inter; i += 64 * kGemvWaves) {
    float ga = 0.0f, up = 0.0f;
#pragma unroll
    for (int z = 0; z < kGemvSplit; ++z) {
      const float2 v = *reinterpret_cast<const float2*>(a.h + ((static_cast<size_t>(z) * rows + j) * a.hstride + i) * 2);
      ga += v.x;
      up += v.y;
    }
    hs[i] = ga / (1.0f + expf(-ga)) * up;
  }
  __syncthreads();
  group_sums(inter, G, 4, sh, [&](int i) {
    const float4 v = *reinterpret_cast<const float4*>(hs + i);
    return (v.x + v.y) + (v.z + v.w);
  });
  __syncthreads();
  float accA = 0.0f, accB = 0.0f;
  for (int c0 = kq; c0 < nc; c0 += 4 * kGemvBatch) {
    if (c0 != kq) issue(c0);
#pragma unroll
    for (int b = 0; b < kGemvBatch; ++b) {
      const int c = c0 + 4 * b;
      if (c < nc) {   // uniform
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int col = 64 * c + 32 * ks + 8 * kb;
          const int g = (64 * c + 32 * ks) / G;
          const uint2 v = sv[b][ks];
          const float sA = f16_bits_to_f32(v.x & 0xFFFFu), bA = f16_bits_to_f32(v.x >> 16);
          const float sB = f16_bits_to_f32(v.y & 0xFFFFu), bB = f16_bits_to_f32(v.y >> 16);
          float pA, pB;
          if constexpr (BITS == 8) {
            pA = ks ? bytes8_dot(q[b][0].z, q[b][0].w, hs + col) : bytes8_dot(q[b][0].x, q[b][0].y, hs + col);
            pB = ks ? bytes8_dot(q[b][1].z, q[b][1].w, hs + col) : bytes8_dot(q[b][1].x, q[b][1].y, hs + col);
          } else {
            pA = word_dot_q(ks ? q[b][0].y : q[b][0].x, hs + col);
            pB = word_dot_q(ks ? q[b][0].w : q[b][0].z, hs + col);
          }
          accA = fmaf(sA, pA, accA);
          accB = fmaf(sB, pB, accB);
          if (kb == 0 && ((64 * c + 32 * ks) % G) == 0) {
            accA = fmaf(bA, sh[g], accA);
            accB = fmaf(bB, sh[g], accB);
          }
        }
      }
    }
  }
  accA += __shfl_xor(accA, 16, kWave);
  accA += __shfl_xor(accA, 32, kWave);
  accB += __shfl_xor(accB, 16, kWave);
  accB += __shfl_xor(accB, 32, kWave);
  if (kb == 0) {
    red[kq][pt4][0][n] = accA;
    red[kq][pt4][1][n] = accB;
  }
  __syncthreads();
  if (threadIdx.x < 128) {
    const int pq = threadIdx.x >> 5, half = (threadIdx.x >> 4) & 1, r = threadIdx.x & 15;
    const int pp = blockIdx.y * 4 + pq;
    if (pp * 32 < H) {
      const float v = ((red[0][pq][half][r] + red[1][pq][half][r]) + red[2][pq][half][r]) + red[3][pq][half][r];
      a.yrow[static_cast<size_t>(j) * H + 32 * pp + 16 * half + r] = v;
    }
  }
}

// Block sum over blockDim threads (multiple of 64, <= 1024) in a fixed order.
__device__ __forceinline__ float block_sum(float v, float* lds16) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if (lane == 0) lds16[wave] = v;
  __syncthreads();
  float s = 0.0f;
  for (int w = 0; w < nw; ++w) s += lds16[w];
  __syncthreads();
  return s;
}

// One workgroup of 512 threads per token; each thread owns float4 columns and
// issues the loads of all K+1 source rows before the FMAs, so a token costs
// one memory round trip per 2048 columns.  Sum order: rank 0..K-1, shared last.
template <int ACT, bool EPI>
__global__ __launch_bounds__(512) void k_combine(const float* __restrict__ yrow, const int32_t* __restrict__ inv,
                                                 const float* __restrict__ w, const float* __restrict__ gamma,
                                                 int T, int K, int H, int has_shared, float* __restrict__ y,
                                                 float* __restrict__ r, uint16_t* __restrict__ x_next) {
  __shared__ float lds16[16];
  __shared__ int src[kMaxTopK + 1];
  __shared__ float wt[kMaxTopK + 1];
  __shared__ int n_src;
  const int t = blockIdx.x, tid = threadIdx.x;
  const int H4 = H / 4;
  constexpr int kPer = kMaxH / 4 / 512;
  // the residual is read first: it does not depend on the source list
  float4 rr[kPer];
  if constexpr (EPI) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c4 = tid + 512 * u;
      rr[u] = c4 < H4 ? reinterpret_cast<const float4*>(r + static_cast<size_t>(t) * H)[c4] : make_float4(0, 0, 0, 0);
    }
  }
  if (tid < 64) {
    // sources in rank order (lane k holds rank k), then the shared expert; a
    // dropped row (inv -1) adds nothing and is left out.  The list is
    // compacted with a ballot: a kept rank goes to the number of kept ranks
    // before it.
    const int k = tid;
    int sr = -1;
    float wk = 0.0f;
    if (k < K) {
      sr = inv ? inv[t * K + k] : t * K + k;
      wk = w[t * K + k];
    }
    const float gm = (k == 0 && has_shared) ? gamma[t] : 0.0f;
    const unsigned long long kept = __ballot(sr >= 0);
    const int pos = __popcll(kept & ((1ull << k) - 1ull));
    if (sr >= 0) {
      src[pos] = sr;
      wt[pos] = wk;
    }
    if (k == 0) {
      int ns = __popcll(kept);
      if (has_shared) {
        src[ns] = T * K + t;
        wt[ns] = gm;
        ++ns;
      }
      n_src = ns;
    }
  }
  __syncthreads();
  const int ns = __builtin_amdgcn_readfirstlane(n_src);   // uniform
  constexpr int kB = 16;
  float ss = 0.0f;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c4 = tid + 512 * u;
    if (c4 < H4) {
      float4 acc = make_float4(0, 0, 0, 0);
      for (int k0 = 0; k0 < ns; k0 += kB) {
        // every load of the batch is issued (sources past the list repeat
        // the last one) before the first is used
        float4 v[kB];
#pragma unroll
        for (int b = 0; b < kB; ++b)
          v[b] = reinterpret_cast<const float4*>(yrow + static_cast<size_t>(src[min(k0 + b, ns - 1)]) * H)[c4];
#pragma unroll
        for (int b = 0; b < kB; ++b) {
          if (k0 + b < ns) {   // uniform
            const float wk = wt[k0 + b];
            acc.x = fmaf(wk, v[b].x, acc.x);
            acc.y = fmaf(wk, v[b].y, acc.y);
            acc.z = fmaf(wk, v[b].z, acc.z);
            acc.w = fmaf(wk, v[b].w, acc.w);
          }
        }
      }
      if (y) reinterpret_cast<float4*>(y + static_cast<size_t>(t) * H)[c4] = acc;
      if constexpr (EPI) {
        float4 rv = rr[u];
        rv.x += acc.x;
        rv.y += acc.y;
        rv.z += acc.z;
        rv.w += acc.w;
        reinterpret_cast<float4*>(r + static_cast<size_t>(t) * H)[c4] = rv;
        rr[u] = rv;
        ss = fmaf(rv.x, rv.x, ss);
        ss = fmaf(rv.y, rv.y, ss);
        ss = fmaf(rv.z, rv.z, ss);
        ss = fmaf(rv.w, rv.w, ss);
      }
    }
  }
  if constexpr (EPI) {
    const float tot = block_sum(ss, lds16);
    const float inv_rms = 1.0f / sqrtf(tot / static_cast<float>(H) + 1e-6f);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c4 = tid + 512 * u;
      if (c4 < H4) {
        const uint32_t a0 = f32_to_act<ACT>(rr[u].x * inv_rms), a1 = f32_to_act<ACT>(rr[u].y * inv_rms);
        const uint32_t a2 = f32_to_act<ACT>(rr[u].z * inv_rms), a3 = f32_to_act<ACT>(rr[u].w * inv_rms);
        reinterpret_cast<uint2*>(x_next + static_cast<size_t>(t) * H)[c4] = make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
      }
    }
  }
}

// The same combine when row (t, k) sits at t*K + k (no bucketing): the source
// rows are known before any load, so every row load, the weights and the
// residual are issued at once; the sums are the same as k_combine's, in the
// same order (rank 0..K-1, shared last).
template <int ACT, bool EPI>
__global__ __launch_bounds__(512) void k_combine_direct(const float* __restrict__ yrow, const float* __restrict__ w,
                                                        const float* __restrict__ gamma, int T, int K, int H,
                                                        int has_shared, float* __restrict__ y,
                                                        float* r, uint16_t* __restrict__ x_next,
                                                        const float* r_in) {
  __shared__ float lds16[16];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int H4 = H / 4;
  constexpr int kPer = kMaxH / 4 / 512;
  constexpr int kB = 16;
  const int ns = K + has_shared;
  auto src_row = [&](int i) { return i < K ? t * K + i : T * K + t; };
  auto weight = [&](int i) { return i < K ? w[t * K + i] : gamma[t]; };
  float ss = 0.0f;
  float4 rr[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int c4 = tid + 512 * u;
    if (c4 < H4) {
      if constexpr (EPI) rr[u] = reinterpret_cast<const float4*>(r_in + static_cast<size_t>(t) * H)[c4];
      float4 acc = make_float4(0, 0, 0, 0);
      for (int k0 = 0; k0 < ns; k0 += kB) {
        float4 v[kB];
#pragma unroll
        for (int b = 0; b < kB; ++b)
          v[b] = reinterpret_cast<const float4*>(yrow + static_cast<size_t>(src_row(min(k0 + b, ns - 1))) * H)[c4];
#pragma unroll
        for (int b = 0; b < kB; ++b) {
          if (k0 + b < ns) {   // uniform
            const float wk = weight(k0 + b);
            acc.x = fmaf(wk, v[b].x, acc.x);
            acc.y = fmaf(wk, v[b].y, acc.y);
            acc.z = fmaf(wk, v[b].z, acc.z);
            acc.w = fmaf(wk, v[b].w, acc.w);
          }
        }
      }
      if (y) reinterpret_cast<float4*>(y + static_cast<size_t>(t) * H)[c4] = acc;
      if constexpr (EPI) {
        float4 rv = rr[u];
        rv.x += acc.x;
        rv.y += acc.y;
        rv.z += acc.z;
        rv.w += acc.w;
        reinterpret_cast<float4*>(r + static_cast<size_t>(t) * H)[c4] = rv;
        rr[u] = rv;
        ss = fmaf(rv.x, rv.x, ss);
        ss = fmaf(rv.y, rv.y, ss);
        ss = fmaf(rv.z, rv.z, ss);
        ss = fmaf(rv.w, rv.w, ss);
      }
    }
  }
  if constexpr (EPI) {
    const float tot = block_sum(ss, lds16);
    const float inv_rms = 1.0f / sqrtf(tot / static_cast<float>(H) + 1e-6f);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c4 = tid + 512 * u;
      if (c4 < H4) {
        const uint32_t a0 = f32_to_act<ACT>(rr[u].x * inv_rms), a1 = f32_to_act<ACT>(rr[u].y * inv_rms);
        const uint32_t a2 = f32_to_act<ACT>(rr[u].z * inv_rms), a3 = f32_to_act<ACT>(rr[u].w * inv_rms);
        reinterpret_cast<uint2*>(x_next + static_cast<size_t>(t) * H)[c4] = make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
      }
    }
  }
}

template <int ACT>
__global__ __launch_bounds__(256) void k_epilogue(const float* __restrict__ y, float* __restrict__ r,
                                                  uint16_t* __restrict__ x_next, int H) {
  __shared__ float lds16[16];
  const int t = blockIdx.x;
  constexpr int kPer = kMaxH / 256;
  float rr[kPer];
  float ss = 0.0f;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int n = threadIdx.x + 256 * u;
    rr[u] = 0.0f;
    if (n < H) {
      const float v = r[static_cast<size_t>(t) * H + n] + y[static_cast<size_t>(t) * H + n];
      r[static_cast<size_t>(t) * H + n] = v;
      rr[u] = v;
      ss = fmaf(v, v, ss);
    }
  }
  const float tot = block_sum(ss, lds16);
  const float inv_rms = 1.0f / sqrtf(tot / static_cast<float>(H) + 1e-6f);
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int n = threadIdx.x + 256 * u;
    if (n < H) x_next[static_cast<size_t>(t) * H + n] = f32_to_act<ACT>(rr[u] * inv_rms);
  }
}

hipError_t launch_gateup_gemv(int act, const FfnArgs& a, hipStream_t s) {
  const int rows = a.T * a.K + (a.Is > 0 ? a.T : 0);
  const int np = (a.hstride + 15) / 16;
  const bool streamed = a.stream.first.list != nullptr;
  if (streamed && (a.route_part != nullptr || a.stream.entry_of == nullptr || a.stream.ready == nullptr ||
                   a.stream.first.len[0] + a.stream.first.len[1] == 0))
    return hipErrorInvalidValue;
  const dim3 grid = streamed ? dim3(kStreamCopyWgs + rows * np * kGemvSplit) : dim3(rows, np, kGemvSplit);
  const dim3 block(64 * kGemvGateUpWaves);
  int kj = 0;   // logits per lane of the fused top-K (0: not fused)
  if (a.route_part != nullptr) {
    if (a.E > 512) return hipErrorInvalidValue;
    kj = a.E <= 64 ? 1 : a.E <= 128 ? 2 : a.E <= 256 ? 4 : 8;
  }
#define GATEUP_LAUNCH(ACT_, BITS_, KJ_)                                                               \
  do {                                                                                                \
    if constexpr (KJ_ == 0) {                                                                         \
      if (streamed) {                                                                                 \
        hipLaunchKernelGGL((k_gateup_gemv<ACT_, BITS_, 0, true>), grid, block, 0, s, a);              \
        break;                                                                                        \
      }                                                                                               \
    }                                                                                                 \
    hipLaunchKernelGGL((k_gateup_gemv<ACT_, BITS_, KJ_>), grid, block, 0, s, a);                      \
  } while (0)
#define GATEUP_KJ(ACT_, BITS_)               \
  do {                                       \
    switch (kj) {                            \
      case 1: GATEUP_LAUNCH(ACT_, BITS_, 1); break; \
      case 2: GATEUP_LAUNCH(ACT_, BITS_, 2); break; \
      case 4: GATEUP_LAUNCH(ACT_, BITS_, 4); break; \
      case 8: GATEUP_LAUNCH(ACT_, BITS_, 8); break; \
      default: GATEUP_LAUNCH(ACT_, BITS_, 0); break; \
    }                                        \
  } while (0)
  if (a.bits == 8) {
    if (act == 2) GATEUP_KJ(2, 8);
    else GATEUP_KJ(1, 8);
  } else {
    if (act == 2) GATEUP_KJ(2, 4);
    else GATEUP_KJ(1, 4);
  }
#undef GATEUP_KJ
#undef GATEUP_LAUNCH
  return hipGetLastError();
}

hipError_t launch_down_gemv(const FfnArgs& a, hipStream_t s) {
  const int rows = a.T * a.K + (a.Is > 0 ? a.T : 0);
  dim3 grid(rows, (a.H + 127) / 128);
  if (a.bits == 8) hipLaunchKernelGGL(k_down_gemv<8>, grid, dim3(64 * kGemvWaves), 0, s, a);
  else hipLaunchKernelGGL(k_down_gemv<4>, grid, dim3(64 * kGemvWaves), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(int act, const float* yrow, const int32_t* inv, const float* w, const float* gamma, int T,
                          int K, int H, bool has_shared, float* y, float* r, uint16_t* x_next, hipStream_t s,
                          const float* r_in) {
  const int hs = has_shared ? 1 : 0;
  if (r_in == nullptr) r_in = r;
  if (inv == nullptr) {
    if (r == nullptr) {
      hipLaunchKernelGGL((k_combine_direct<2, false>), dim3(T), dim3(512), 0, s, yrow, w, gamma, T, K, H, hs, y, r,
                         x_next, r_in);
    } else if (act == 2) {
      hipLaunchKernelGGL((k_combine_direct<2, true>), dim3(T), dim3(512), 0, s, yrow, w, gamma, T, K, H, hs, y, r,
                         x_next, r_in);
    } else {
      hipLaunchKernelGGL((k_combine_direct<1, true>), dim3(T), dim3(512), 0, s, yrow, w, gamma, T, K, H, hs, y, r,
                         x_next, r_in);
    }
    return hipGetLastError();
  }
  if (r_in != r) return hipErrorInvalidValue;   // the bucketed combine updates r in place only
  if (r == nullptr) {
    hipLaunchKernelGGL((k_combine<2, false>), dim3(T), dim3(512), 0, s, yrow, inv, w, gamma, T, K, H, hs, y, r,
                       x_next);
  } else if (act == 2) {
    hipLaunchKernelGGL((k_combine<2, true>), dim3(T), dim3(512), 0, s, yrow, inv, w, gamma, T, K, H, hs, y, r,
                       x_next);
  } else {
    hipLaunchKernelGGL((k_combine<1, true>), dim3(T), dim3(512), 0, s, yrow, inv, w, gamma, T, K, H, hs, y, r,
                       x_next);
  }
  return hipGetLastError();
}

hipError_t launch_epilogue(int act, const float* y, float* r, uint16_t* x_next, int T, int H, hipStream_t s) {
  if (act == 2) hipLaunchKernelGGL(k_epilogue<2>, dim3(T), dim3(256), 0, s, y, r, x_next, H);
  else hipLaunchKernelGGL(k_epilogue<1>, dim3(T), dim3(256), 0, s, y, r, x_next, H);
  return hipGetLastError();
}

}  // namespace moe
