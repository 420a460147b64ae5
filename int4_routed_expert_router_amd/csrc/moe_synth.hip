// Seeded synthetic expert blobs generated on the device (input generator for
// benchmarks and tests; holds none of the MoE method's arithmetic).
#include <hip/hip_runtime.h>

#include "moe.h"
#include "moe_synth.h"

namespace moe {
namespace synth {

// Philox4x32-10 (Salmon et al., SC'11, section 3.2): multipliers and Weyl key
// increments of the 4x32 variant, ten rounds.
struct P4 {
  uint32_t v[4];
};
__device__ __forceinline__ P4 philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint32_t hi0 = __umulhi(M0, c0), lo0 = M0 * c0;
    const uint32_t hi1 = __umulhi(M1, c2), lo1 = M1 * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return P4{{c0, c1, c2, c3}};
}

// 8 generator values (nibble i = value i) -> blob word (value j in nibble (j>>1)+4(j&1))
__device__ __forceinline__ uint32_t to_blob_word(uint32_t g) {
  uint32_t out = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) out |= ((g >> (4 * j)) & 0xFu) << (4 * ((j >> 1) + 4 * (j & 1)));
  return out;
}

__device__ __forceinline__ uint32_t gen_word8(uint32_t key0, uint32_t layer, uint32_t eid, uint32_t tensor,
                                              uint64_t j) {
  const P4 r = philox(static_cast<uint32_t>(j >> 5), eid, tensor, 0, key0, layer);
  return r.v[(j & 31) >> 3];
}

// int8: values j .. j+7 (j a multiple of 8) = the bytes of words (j%16)/4 and
// (j%16)/4 + 1 of block j/16, in natural order
__device__ __forceinline__ uint2 gen_bytes8(uint32_t key0, uint32_t layer, uint32_t eid, uint32_t tensor, uint64_t j) {
  const P4 r = philox(static_cast<uint32_t>(j >> 4), eid, tensor, 0, key0, layer);
  return (j & 8) ? make_uint2(r.v[2], r.v[3]) : make_uint2(r.v[0], r.v[1]);
}

// bias_mul = -2^(bits-1): b = -8 s for int4, -128 s for int8 (exact)
__device__ __forceinline__ uint32_t gen_scale_bias(uint32_t key0, uint32_t layer, uint32_t eid, uint32_t tensor,
                                                   uint64_t j, float lo, float span, float bias_mul) {
#pragma clang fp contract(off)
  const P4 r = philox(static_cast<uint32_t>(j >> 2), eid, tensor, 0, key0, layer);
  const float u = static_cast<float>(r.v[j & 3] >> 8) * 5.9604644775390625e-8f;  // 2^-24, exact
  const float prod = u * span;
  const float s32 = prod + lo;
  const _Float16 s = static_cast<_Float16>(s32);
  const _Float16 b = static_cast<_Float16>(bias_mul * static_cast<float>(s));
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, s)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

// One work unit writes one 16-byte lane record of a value block (int4: the
// lane's four words of a 1 KiB chunk block; int8: the lane's 16 bytes in one
// tile plane of a 2 KiB chunk block) or one 8-byte scale entry.
template <int BITS>
__global__ __launch_bounds__(256) void k_fill(uint32_t key0, uint32_t layer, int expert_first, int H, int I, int G,
                                              float lo, float span, uint8_t* dst, uint64_t stride) {
  constexpr int NQ = BITS / 4;
  const uint32_t eid = static_cast<uint32_t>(expert_first + static_cast<int>(blockIdx.y));
  uint8_t* blob = dst + blockIdx.y * stride;
  const uint64_t u_gu = static_cast<uint64_t>(I / 16) * (H / 64) * 64 * NQ;
  const uint64_t u_d = static_cast<uint64_t>(H / 32) * (I / 64) * 64 * NQ;
  const uint64_t u_gus = static_cast<uint64_t>(I / 16) * (H / G) * 16;
  const uint64_t u_ds = static_cast<uint64_t>(H / 32) * (I / G) * 16;
  const uint64_t total = u_gu + u_d + u_gus + u_ds;
  for (uint64_t u = blockIdx.x * 256ull + threadIdx.x; u < total; u += static_cast<uint64_t>(gridDim.x) * 256) {
    if (u < u_gu + u_d) {
      const bool gu = u < u_gu;
      const uint64_t v = gu ? u : u - u_gu;
      const int in_dim = gu ? H : I;
      const int nc = in_dim / 64;
      const int l = static_cast<int>(v & 63);
      const int n = l & 15, kb = l >> 4;
      uint8_t* sec = blob + (gu ? 0 : static_cast<uint64_t>(I) * H * BITS / 4);
      if constexpr (BITS == 8) {
        const int tile = static_cast<int>((v >> 6) & 1);
        const uint64_t blk = v >> 7;
        const int c = static_cast<int>(blk % nc);
        const int p = static_cast<int>(blk / nc);
        const int row = gu ? 16 * p + n : 32 * p + 16 * tile + n;
        const uint32_t tensor = gu ? static_cast<uint32_t>(tile) : 2u;
        uint2 half[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int col = 64 * c + 32 * ks + 8 * kb;
          half[ks] = gen_bytes8(key0, layer, eid, tensor, static_cast<uint64_t>(row) * in_dim + col);
        }
        *reinterpret_cast<uint4*>(sec + blk * 2048 + 1024 * tile + 16 * l) =
            make_uint4(half[0].x, half[0].y, half[1].x, half[1].y);
        continue;
      }
      const uint64_t blk = v >> 6;
      const int c = static_cast<int>(blk % nc);
      const int p = static_cast<int>(blk / nc);
      uint32_t words[4];
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const int tile = wd >> 1, ks = wd & 1;
        const int row = gu ? 16 * p + n : 32 * p + 16 * tile + n;
        const uint32_t tensor = gu ? static_cast<uint32_t>(tile) : 2u;
        const int col = 64 * c + 32 * ks + 8 * kb;
        const uint64_t j = static_cast<uint64_t>(row) * in_dim + col;
        words[wd] = to_blob_word(gen_word8(key0, layer, eid, tensor, j));
      }
      *reinterpret_cast<uint4*>(sec + blk * 1024 + 16 * l) = make_uint4(words[0], words[1], words[2], words[3]);
    } else {
      const bool gu = u < u_gu + u_d + u_gus;
      const uint64_t v = gu ? u - u_gu - u_d : u - u_gu - u_d - u_gus;
      const int in_dim = gu ? H : I;
      const int ng = in_dim / G;
      const int n = static_cast<int>(v & 15);
      const uint64_t pg = v >> 4;
      const int g = static_cast<int>(pg % ng);
      const int p = static_cast<int>(pg / ng);
      uint32_t ab[2];
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        const int row = gu ? 16 * p + n : 32 * p + 16 * tile + n;
        const uint32_t tensor = gu ? 3u + tile : 5u;
        const uint64_t j = static_cast<uint64_t>(row) * ng + g;
        ab[tile] = gen_scale_bias(key0, layer, eid, tensor, j, lo, span, -static_cast<float>(1 << (BITS - 1)));
      }
      const uint64_t sec = 3ull * I * H * BITS / 8 + (gu ? 0 : 8ull * I * H / G);
      *reinterpret_cast<uint2*>(blob + sec + v * 8) = make_uint2(ab[0], ab[1]);
    }
  }
}

__global__ void k_philox(const uint32_t* ctr, const uint32_t* key, uint32_t* out, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const P4 r = philox(ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3], key[2 * i], key[2 * i + 1]);
  for (int k = 0; k < 4; ++k) out[4 * i + k] = r.v[k];
}

}  // namespace synth
}  // namespace moe

namespace {
thread_local char g_err[256] = "";
}  // namespace

extern "C" moe_status moe_synth_fill_experts(uint64_t seed, int32_t layer, int32_t expert_first, int32_t n_experts,
                                             int32_t H, int32_t I, int32_t G, int32_t bits, float lo, float span,
                                             uint8_t* dst, uint64_t stride, moe_stream stream) {
  const uint64_t bytes = moe_blob_bytes_q(H, I, G, bits);
  if (bytes == 0 || n_experts < 0 || layer < 0 || expert_first < 0) return MOE_ESHAPE;
  if (n_experts == 0) return MOE_OK;
  if (!dst || (reinterpret_cast<uintptr_t>(dst) % 256) || stride % 256 || stride < bytes) return MOE_EINVAL;
  const uint64_t units = bytes / 16;  // at least this many work units per expert
  const unsigned gx = static_cast<unsigned>(units / 256 / 4 + 1);
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint32_t k0 = static_cast<uint32_t>(seed & 0xFFFFFFFFu), ly = static_cast<uint32_t>(layer);
  if (bits == 8)
    hipLaunchKernelGGL(moe::synth::k_fill<8>, dim3(gx, n_experts), dim3(256), 0, s, k0, ly, expert_first, H, I, G, lo, span, dst,
                       stride);
  else
    hipLaunchKernelGGL(moe::synth::k_fill<4>, dim3(gx, n_experts), dim3(256), 0, s, k0, ly, expert_first, H, I, G, lo, span, dst,
                       stride);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}

extern "C" moe_status moe_synth_philox(const uint32_t* ctr, const uint32_t* key, uint32_t* out, int32_t n,
                                       moe_stream stream) {
  if (n < 0) return MOE_ESHAPE;
  if (n == 0) return MOE_OK;
  if (!ctr || !key || !out) return MOE_EINVAL;
  hipLaunchKernelGGL(moe::synth::k_philox, dim3((n + 255) / 256), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), ctr, key,
                     out, n);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}
