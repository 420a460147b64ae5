// Device helpers shared by the MoE kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// ---- 16-bit float decoding -------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}
// ACT: 1 = fp16 activations, 2 = bf16 activations
template <int ACT>
__device__ __forceinline__ float act_to_f32(uint32_t b) {
  if constexpr (ACT == 2) return bf16_bits_to_f32(b);
  else return f16_bits_to_f32(b);
}

// Round-to-nearest-even float -> 16-bit pattern of the activation type.
template <int ACT>
__device__ __forceinline__ uint16_t f32_to_act(float v) {
  if constexpr (ACT == 2) {
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
  } else {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
  }
}

// ---- wave all-reductions without LDS round trips ---------------------------
// DPP within rows of 16 lanes (pairs, quads, 8-lane halves, rows), then the
// gfx950 row-swap permutes across rows.  At every step a lane combines its
// value with exactly one partner that holds the same pair of operands, and
// the operation is commutative, so all 64 lanes end with identical bits and
// the order of the reduction is fixed.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), kCtrl, 0xF, 0xF, false));
}
template <class Op>
__device__ __forceinline__ uint32_t wave_allreduce_u32(uint32_t v, Op op) {
  v = op(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = op(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = op(v, dpp_u32<0x141>(v));  // row_half_mirror
  v = op(v, dpp_u32<0x140>(v));  // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(static_cast<int>(v), static_cast<int>(v), false, false);
  v = op(static_cast<uint32_t>(a[0]), static_cast<uint32_t>(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(static_cast<int>(v), static_cast<int>(v), false, false);
  v = op(static_cast<uint32_t>(b[0]), static_cast<uint32_t>(b[1]));
  return v;
}
// Sum over each row of 16 lanes (the first four steps of the all-reduce):
// every lane of a row ends with the row's sum, with identical bits.
__device__ __forceinline__ uint32_t dpp_row_sum(uint32_t v) {
  auto add = [](uint32_t a, uint32_t b) { return __float_as_uint(__uint_as_float(a) + __uint_as_float(b)); };
  v = add(v, dpp_u32<0xB1>(v));
  v = add(v, dpp_u32<0x4E>(v));
  v = add(v, dpp_u32<0x141>(v));
  v = add(v, dpp_u32<0x140>(v));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  return __uint_as_float(wave_allreduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}
__device__ __forceinline__ float wave_max(float v) {
  return __uint_as_float(wave_allreduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_allreduce_u32(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_allreduce_u32(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}

// Wave reduction into a scalar (uniform) result: DPP within rows of 16, then
// the row broadcasts (lane 15 of each row into the next row, lane 31 into
// rows 2 and 3), after which lane 63 holds the reduction of all 64 lanes.
// Disabled rows keep their value (old = the operand).  Six DPP steps and a
// lane read, against eight steps for the all-lane form; for max and min the
// result does not depend on the order.
// (the moved value of a disabled row is the operation's identity, so the
// move folds into the operation as one DPP instruction)
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_upd_u32(uint32_t v, uint32_t identity) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(identity), static_cast<int>(v), kCtrl, kRowMask, 0xF, false));
}
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_scalar_u32(uint32_t v, Op op, uint32_t id) {
  v = op(v, dpp_upd_u32<0xB1, 0xF>(v, id));    // quad_perm [1,0,3,2]
  v = op(v, dpp_upd_u32<0x4E, 0xF>(v, id));    // quad_perm [2,3,0,1]
  v = op(v, dpp_upd_u32<0x141, 0xF>(v, id));   // row_half_mirror
  v = op(v, dpp_upd_u32<0x140, 0xF>(v, id));   // row_mirror
  v = op(v, dpp_upd_u32<0x142, 0xA>(v, id));   // row_bcast:15 into rows 1 and 3
  v = op(v, dpp_upd_u32<0x143, 0xC>(v, id));   // row_bcast:31 into rows 2 and 3
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}
__device__ __forceinline__ uint32_t wave_max_u32_s(uint32_t v) {
  return wave_reduce_scalar_u32(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; }, 0u);
}
__device__ __forceinline__ uint32_t wave_min_u32_s(uint32_t v) {
  return wave_reduce_scalar_u32(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; }, 0xFFFFFFFFu);
}

// ---- int4 nibble words -------------------------------------------------------
// A 32-bit word holds 8 values; value j sits in nibble (j>>1) + 4*(j&1).
//
// Pairs for packed 16-bit dot products: pair m (m = 0..3) holds values 2m
// (low half) and 2m+1 (high half) = nibbles m and m+4, re-based so that each
// half encodes v = 1 + q/16 exactly (bf16: q in mantissa bits 3..6 under
// exponent 0x3F8; fp16: q in mantissa bits 6..9 under exponent 0x3C0).  Then
// sum_j q_j x_j = 16 * sum_j v_j x_j - 16 * sum_j x_j.
template <int ACT>
__device__ __forceinline__ uint32_t q_pair(uint32_t w, int m) {
  if constexpr (ACT == 2) {
    uint32_t t = (m == 0) ? (w << 3) : (w >> (4 * m - 3));
    return (t & 0x00780078u) | 0x3F803F80u;
  } else {
    uint32_t t = (m == 0) ? (w << 6) : (m == 1) ? (w << 2) : (w >> (4 * m - 6));
    return (t & 0x03C003C0u) | 0x3C003C00u;
  }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <int ACT>
__device__ __forceinline__ float dot2_acc(uint32_t a, uint32_t b, float c) {
  if constexpr (ACT == 2)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}

// sum_j v_j * x_j over one word, x given as 4 packed 16-bit pairs (cols 2m, 2m+1).
template <int ACT>
__device__ __forceinline__ float word_dot_v(uint32_t w, uint4 x) {
  float p = dot2_acc<ACT>(q_pair<ACT>(w, 0), x.x, 0.0f);
  p = dot2_acc<ACT>(q_pair<ACT>(w, 1), x.y, p);
  p = dot2_acc<ACT>(q_pair<ACT>(w, 2), x.z, p);
  p = dot2_acc<ACT>(q_pair<ACT>(w, 3), x.w, p);
  return p;
}

// sum_j q_j * h_j over one word with fp32 h[0..7] (exact integer q).
__device__ __forceinline__ float word_dot_q(uint32_t w, const float* h) {
  const uint32_t lo = w & 0x0F0F0F0Fu;          // nibbles 0,2,4,6 = values 0,4,1,5
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // nibbles 1,3,5,7 = values 2,6,3,7
  float p = static_cast<float>(lo & 0xFFu) * h[0];
  p = fmaf(static_cast<float>((lo >> 16) & 0xFFu), h[1], p);
  p = fmaf(static_cast<float>(hi & 0xFFu), h[2], p);
  p = fmaf(static_cast<float>((hi >> 16) & 0xFFu), h[3], p);
  p = fmaf(static_cast<float>((lo >> 8) & 0xFFu), h[4], p);
  p = fmaf(static_cast<float>(lo >> 24), h[5], p);
  p = fmaf(static_cast<float>((hi >> 8) & 0xFFu), h[6], p);
  p = fmaf(static_cast<float>(hi >> 24), h[7], p);
  return p;
}

// sum_j q_j * x_j over 8 int8 values (bytes 0..3 of lo, then of hi) with fp32
// x[0..7]; every product is exact in fp32.
__device__ __forceinline__ float bytes8_dot(uint32_t lo, uint32_t hi, const float* x) {
  float p = static_cast<float>(lo & 0xFFu) * x[0];
  p = fmaf(static_cast<float>((lo >> 8) & 0xFFu), x[1], p);
  p = fmaf(static_cast<float>((lo >> 16) & 0xFFu), x[2], p);
  p = fmaf(static_cast<float>(lo >> 24), x[3], p);
  p = fmaf(static_cast<float>(hi & 0xFFu), x[4], p);
  p = fmaf(static_cast<float>((hi >> 8) & 0xFFu), x[5], p);
  p = fmaf(static_cast<float>((hi >> 16) & 0xFFu), x[6], p);
  p = fmaf(static_cast<float>(hi >> 24), x[7], p);
  return p;
}

// ---- blob geometry (see the public header for the byte layout) -------------
// bits = 4 or 8: the value sections scale with the weight width, the scale
// sections do not.
__host__ __device__ __forceinline__ uint64_t blob_gu_q(int, int) { return 0; }
__host__ __device__ __forceinline__ uint64_t blob_d_q(int H, int I, int bits = 4) { return (uint64_t)I * H * bits / 4; }
__host__ __device__ __forceinline__ uint64_t blob_gu_s(int H, int I, int bits = 4) { return 3ull * I * H * bits / 8; }
__host__ __device__ __forceinline__ uint64_t blob_d_s(int H, int I, int G, int bits = 4) {
  return 3ull * I * H * bits / 8 + 8ull * I * H / G;
}
__host__ __device__ __forceinline__ uint64_t blob_size(int H, int I, int G, int bits = 4) {
  return 3ull * I * H * bits / 8 + 12ull * I * H / G;
}

// fp16 scale/bias entry [s_A, b_A, s_B, b_B] of (pair-tile p, group g, row n)
struct ScaleBias {
  float sA, bA, sB, bB;
};
__device__ __forceinline__ ScaleBias load_sb(const uint8_t* sec, int p, int ng, int g, int n) {
  const uint2 v = *reinterpret_cast<const uint2*>(sec + ((static_cast<uint64_t>(p) * ng + g) * 16 + n) * 8);
  ScaleBias r;
  r.sA = f16_bits_to_f32(v.x & 0xFFFFu);
  r.bA = f16_bits_to_f32(v.x >> 16);
  r.sB = f16_bits_to_f32(v.y & 0xFFFFu);
  r.bB = f16_bits_to_f32(v.y >> 16);
  return r;
}

}  // namespace moe
