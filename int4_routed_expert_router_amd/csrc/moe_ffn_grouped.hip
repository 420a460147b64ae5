// Batched grouped-GEMM family on the gfx950 matrix cores.
//
// When a batch routes many tokens to the same experts, each expert's weights
// are streamed for all of its tokens together: the rows of the batch are
// bucketed by expert (stable counting sort), and workgroups multiply up to 16
// of one expert's token rows by a slice of that expert's weights with
// v_mfma_f32_16x16x32_{bf16,f16}.
//
// Precision.  The weight operand is the nibble itself, exactly: each 16-bit
// lane value encodes v = 1 + q/16 (exact in bf16 and fp16), so one MFMA over a
// 32-column half computes P = sum v*x with exact products and fp32
// accumulation.  The affine group dequantisation is applied in fp32:
//     sum_c (s q_c + b) x_c = 16 s P + (b - 16 s) sum_c x_c,
// the scale term per 64-column chunk (one FMA per output), the bias term once
// per work item as one more matrix product over the groups,
// [tokens x groups](sum x) . [groups x rows](b - 16 s), with both operands
// split into bf16 hi + lo pairs (four MFMAs, error near 2^-16 relative).
// Activations are exact in the operand type; the SwiGLU output h enters the
// down projection as a hi + lo bf16 pair (h = hi + lo to 16 significant bits).
//
// Operand layout of v_mfma_f32_16x16x32 (64 lanes, lane l: n = l % 16,
// kb = l / 16): A lane holds row m = n, k = 8kb..8kb+7; B lane holds column n,
// k = 8kb..8kb+7; C lane holds rows 4kb..4kb+3 of column n.  The expert blob
// stores each lane's B values contiguously (see the public header), so one
// 16-byte load per lane fetches the B operands of two 16-row tiles for a
// 64-column chunk.
//
// Scheduling.  A unit is (expert, block of output rows); it is split into
// sub-items of 16 tokens.  Units are ordered longest first (the shared expert,
// then routed experts by descending token count).  The sub-items of one unit
// get workgroup ids that are equal modulo 8, so they land on the same XCD
// (workgroups are dealt to the 8 XCDs round-robin) and re-reads of the unit's
// weights hit that XCD's L2.  Each sub-item stages its tokens' activations in
// LDS once, with direct global-to-LDS loads, then runs a barrier-free loop
// over the weight chunks with the weight loads kPF chunks ahead.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int kSub = 16;            // tokens per work item (one MFMA M-tile)
constexpr int kStageCols = 2048;    // activation columns staged per pass (gate/up)
constexpr int kStageColsD = 512;    // h columns staged per pass (down)
constexpr int kPF = 8;              // weight chunks in flight per wave (divides the chunks of a pass)
constexpr int kMaxGridGU = 1024;   // persistent grids (multiples of 8: a workgroup keeps its XCD residue)
constexpr int kMaxGridD = 2048;

template <int ACT>
__device__ __forceinline__ f32x4_t mfma(uint4 a, uint4 b, f32x4_t c) {
  if constexpr (ACT == 2)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
}

// The 8 values of a blob word as an MFMA operand (value j -> slot j).
template <int ACT>
__device__ __forceinline__ uint4 word_operand(uint32_t w) {
  return make_uint4(q_pair<ACT>(w, 0), q_pair<ACT>(w, 1), q_pair<ACT>(w, 2), q_pair<ACT>(w, 3));
}

// fp32 -> (hi, lo) bf16 bit patterns with hi + lo = v to 16 significant bits.
__device__ __forceinline__ void split_bf16(float v, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_act<2>(v);
  lo = f32_to_act<2>(v - bf16_bits_to_f32(hi));
}

// 16-byte global -> LDS copy by all active lanes of a wave; lane i writes
// 16 bytes at lds_base + 16 i (lds_base is wave-uniform).
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_ptr)(lds_base), 16, 0, 0);
}

// Staged tile: rows x cols 16-bit values in 16-byte units; unit (m, u8) holds
// columns 8*u8..8*u8+7 of row m at position m*(cols/8) + (u8 ^ (m & 7)), so the
// 16 lanes reading the same column block of 16 rows hit different banks.
__device__ __forceinline__ int unit_pos(int m, int u8, int units_per_row) {
  return m * units_per_row + (u8 ^ (m & 7));
}

struct Unit {
  const uint8_t* blob;
  int r0;      // first row of this expert (sorted order) in the row space of h / yrow
  int M;       // tokens of this expert
  int inter;
  int block;   // output block within the expert
  bool shared;
};

// Unit u: units [0, nb_s) are the shared expert's blocks, then n_act routed
// experts (active[] is in descending token-count order) of nb blocks each.
__device__ __forceinline__ bool get_unit(const FfnArgs& a, int u, int n_act, int nb, int nb_s, Unit& un) {
  if (u < nb_s) {
    un.blob = a.shared;
    un.r0 = a.T * a.K;
    un.M = a.T;
    un.inter = a.Is;
    un.block = u;
    un.shared = true;
    return true;
  }
  u -= nb_s;
  if (u >= n_act * nb) return false;
  const int e = a.active[u / nb];
  un.blob = a.experts + (a.offsets ? a.offsets[e] : static_cast<uint64_t>(e) * a.stride);
  un.r0 = a.expert_off[e];
  un.M = a.expert_off[e + 1] - un.r0;
  un.inter = a.I;
  un.block = u % nb;
  un.shared = false;
  return true;
}

// Work id -> (unit, sub-item): ids come in windows of 8*S; window w holds units
// 8w..8w+7, and sub-item s of unit 8w+r has id 8*S*w + 8*s + r.
__device__ __forceinline__ void decode_id(int id, int S, int& unit, int& sub) {
  const int win = 8 * S;
  const int w = id / win, rem = id - w * win;
  sub = rem >> 3;
  unit = 8 * w + (rem & 7);
}

// Bias MFMA operands for groups [g0, g0+32) of the lane's row: B = (b - 16 s)
// of tile A and tile B as hi/lo bf16 (zero beyond ng).
__device__ __forceinline__ void bias_operands(const uint8_t* ssec, int p, int ng, int g0, int n, int kb, uint4& ah,
                                              uint4& al, uint4& bh, uint4& bl) {
  // all eight loads first (clamped index, no branches), so they overlap
  uint2 v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int g = min(g0 + 8 * kb + j, ng - 1);
    v[j] = *reinterpret_cast<const uint2*>(ssec + ((static_cast<uint64_t>(p) * ng + g) * 16 + n) * 8);
  }
  uint32_t vah[4], val[4], vbh[4], vbl[4];
#pragma unroll
  for (int j2 = 0; j2 < 4; ++j2) {
    uint32_t h2[2][2], l2[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = 2 * j2 + h;
      const bool in = g0 + 8 * kb + j < ng;
      const float ba = in ? fmaf(-16.0f, f16_bits_to_f32(v[j].x & 0xFFFFu), f16_bits_to_f32(v[j].x >> 16)) : 0.0f;
      const float bb = in ? fmaf(-16.0f, f16_bits_to_f32(v[j].y & 0xFFFFu), f16_bits_to_f32(v[j].y >> 16)) : 0.0f;
      split_bf16(ba, h2[0][h], l2[0][h]);
      split_bf16(bb, h2[1][h], l2[1][h]);
    }
    vah[j2] = h2[0][0] | (h2[0][1] << 16);
    val[j2] = l2[0][0] | (l2[0][1] << 16);
    vbh[j2] = h2[1][0] | (h2[1][1] << 16);
    vbl[j2] = l2[1][0] | (l2[1][1] << 16);
  }
  ah = make_uint4(vah[0], vah[1], vah[2], vah[3]);
  al = make_uint4(val[0], val[1], val[2], val[3]);
  bh = make_uint4(vbh[0], vbh[1], vbh[2], vbh[3]);
  bl = make_uint4(vbl[0], vbl[1], vbl[2], vbl[3]);
}

// A operand of the bias MFMA: group sums of row m (lane n), groups g0+8kb..+7, hi/lo.
__device__ __forceinline__ void sum_operands(const float* sums, int stride, int ng, int g0, int n, int kb, uint4& hi,
                                             uint4& lo) {
  uint32_t vh[4], vl[4];
#pragma unroll
  for (int j2 = 0; j2 < 4; ++j2) {
    uint32_t h[2], l[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int g = g0 + 8 * kb + 2 * j2 + k;
      split_bf16(g < ng ? sums[n * stride + g] : 0.0f, h[k], l[k]);
    }
    vh[j2] = h[0] | (h[1] << 16);
    vl[j2] = l[0] | (l[1] << 16);
  }
  hi = make_uint4(vh[0], vh[1], vh[2], vh[3]);
  lo = make_uint4(vl[0], vl[1], vl[2], vl[3]);
}

__device__ __forceinline__ f32x4_t bias_mfma(uint4 sh, uint4 sl, uint4 bh, uint4 bl, f32x4_t c) {
  c = mfma<2>(sh, bh, c);
  c = mfma<2>(sh, bl, c);
  c = mfma<2>(sl, bh, c);
  c = mfma<2>(sl, bl, c);
  return c;
}

// ---------------------------------------------------------------------------
// gate/up + SwiGLU.  Unit = (expert, 64 rows of I); wave w owns gate/up
// pair-tile p = 4*block + w.  Output: h as separate hi and lo bf16 planes.
// ---------------------------------------------------------------------------
template <int ACT, int G>
__global__ __launch_bounds__(256) void k_gateup_grouped(FfnArgs a, int S) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[kSub * kStageCols];
  __shared__ float gsum[kSub][kStageCols / 32 + 1];
  __shared__ int tok[kSub];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kb = lane >> 4;
  const int H = a.H, K = a.K;
  const int nc = H / 64, ng = H / G;
  const int n_act = *a.n_active;
  const int nb = a.I / 64, nb_s = a.Is / 64;
  const int units = nb_s + n_act * nb;
  const int ids = ((units + 7) / 8) * 8 * S;
  const int hplane = (a.T * a.K + (a.Is > 0 ? a.T : 0)) * a.hstride;
  uint16_t* h_hi = reinterpret_cast<uint16_t*>(a.h);
  uint16_t* h_lo = h_hi + hplane;
  for (int id = blockIdx.x; id < ids; id += gridDim.x) {
    int ui, sub;
    decode_id(id, S, ui, sub);
    Unit un;
    if (!get_unit(a, ui, n_act, nb, nb_s, un)) continue;
    const int m0 = sub * kSub;
    if (m0 >= un.M) continue;
    const int mc = min(kSub, un.M - m0);
    const int p = 4 * un.block + wave;
    const uint4* qblk = reinterpret_cast<const uint4*>(un.blob) + static_cast<size_t>(p) * nc * 64;
    const uint8_t* ssec = un.blob + blob_gu_s(H, un.inter);
    __syncthreads();  // previous item's LDS readers are done
    if (tid < mc) tok[tid] = un.shared ? (m0 + tid) : a.perm[un.r0 + m0 + tid] / K;
    // weight prefetch for the first kPF chunks
    uint4 qn[kPF];
    uint2 sn[kPF];
#pragma unroll
    for (int u = 0; u < kPF; ++u) {
      if (u < nc) {
        qn[u] = qblk[static_cast<size_t>(u) * 64 + lane];
        sn[u] = *reinterpret_cast<const uint2*>(ssec + ((static_cast<uint64_t>(p) * ng + (64 * u) / G) * 16 + n) * 8);
      }
    }
    f32x4_t accg = {0, 0, 0, 0}, accu = {0, 0, 0, 0};
    f32x4_t bsg = {0, 0, 0, 0}, bsu = {0, 0, 0, 0};
    for (int k0 = 0; k0 < H; k0 += kStageCols) {
      const int kr = min(kStageCols, H - k0);
      const int upr = kr / 8;
      __syncthreads();  // tok visible; previous pass done
      // stage x[tok[0..mc), k0..k0+kr) with direct loads into LDS
      for (int op = wave; op * 64 < kSub * upr; op += 4) {
        const int u = op * 64 + lane;
        const int m = u / upr, ph = u - m * upr;
        if (m < mc) {
          const int u8 = ph ^ (m & 7);
          dma16(a.x + static_cast<size_t>(tok[m]) * H + k0 + 8 * u8, &xs[op * 64 * 8]);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);  // this wave's direct-to-LDS loads have landed
      __syncthreads();
      // group sums of the staged columns
      const int gpr = kr / G;
      for (int idx = tid; idx < kSub * gpr; idx += 256) {
        const int m = idx / gpr, g = idx - m * gpr;
        float s = 0.0f;
        if (m < mc) {
          for (int c8 = 0; c8 < G / 8; ++c8) {
            const uint4 v = *reinterpret_cast<const uint4*>(&xs[unit_pos(m, g * (G / 8) + c8, upr) * 8]);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) s += act_to_f32<ACT>(w4[i] & 0xFFFFu) + act_to_f32<ACT>(w4[i] >> 16);
          }
        }
        gsum[m][g] = s;
      }
      __syncthreads();
      // bias term for the groups of this pass
      for (int g0 = 0; g0 < gpr; g0 += 32) {
        uint4 sh, sl, bah, bal, bbh, bbl;
        sum_operands(&gsum[0][0], kStageCols / 32 + 1, gpr, g0, n, kb, sh, sl);
        bias_operands(ssec, p, ng, k0 / G + g0, n, kb, bah, bal, bbh, bbl);
        // groups beyond this pass are zero in sh/sl (sum_operands pads with 0)
        bsg = bias_mfma(sh, sl, bah, bal, bsg);
        bsu = bias_mfma(sh, sl, bbh, bbl, bsu);
      }
      // scale term over the chunks of this pass
      f32x4_t pg = {0, 0, 0, 0}, pu = {0, 0, 0, 0};
      const int c_lo = k0 / 64, c_hi = (k0 + kr) / 64;
      // The whole pass is unrolled: chunk c lives in register slot (c - c_lo) % kPF
      // (c_lo is a multiple of kPF), is consumed, then the slot is refilled with
      // chunk c + kPF (index clamped, so the refill is unconditional and writes
      // the slot's own registers).  No loop back-edge forces the in-flight
      // refills to complete early.
#pragma unroll
      for (int ci = 0; ci < kStageCols / 64; ++ci) {
        {
          const int u = ci % kPF;
          const int c = c_lo + ci;
          const uint4 q = qn[u];
          const uint2 sr = sn[u];
          const uint4 bg0 = word_operand<ACT>(q.x), bg1 = word_operand<ACT>(q.y);
          const uint4 bu0 = word_operand<ACT>(q.z), bu1 = word_operand<ACT>(q.w);
          const float sg = f16_bits_to_f32(sr.x & 0xFFFFu), su = f16_bits_to_f32(sr.y & 0xFFFFu);
          const int cn = min(c + kPF, nc - 1);
          qn[u] = qblk[static_cast<size_t>(cn) * 64 + lane];
          sn[u] = *reinterpret_cast<const uint2*>(ssec + ((static_cast<uint64_t>(p) * ng + (64 * cn) / G) * 16 + n) * 8);
          if (c < c_hi) {
            const int u8 = (c * 64 - k0) / 8 + kb;
            const uint4 a0 = *reinterpret_cast<const uint4*>(&xs[unit_pos(n, u8, upr) * 8]);
            const uint4 a1 = *reinterpret_cast<const uint4*>(&xs[unit_pos(n, u8 + 4, upr) * 8]);
            if constexpr (G == 32) {
              const uint2 sr1 = *reinterpret_cast<const uint2*>(
                  ssec + ((static_cast<uint64_t>(p) * ng + 2 * c + 1) * 16 + n) * 8);
              const float sg1 = f16_bits_to_f32(sr1.x & 0xFFFFu), su1 = f16_bits_to_f32(sr1.y & 0xFFFFu);
              const f32x4_t z = {0, 0, 0, 0};
              const f32x4_t g0v = mfma<ACT>(a0, bg0, z), u0v = mfma<ACT>(a0, bu0, z);
              const f32x4_t g1v = mfma<ACT>(a1, bg1, z), u1v = mfma<ACT>(a1, bu1, z);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                accg[i] = fmaf(sg, g0v[i], accg[i]);
                accu[i] = fmaf(su, u0v[i], accu[i]);
                accg[i] = fmaf(sg1, g1v[i], accg[i]);
                accu[i] = fmaf(su1, u1v[i], accu[i]);
              }
            } else {
              pg = mfma<ACT>(a0, bg0, pg);
              pu = mfma<ACT>(a0, bu0, pu);
              pg = mfma<ACT>(a1, bg1, pg);
              pu = mfma<ACT>(a1, bu1, pu);
              if (G == 64 || (c & 1)) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  accg[i] = fmaf(sg, pg[i], accg[i]);
                  accu[i] = fmaf(su, pu[i], accu[i]);
                }
                pg = f32x4_t{0, 0, 0, 0};
                pu = f32x4_t{0, 0, 0, 0};
              }
            }
          }
        }
      }
    }
    // SwiGLU; lane holds tokens 4kb..4kb+3 of column n of pair-tile p
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * kb + i;
      if (m < mc) {
        const float ga = fmaf(16.0f, accg[i], bsg[i]);
        const float up = fmaf(16.0f, accu[i], bsu[i]);
        const float hv = ga / (1.0f + expf(-ga)) * up;
        uint32_t hi, lo;
        split_bf16(hv, hi, lo);
        const size_t o = static_cast<size_t>(un.r0 + m0 + m) * a.hstride + 16 * p + n;
        h_hi[o] = static_cast<uint16_t>(hi);
        h_lo[o] = static_cast<uint16_t>(lo);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// down projection.  Unit = (expert, 128 output rows); wave w owns down
// pair-tile p = 4*block + w (32 rows).  Reads h (hi/lo planes) of its tokens.
// ---------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void k_down_grouped(FfnArgs a, int S) {
  __shared__ __attribute__((aligned(16))) uint16_t hsh[kSub * kStageColsD];
  __shared__ __attribute__((aligned(16))) uint16_t hsl[kSub * kStageColsD];
  __shared__ float gsum[kSub][kStageColsD / 32 + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kb = lane >> 4;
  const int H = a.H;
  const int n_act = *a.n_active;
  const int nb = (H + 127) / 128;
  const int nb_s = (a.Is > 0) ? nb : 0;
  const int units = nb_s + n_act * nb;
  const int ids = ((units + 7) / 8) * 8 * S;
  const int hplane = (a.T * a.K + (a.Is > 0 ? a.T : 0)) * a.hstride;
  const uint16_t* h_hi = reinterpret_cast<const uint16_t*>(a.h);
  const uint16_t* h_lo = h_hi + hplane;
  for (int id = blockIdx.x; id < ids; id += gridDim.x) {
    int ui, sub;
    decode_id(id, S, ui, sub);
    Unit un;
    if (!get_unit(a, ui, n_act, nb, nb_s, un)) continue;
    const int m0 = sub * kSub;
    if (m0 >= un.M) continue;
    const int mc = min(kSub, un.M - m0);
    const int p = 4 * un.block + wave;
    const bool active_wave = p * 32 < H;
    const int I = un.inter;
    const int nc = I / 64, ng = I / G;
    const uint4* qblk = reinterpret_cast<const uint4*>(un.blob + blob_d_q(H, I)) + static_cast<size_t>(p) * nc * 64;
    const uint8_t* ssec = un.blob + blob_d_s(H, I, G);
    const size_t row0 = static_cast<size_t>(un.r0 + m0);
    uint4 qn[kPF];
    uint2 sn[kPF];
    if (active_wave) {
#pragma unroll
      for (int u = 0; u < kPF; ++u) {
        if (u < nc) {
          qn[u] = qblk[static_cast<size_t>(u) * 64 + lane];
          sn[u] = *reinterpret_cast<const uint2*>(ssec + ((static_cast<uint64_t>(p) * ng + (64 * u) / G) * 16 + n) * 8);
        }
      }
    }
    f32x4_t acca = {0, 0, 0, 0}, accb = {0, 0, 0, 0};
    f32x4_t bsa = {0, 0, 0, 0}, bsb = {0, 0, 0, 0};
    for (int k0 = 0; k0 < I; k0 += kStageColsD) {
      const int kr = min(kStageColsD, I - k0);
      const int upr = kr / 8;
      __syncthreads();
      for (int op = wave; op * 64 < kSub * upr; op += 4) {
        const int u = op * 64 + lane;
        const int m = u / upr, ph = u - m * upr;
        if (m < mc) {
          const int u8 = ph ^ (m & 7);
          const size_t src = (row0 + m) * a.hstride + k0 + 8 * u8;
          dma16(h_hi + src, &hsh[op * 64 * 8]);
          dma16(h_lo + src, &hsl[op * 64 * 8]);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);  // this wave's direct-to-LDS loads have landed
      __syncthreads();
      const int gpr = kr / G;
      for (int idx = tid; idx < kSub * gpr; idx += 256) {
        const int m = idx / gpr, g = idx - m * gpr;
        float s = 0.0f;
        if (m < mc) {
          for (int c8 = 0; c8 < G / 8; ++c8) {
            const int pos = unit_pos(m, g * (G / 8) + c8, upr) * 8;
            const uint4 vh = *reinterpret_cast<const uint4*>(&hsh[pos]);
            const uint4 vl = *reinterpret_cast<const uint4*>(&hsl[pos]);
            const uint32_t wh[4] = {vh.x, vh.y, vh.z, vh.w}, wl[4] = {vl.x, vl.y, vl.z, vl.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
              s += (bf16_bits_to_f32(wh[i] & 0xFFFFu) + bf16_bits_to_f32(wl[i] & 0xFFFFu)) +
                   (bf16_bits_to_f32(wh[i] >> 16) + bf16_bits_to_f32(wl[i] >> 16));
          }
        }
        gsum[m][g] = s;
      }
      __syncthreads();
      if (!active_wave) continue;
      for (int g0 = 0; g0 < gpr; g0 += 32) {
        uint4 sh, sl, bah, bal, bbh, bbl;
        sum_operands(&gsum[0][0], kStageColsD / 32 + 1, gpr, g0, n, kb, sh, sl);
        bias_operands(ssec, p, ng, k0 / G + g0, n, kb, bah, bal, bbh, bbl);
        bsa = bias_mfma(sh, sl, bah, bal, bsa);
        bsb = bias_mfma(sh, sl, bbh, bbl, bsb);
      }
      f32x4_t pa = {0, 0, 0, 0}, pb = {0, 0, 0, 0};
      const int c_lo = k0 / 64, c_hi = (k0 + kr) / 64;
#pragma unroll
      for (int ci = 0; ci < kStageColsD / 64; ++ci) {
        {
          const int u = ci % kPF;
          const int c = c_lo + ci;
          const uint4 q = qn[u];
          const uint2 sr = sn[u];
          const uint4 ba0 = word_operand<2>(q.x), ba1 = word_operand<2>(q.y);
          const uint4 bb0 = word_operand<2>(q.z), bb1 = word_operand<2>(q.w);
          const float sa = f16_bits_to_f32(sr.x & 0xFFFFu), sb = f16_bits_to_f32(sr.y & 0xFFFFu);
          if (nc > kPF) {  // refills only when the expert has more chunks than slots
            const int cn = min(c + kPF, nc - 1);
            qn[u] = qblk[static_cast<size_t>(cn) * 64 + lane];
            sn[u] = *reinterpret_cast<const uint2*>(
                ssec + ((static_cast<uint64_t>(p) * ng + (64 * cn) / G) * 16 + n) * 8);
          }
          if (c < c_hi) {
            const int u8 = (c * 64 - k0) / 8 + kb;
            const int p0 = unit_pos(n, u8, upr) * 8, p1 = unit_pos(n, u8 + 4, upr) * 8;
            const uint4 h0 = *reinterpret_cast<const uint4*>(&hsh[p0]);
            const uint4 h1 = *reinterpret_cast<const uint4*>(&hsh[p1]);
            const uint4 l0 = *reinterpret_cast<const uint4*>(&hsl[p0]);
            const uint4 l1 = *reinterpret_cast<const uint4*>(&hsl[p1]);
            if constexpr (G == 32) {
              const uint2 sr1 = *reinterpret_cast<const uint2*>(
                  ssec + ((static_cast<uint64_t>(p) * ng + 2 * c + 1) * 16 + n) * 8);
              const float sa1 = f16_bits_to_f32(sr1.x & 0xFFFFu), sb1 = f16_bits_to_f32(sr1.y & 0xFFFFu);
              const f32x4_t z = {0, 0, 0, 0};
              const f32x4_t x0 = mfma<2>(l0, ba0, mfma<2>(h0, ba0, z));
              const f32x4_t y0 = mfma<2>(l0, bb0, mfma<2>(h0, bb0, z));
              const f32x4_t x1 = mfma<2>(l1, ba1, mfma<2>(h1, ba1, z));
              const f32x4_t y1 = mfma<2>(l1, bb1, mfma<2>(h1, bb1, z));
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                acca[i] = fmaf(sa, x0[i], acca[i]);
                accb[i] = fmaf(sb, y0[i], accb[i]);
                acca[i] = fmaf(sa1, x1[i], acca[i]);
                accb[i] = fmaf(sb1, y1[i], accb[i]);
              }
            } else {
              pa = mfma<2>(h0, ba0, pa);
              pa = mfma<2>(l0, ba0, pa);
              pb = mfma<2>(h0, bb0, pb);
              pb = mfma<2>(l0, bb0, pb);
              pa = mfma<2>(h1, ba1, pa);
              pa = mfma<2>(l1, ba1, pa);
              pb = mfma<2>(h1, bb1, pb);
              pb = mfma<2>(l1, bb1, pb);
              if (G == 64 || (c & 1)) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  acca[i] = fmaf(sa, pa[i], acca[i]);
                  accb[i] = fmaf(sb, pb[i], accb[i]);
                }
                pa = f32x4_t{0, 0, 0, 0};
                pb = f32x4_t{0, 0, 0, 0};
              }
            }
          }
        }
      }
    }
    if (active_wave) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * kb + i;
        if (m < mc) {
          float* yr = a.yrow + (row0 + m) * H + 32 * p;
          yr[n] = fmaf(16.0f, acca[i], bsa[i]);
          yr[16 + n] = fmaf(16.0f, accb[i], bsb[i]);
        }
      }
    }
  }
}

static int ids_upper(int units_upper, int S) { return ((units_upper + 7) / 8) * 8 * S; }
static int grid_for(int ids, int cap) { return ids < cap ? (ids > 0 ? ids : 1) : cap; }

hipError_t launch_gateup_grouped(int act, const FfnArgs& a, hipStream_t s) {
  const int n_act_max = (a.T * a.K < a.E) ? a.T * a.K : a.E;
  const int S = (a.T + kSub - 1) / kSub;
  const int grid = grid_for(ids_upper(n_act_max * (a.I / 64) + a.Is / 64, S), kMaxGridGU);
#define GU_LAUNCH(A_, G_) hipLaunchKernelGGL((k_gateup_grouped<A_, G_>), dim3(grid), dim3(256), 0, s, a, S)
  if (act == 2) {
    if (a.G == 32) GU_LAUNCH(2, 32);
    else if (a.G == 64) GU_LAUNCH(2, 64);
    else GU_LAUNCH(2, 128);
  } else {
    if (a.G == 32) GU_LAUNCH(1, 32);
    else if (a.G == 64) GU_LAUNCH(1, 64);
    else GU_LAUNCH(1, 128);
  }
#undef GU_LAUNCH
  return hipGetLastError();
}

hipError_t launch_down_grouped(const FfnArgs& a, hipStream_t s) {
  const int n_act_max = (a.T * a.K < a.E) ? a.T * a.K : a.E;
  const int nb = (a.H + 127) / 128;
  const int S = (a.T + kSub - 1) / kSub;
  const int grid = grid_for(ids_upper(n_act_max * nb + (a.Is > 0 ? nb : 0), S), kMaxGridD);
  if (a.G == 32) hipLaunchKernelGGL((k_down_grouped<32>), dim3(grid), dim3(256), 0, s, a, S);
  else if (a.G == 64) hipLaunchKernelGGL((k_down_grouped<64>), dim3(grid), dim3(256), 0, s, a, S);
  else hipLaunchKernelGGL((k_down_grouped<128>), dim3(grid), dim3(256), 0, s, a, S);
  return hipGetLastError();
}

}  // namespace moe
