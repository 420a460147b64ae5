// Batched grouped-GEMM family on the gfx950 matrix cores.
//
// When a batch routes many tokens to the same experts, each expert's weights
// are streamed once per run of up to 16 of its token rows (a *unit*, built by
// the bucketing kernel) and multiplied on the matrix cores with
// v_mfma_f32_16x16x32_f16: A = the unit's activations, B = the weights.
//
// Work split.  A unit's output is cut into pair-tiles (gate/up: 16 rows of
// gate plus the same 16 rows of up; down: 32 rows of the output).  All
// pair-tiles of all units form one list, and workgroup w (one per CU) takes
// the contiguous range [w L / W, (w+1) L / W) of it, so every CU streams the
// same number of weight bytes.  Logical workgroup indices are assigned so that
// consecutive ranges (the tiles of one unit, and the units of one expert) run
// on one XCD and share its L2.  Inside a workgroup the reduction dimension is
// split across waves (gate/up: 8 waves take every 8th 64-column chunk of one
// pair-tile; down: 4 pair-tiles at a time, 2 waves each), and the partial
// tiles are summed through LDS in a fixed order.
//
// Weight stream.  Each wave keeps the chunks of the next kDepth tiles in
// flight in register slots: the slot of a chunk is refilled (with the same
// chunk of the tile kDepth steps ahead) as soon as it has been decoded, so the
// loads never wait for the products and never cross a barrier.
//
// Operands.  A nibble q becomes an fp16 operand with a single mask: the
// blob word keeps values 2m, 2m+1 of a 16-byte lane group in nibbles m and
// m + 4, so w & 0x000F000F and (w >> 8) & 0x000F000F are two fp16 subnormals
// q * 2^-24 (values 0, 1 and 4, 5) and w & 0x00F000F0, (w >> 8) & 0x00F000F0
// are q * 2^-20 (values 2, 3 and 6, 7).  The matrix cores take fp16
// subnormal inputs exactly, so the activations at the second kind of
// position are given scaled by 1/16 and every product is q * x * 2^-24,
// exact in fp32.  The affine group dequantisation is applied in fp32:
//     sum_c (s q_c + b) x_c = s * 2^24 * P + b * sum_c x_c,
// with the column sums of the unit's activations computed once per unit.
// Activations become fp16 (bf16 inputs are exact in fp16 within its range;
// the grouped family needs |x| and |h| to round below 65520, and the gate/up
// kernel reports any value that does not in the call's status word); the
// SwiGLU output h enters the down projection as fp16 (11 significant bits,
// one rounding of the fp32 h), written operand-ready by the gate/up kernel
// together with the fp32 sums of those fp16 values over 16-column blocks for
// the down kernel's bias term.
//
// int8 experts (BITS = 8) use the same stream with two 16-byte loads per lane
// and chunk (the tile A and tile B planes of the blob).  A byte q becomes
// the fp16 subnormal q * 2^-24 with the same kind of mask: w & 0x00FF00FF and
// (w >> 8) & 0x00FF00FF hold values (0, 2) and (1, 3) of a word, so the A
// operand is packed in that order, (x0, x2, x1, x3, x4, x6, x5, x7), and
// unscaled; the gate/up epilogue stores h with the columns of every 4 in
// the order (0, 2, 1, 3) for the down projection.
//
// Operand layout of v_mfma_f32_16x16x32 (64 lanes, lane l: n = l % 16,
// kb = l / 16): A lane holds row m = n, k = 8kb..8kb+7; B lane holds column n,
// k = 8kb..8kb+7; C lane holds rows 4kb..4kb+3 of column n.  The expert blob
// stores each lane's B values contiguously (see the public header), so one
// 16-byte load per lane fetches the B operands of two 16-row tiles for a
// 64-column chunk.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int kSub = kSubTokens;
constexpr int kWaves = 8;              // waves per workgroup (both kernels)
constexpr int kSlot = 4;               // weight chunks per wave and tile step
constexpr float kQScale = 16777216.0f; // 2^24: products are q * x * 2^-24

__device__ __forceinline__ f32x4_t mfma(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0,
                                                0, 0);
}

// B operand of one blob word (8 values): fp16 subnormals, see above.
__device__ __forceinline__ uint4 word_operand(uint32_t w) {
  const uint32_t t = w >> 8;
  return make_uint4(w & 0x000F000Fu, w & 0x00F000F0u, t & 0x000F000Fu, t & 0x00F000F0u);
}
// B operand of 8 int8 values (bytes 0..3 of lo, then of hi): halves
// (v0, v2), (v1, v3), (v4, v6), (v5, v7) as q * 2^-24.
__device__ __forceinline__ uint4 byte_operand(uint32_t lo, uint32_t hi) {
  return make_uint4(lo & 0x00FF00FFu, (lo >> 8) & 0x00FF00FFu, hi & 0x00FF00FFu, (hi >> 8) & 0x00FF00FFu);
}
// Storage column of column c of h for the int8 down projection: within every
// group of 4 the order (0, 2, 1, 3).
__device__ __forceinline__ int h8_col(int c) { return (c & ~3) | ((c & 1) << 1) | ((c >> 1) & 1); }

__device__ __forceinline__ uint32_t f32_to_f16_bits(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}
__device__ __forceinline__ float f16_bits_f32(uint32_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
}

// Nonzero when either fp16 half of w is an infinity or a NaN (exponent bits
// all ones): the value did not fit the fp16 operand.
__device__ __forceinline__ uint32_t f16x2_nonfinite(uint32_t w) {
  const uint32_t e = w & 0x7C007C00u;
  return static_cast<uint32_t>((e & 0xFFFFu) == 0x7C00u) | static_cast<uint32_t>((e >> 16) == 0x7C00u);
}

// A operand from 8 activations (16 bytes, value j at half j): fp16; int4:
// values 2, 3, 6, 7 scaled by 1/16; int8: unscaled, in the order 0, 2, 1, 3,
// 4, 6, 5, 7.  Adds the 8 activations to sum; sets bad when one of them is
// outside the fp16 range.
template <int ACT, int BITS = 4>
__device__ __forceinline__ uint4 act_operand(uint4 raw, float& sum, uint32_t& bad) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t o[4];
  if constexpr (BITS == 8) {
    float v[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      v[2 * d] = act_to_f32<ACT>(w[d] & 0xFFFFu);
      v[2 * d + 1] = act_to_f32<ACT>(w[d] >> 16);
      sum += v[2 * d] + v[2 * d + 1];
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      o[2 * p] = f32_to_f16_bits(v[4 * p]) | (f32_to_f16_bits(v[4 * p + 2]) << 16);
      o[2 * p + 1] = f32_to_f16_bits(v[4 * p + 1]) | (f32_to_f16_bits(v[4 * p + 3]) << 16);
    }
  } else {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float v0 = act_to_f32<ACT>(w[d] & 0xFFFFu), v1 = act_to_f32<ACT>(w[d] >> 16);
      sum += v0 + v1;
      const float f = (d & 1) ? 0.0625f : 1.0f;
      o[d] = f32_to_f16_bits(v0 * f) | (f32_to_f16_bits(v1 * f) << 16);
    }
  }
  bad |= f16x2_nonfinite(o[0]) | f16x2_nonfinite(o[1]) | f16x2_nonfinite(o[2]) | f16x2_nonfinite(o[3]);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Wave-uniform read of memory that no kernel of the launch writes (unit
// records, counts, expert offsets): through the constant address space, so
// the compiler uses scalar loads, which do not enter the vector-memory
// counter that orders the weight stream.
template <class T>
__device__ __forceinline__ T load_uniform(const T* p) {
  return *reinterpret_cast<const __attribute__((address_space(4))) T*>(
      reinterpret_cast<const __attribute__((address_space(4))) char*>(reinterpret_cast<uintptr_t>(p)));
}

template <int V>
struct Half {
  static constexpr int value = V;
};

struct UnitHdr {
  int row0, mc, expert;
};
__device__ __forceinline__ UnitHdr unit_hdr(const int32_t* units, int u) {
  const int32_t* r = units + static_cast<size_t>(u) * kUnitInts;
  return UnitHdr{load_uniform(r), load_uniform(r + 1), load_uniform(r + 2)};
}

__device__ __forceinline__ const uint8_t* expert_blob(const FfnArgs& a, int expert) {
  return expert < 0 ? a.shared
                    : a.experts + (a.offsets ? load_uniform(a.offsets + expert) : static_cast<uint64_t>(expert) * a.stride);
}

// Logical index of this workgroup: consecutive logical indices share an XCD
// (hardware assigns workgroups to the 8 XCDs round-robin).
__device__ __forceinline__ int logical_wg() {
  const int W = gridDim.x;
  return (blockIdx.x & 7) * (W >> 3) + (blockIdx.x >> 3);
}

// One slot of the weight stream: 16 bytes of nibbles (int8: 16 bytes of each
// tile plane) and the fp16 (s, b) pairs of the chunk's group(s) for the
// lane's row n of both tiles.
struct Slot {
  uint4 q, q2;    // q2: tile B plane (int8 only)
  uint2 s0, s1;   // s1: second group of the chunk (G = 32 only)
};
// vector-memory loads of one slot (the down kernel's staged barrier counts them)
template <int G, int BITS>
constexpr int kLoadsPerSlot = BITS / 4 + (G == 32 ? 2 : 1);
template <int G, int BITS = 4>
__device__ __forceinline__ void load_slot(Slot& sl, const uint4* qb, const uint8_t* sb, int c) {
  if constexpr (BITS == 8) {
    sl.q = qb[static_cast<size_t>(2 * c) * 64];
    sl.q2 = qb[static_cast<size_t>(2 * c + 1) * 64];
  } else {
    sl.q = qb[static_cast<size_t>(c) * 64];
  }
  if constexpr (G == 32) {
    sl.s0 = *reinterpret_cast<const uint2*>(sb + static_cast<size_t>(2 * c) * 128);
    sl.s1 = *reinterpret_cast<const uint2*>(sb + static_cast<size_t>(2 * c + 1) * 128);
  } else {
    sl.s0 = *reinterpret_cast<const uint2*>(sb + static_cast<size_t>((64 * c) / G) * 128);
  }
}

// Pins a value as computed at this point: the compiler may not move its
// computation below a later memory access.  Used to make sure a weight slot is
// fully decoded before its refill is issued, so that the refill lands in the
// same registers (no copies, no early waits on the refill).
__device__ __forceinline__ void pin(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w) : : "memory");
}
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v) : : "memory"); }



// Decoded slot: B operands of both tiles for both 32-column halves, scales
// and biases (per half; equal unless G = 32).
struct Decoded {
  uint4 bA0, bA1, bB0, bB1;
  float sA0, sB0, sA1, sB1;
  float cA0, cB0, cA1, cB1;
};
template <int G, int BITS = 4>
__device__ __forceinline__ Decoded decode_slot(const Slot& sl) {
  Decoded d;
  if constexpr (BITS == 8) {
    d.bA0 = byte_operand(sl.q.x, sl.q.y);
    d.bA1 = byte_operand(sl.q.z, sl.q.w);
    d.bB0 = byte_operand(sl.q2.x, sl.q2.y);
    d.bB1 = byte_operand(sl.q2.z, sl.q2.w);
  } else {
    d.bA0 = word_operand(sl.q.x);
    d.bA1 = word_operand(sl.q.y);
    d.bB0 = word_operand(sl.q.z);
    d.bB1 = word_operand(sl.q.w);
  }
  d.sA0 = f16_bits_to_f32(sl.s0.x & 0xFFFFu);
  d.sB0 = f16_bits_to_f32(sl.s0.y & 0xFFFFu);
  d.cA0 = f16_bits_to_f32(sl.s0.x >> 16);
  d.cB0 = f16_bits_to_f32(sl.s0.y >> 16);
  if constexpr (G == 32) {
    d.sA1 = f16_bits_to_f32(sl.s1.x & 0xFFFFu);
    d.sB1 = f16_bits_to_f32(sl.s1.y & 0xFFFFu);
    d.cA1 = f16_bits_to_f32(sl.s1.x >> 16);
    d.cB1 = f16_bits_to_f32(sl.s1.y >> 16);
  } else {
    d.sA1 = d.sA0;
    d.sB1 = d.sB0;
    d.cA1 = d.cA0;
    d.cB1 = d.cB0;
  }
  pin(d.bA0);
  pin(d.bA1);
  pin(d.bB0);
  pin(d.bB1);
  pin(d.sA0);
  pin(d.sB0);
  pin(d.cA0);
  pin(d.cB0);
  if constexpr (G == 32) {
    pin(d.sA1);
    pin(d.sB1);
    pin(d.cA1);
    pin(d.cB1);
  }
  return d;
}

// Products of one chunk: P = A . B for both tiles (per 32-column half when
// the halves belong to different groups).  With DUAL the A operand is a hi +
// lo pair (a0 + l0, a1 + l1), both multiplied.
struct Prod {
  f32x4_t pA0, pB0, pA1, pB1;   // pA1, pB1: second half (G = 32 only)
};
template <int G, bool DUAL>
__device__ __forceinline__ Prod chunk_mfma(const Decoded& d, uint4 a0, uint4 a1, uint4 l0, uint4 l1) {
  const f32x4_t z = {0, 0, 0, 0};
  Prod p;
  if constexpr (G == 32) {
    p.pA0 = mfma(a0, d.bA0, z);
    p.pB0 = mfma(a0, d.bB0, z);
    p.pA1 = mfma(a1, d.bA1, z);
    p.pB1 = mfma(a1, d.bB1, z);
    if constexpr (DUAL) {
      p.pA0 = mfma(l0, d.bA0, p.pA0);
      p.pB0 = mfma(l0, d.bB0, p.pB0);
      p.pA1 = mfma(l1, d.bA1, p.pA1);
      p.pB1 = mfma(l1, d.bB1, p.pB1);
    }
  } else {
    p.pA0 = mfma(a0, d.bA0, z);
    p.pB0 = mfma(a0, d.bB0, z);
    if constexpr (DUAL) {
      p.pA0 = mfma(l0, d.bA0, p.pA0);
      p.pB0 = mfma(l0, d.bB0, p.pB0);
    }
    p.pA0 = mfma(a1, d.bA1, p.pA0);
    p.pB0 = mfma(a1, d.bB1, p.pB0);
    if constexpr (DUAL) {
      p.pA0 = mfma(l1, d.bA1, p.pA0);
      p.pB0 = mfma(l1, d.bB1, p.pB0);
    }
  }
  return p;
}

// Scale and bias of one chunk: acc += s * P, bias += b * colsum.  cs0, cs1:
// column sums of the two halves for the lane's 4 output rows (tokens).
struct Coef {
  float sA0, sB0, cA0, cB0, sA1, sB1, cA1, cB1;
};
__device__ __forceinline__ Coef coef_of(const Decoded& d) {
  return Coef{d.sA0, d.sB0, d.cA0, d.cB0, d.sA1, d.sB1, d.cA1, d.cB1};
}
template <int G>
__device__ __forceinline__ void chunk_scale(const Prod& p, const Coef& k, const float* cs0, const float* cs1,
                                            f32x4_t& accA, f32x4_t& accB, f32x4_t& biasA, f32x4_t& biasB) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (G == 32) {
      accA[i] = fmaf(k.sA1, p.pA1[i], fmaf(k.sA0, p.pA0[i], accA[i]));
      accB[i] = fmaf(k.sB1, p.pB1[i], fmaf(k.sB0, p.pB0[i], accB[i]));
      biasA[i] = fmaf(k.cA1, cs1[i], fmaf(k.cA0, cs0[i], biasA[i]));
      biasB[i] = fmaf(k.cB1, cs1[i], fmaf(k.cB0, cs0[i], biasB[i]));
    } else {
      accA[i] = fmaf(k.sA0, p.pA0[i], accA[i]);
      accB[i] = fmaf(k.sB0, p.pB0[i], accB[i]);
      biasA[i] = fmaf(k.cA0, cs0[i], biasA[i]);
      biasB[i] = fmaf(k.cB0, cs0[i], biasB[i]);
    }
  }
}

// 16-byte global -> LDS copy by the active lanes of a wave; lane i writes
// 16 bytes at lds_base + 16 i (lds_base is wave-uniform).
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_ptr)(lds_base), 16, 0, 0);
}

// Staged tile of 16 rows: 16-byte unit (m, u8) (columns 8*u8..8*u8+7 of row m)
// sits at m*upr + (u8 ^ (m & 7)), so the 16 lanes reading one column block of
// the 16 rows hit different banks.
__device__ __forceinline__ int unit_pos(int m, int u8, int upr) { return m * upr + (u8 ^ (m & 7)); }

// Stages rows m < mc of a 16-row activation tile (row m = src + off[m] * pitch,
// width `cols` 16-bit values) into LDS at lds, in the swizzled unit layout.
// All threads of the workgroup call it; the caller waits and synchronises.
__device__ __forceinline__ void stage_rows(const uint16_t* src, const int* off, int mc, size_t pitch, int cols,
                                           uint16_t* lds, int wave, int lane) {
  const int upr = cols / 8;
  for (int op = wave; op * 64 < kSub * upr; op += kWaves) {
    const int u = op * 64 + lane;
    const int m = u / upr, ph = u - m * upr;
    if (m < mc) dma16(src + static_cast<size_t>(off[m]) * pitch + 8 * (ph ^ (m & 7)), &lds[op * 64 * 8]);
  }
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (gfx9 encoding; lgkm and export counts untouched).
constexpr int vmcnt_imm(int n) { return ((n >> 4) << 14) | (0xF << 8) | (0x7 << 4) | (n & 0xF); }
constexpr int kLgkm0 = (3 << 14) | (0x7 << 4) | 0xF;   // lgkmcnt(0) only

// Workgroup barrier after this wave's direct-to-LDS loads issued before the
// last `after` vector-memory operations have landed.  Unlike __syncthreads(),
// whose fence waits for every outstanding load, it leaves the newest `after`
// loads (the weight prefetch) in flight.
template <int after>
__device__ __forceinline__ void staged_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(after));
  __builtin_amdgcn_s_waitcnt(kLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


// ---------------------------------------------------------------------------
// gate/up + SwiGLU.  Tile = gate/up pair-tile pt of a unit (16 rows of gate
// and of up for the unit's <= 16 tokens, full hidden width); wave w takes the
// chunks c_j = w + 8 j (j < 4).  Each wave holds the A operands of its own
// chunks for the current unit in registers (no LDS staging), and loads the
// next unit's activations as soon as its weight stream reaches that unit.
// Output: h as fp16, operand-ready for the down projection (columns with
// (col & 2) != 0 scaled by 1/16), at rows row0.., columns 16 pt.., and
// hsum[row][pt] = sum over the 16 columns of those fp16 values (unscaled).
// FULL: H is the family's largest (2048, 32 chunks), so every chunk w + 8 j
// a wave forms is in range and the product loop carries no range tests.
// ---------------------------------------------------------------------------
template <int ACT, int G, int BITS, bool FULL, int NW>
__global__ __launch_bounds__(64 * NW) void k_gateup_tiles(FfnArgs a) {
  // NW waves split each tile's chunks: NW = 8 takes 4 chunks per wave and
  // tile (two waves per SIMD), NW = 16 takes 2 (four waves per SIMD, half the
  // registers per wave)
  constexpr int kWaves = NW;
  constexpr int kSlot = 32 / NW;
  constexpr int NQ = BITS / 4;   // 16-byte weight loads per lane and chunk
  // tiles are processed in pairs (one barrier per pair); the two tiles of a
  // pair use the two slot groups, so kDepth = 2 tiles are in flight per wave
  constexpr int kDepth = 2;
  constexpr int kHalves = G == 32 ? 2 : 1;  // groups per chunk
  // partial tiles of a pair: buffer, tile, wave, gate / up, row e, lane.  The
  // row stride of 80 floats puts rows e and e + 1 on opposite bank halves, so
  // the reduction reads (64 lanes: 4 rows x 16 consecutive lanes) take the
  // minimum two LDS cycles; with 16 waves the stride is 72 (two-way
  // conflicts) so that the partials fit the 160 KB of LDS.
  constexpr int kRowStride = NW == 8 ? 80 : 72;
  __shared__ float red[2][2][kWaves][2][4][kRowStride];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kb = lane >> 4;
  const int H = a.H, nc = H / 64, ng = H / G;
  const int n_su = load_uniform(a.n_units), n_ru = load_uniform(a.n_units + 1);
  const int nts = a.Is / 16, ntr = a.I / 16;
  const int L = n_su * nts + n_ru * ntr, lw = logical_wg();
  const int t0 = static_cast<int>((static_cast<long long>(lw) * L) >> kGridTilesLog2);
  const int t1 = static_cast<int>((static_cast<long long>(lw + 1) * L) >> kGridTilesLog2);
  if (t0 >= t1) return;
  uint16_t* h16 = reinterpret_cast<uint16_t*>(a.h);
  const int hs_stride = a.hstride / 16;
  // tile cursor: (unit, pair-tile); units before n_su have nts tiles, the rest ntr
  struct Cursor {
    int u, pt;
  };
  auto locate = [&](int t) -> Cursor {
    const int tsh = n_su * nts;
    if (t < tsh) return Cursor{t / nts, t % nts};
    return Cursor{n_su + (t - tsh) / ntr, (t - tsh) % ntr};
  };
  auto advance = [&](Cursor& cr) {
    if (++cr.pt == (cr.u < n_su ? nts : ntr)) {
      ++cr.u;
      cr.pt = 0;
    }
  };
  // ---- activations: raw prefetch (xr) of unit pu, operands (xa) of unit xu
  uint4 xr[kSlot][2];   // raw activations of the prefetched unit
  uint4 xa[kSlot][2];   // A operands of the current unit (this wave's chunks)
  // column sums for the lane's output rows 4kb..4kb+3: in registers, or for
  // group 32 (two groups per chunk, the register-heaviest case) in this
  // wave's part of LDS, read back per chunk
  constexpr bool kSumsInLds = G == 32;
  float csv[kSumsInLds ? 1 : kSlot][kHalves][4];
  __shared__ __attribute__((aligned(16))) float csl[kSumsInLds ? kWaves : 1][kSlot][kHalves][kSub];
  auto sums_of = [&](int j, int hh, float* out) {
    if constexpr (kSumsInLds) {
      const float4 v = *reinterpret_cast<const float4*>(&csl[wave][j][hh][4 * kb]);
      out[0] = v.x;
      out[1] = v.y;
      out[2] = v.z;
      out[3] = v.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = csv[j][hh][i];
    }
  };
  int pu = -1, prow0 = 0, pmc = 0;
  int xu = -1, row0 = 0, mc = 0;
  // issue the activation loads of unit u (record rec) into xr
  auto prefetch_x = [&](int u, const int32_t* rec) {
    const int r0 = load_uniform(rec), m_c = load_uniform(rec + 1);
    int tk = load_uniform(rec + 4);   // lanes beyond the unit's rows read row 0 (unused)
#pragma unroll
    for (int i = 1; i < kSub; ++i) {
      const int ti = load_uniform(rec + 4 + i);
      tk = (n == i && i < m_c) ? ti : tk;
    }
    const uint16_t* xrow = a.x + static_cast<size_t>(tk) * H + 8 * kb;
#pragma unroll
    for (int j = 0; j < kSlot; ++j) {
      const int c = min(wave + kWaves * j, nc - 1);
      xr[j][0] = *reinterpret_cast<const uint4*>(xrow + 64 * c);
      xr[j][1] = *reinterpret_cast<const uint4*>(xrow + 64 * c + 32);
    }
    pu = u;
    prow0 = r0;
    pmc = m_c;
  };
  // xr -> A operands and the column sums (32-column halves) for the C
  // layout rows
  auto take_x = [&]() {
    uint32_t bad = 0;
#pragma unroll
    for (int j = 0; j < kSlot; ++j) {
      float s0 = 0.0f, s1 = 0.0f;
      xa[j][0] = act_operand<ACT, BITS>(xr[j][0], s0, bad);
      xa[j][1] = act_operand<ACT, BITS>(xr[j][1], s1, bad);
      float hs[kHalves];
      if constexpr (G == 32) {
        hs[0] = s0;
        hs[1] = s1;
      } else {
        hs[0] = s0 + s1;
      }
#pragma unroll
      for (int hh = 0; hh < kHalves; ++hh) {
        // sum over the 4 lane rows (kb) holding token n, then fetch the sums of
        // tokens 4kb..4kb+3 (the rows of this lane's accumulator)
        uint32_t v = __float_as_uint(hs[hh]);
        const auto p16 = __builtin_amdgcn_permlane16_swap(static_cast<int>(v), static_cast<int>(v), false, false);
        v = __float_as_uint(__uint_as_float(static_cast<uint32_t>(p16[0])) + __uint_as_float(static_cast<uint32_t>(p16[1])));
        const auto p32 = __builtin_amdgcn_permlane32_swap(static_cast<int>(v), static_cast<int>(v), false, false);
        v = __float_as_uint(__uint_as_float(static_cast<uint32_t>(p32[0])) + __uint_as_float(static_cast<uint32_t>(p32[1])));
        if constexpr (kSumsInLds) {
          if (kb == 0) csl[wave][j][hh][n] = __uint_as_float(v);   // token n (lanes kb > 0 hold the same)
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            csv[j][hh][i] = __uint_as_float(static_cast<uint32_t>(__shfl(static_cast<int>(v), 4 * kb + i, kWave)));
        }
      }
    }
    if (bad) atomicOr(a.status, kStatusF16Range);
    xu = pu;
    row0 = prow0;
    mc = pmc;
    pu = -1;
  };
  // ---- weight stream: the refill cursor runs kDepth tiles ahead (clamped to
  // the last tile); the unit's expert is looked up only when the unit
  // changes, and a new unit's activations are fetched right away when the
  // raw buffer is free, else after the current unit's are taken
  int su = -1;
  const uint8_t* sblob = nullptr;
  int sI = 0;
  int want = -1;   // unit whose activations still have to be fetched
  auto tile_src = [&](const Cursor cr, const uint4*& qb, const uint8_t*& sb) {
    if (cr.u != su) {
      const int32_t* rec = a.units + static_cast<size_t>(cr.u) * kUnitInts;
      const int ex = load_uniform(rec + 2);
      su = cr.u;
      sblob = expert_blob(a, ex);
      sI = ex < 0 ? a.Is : a.I;
      if (cr.u != xu && cr.u != pu) {
        if (pu < 0) prefetch_x(cr.u, rec);
        else want = cr.u;
      }
    }
    qb = reinterpret_cast<const uint4*>(sblob) + static_cast<size_t>(cr.pt) * nc * 64 * NQ + lane;
    sb = sblob + blob_gu_s(H, sI, BITS) + (static_cast<size_t>(cr.pt) * ng * 16 + n) * 8;
  };
  Cursor cc = locate(t0);   // compute cursor (tile t)
  Cursor rc = cc;           // refill cursor (tile min(t + kDepth, t1 - 1))
  int rt = t0;
  // first unit: activations first, then the weights of the first kDepth tiles
  prefetch_x(cc.u, a.units + static_cast<size_t>(cc.u) * kUnitInts);
  Slot sl[kDepth * kSlot];
#pragma unroll
  for (int hf = 0; hf < kDepth; ++hf) {
    const uint4* qb;
    const uint8_t* sb;
    tile_src(rc, qb, sb);
#pragma unroll
    for (int j = 0; j < kSlot; ++j) load_slot<G, BITS>(sl[hf * kSlot + j], qb, sb, min(wave + kWaves * j, nc - 1));
    if (rt + 1 < t1) {
      ++rt;
      advance(rc);
    }
  }
  // chunk products of tile t (slot group hf) -> this wave's partial in
  // red[pb][hf]; returns the tile's rows and pair-tile for the reduction
  struct TileOut {
    int row0, mc, pt;
  };
  auto compute = [&](const int t, auto hfc, const int pb) -> TileOut {
    constexpr int hf = decltype(hfc)::value;
    if (cc.u != xu) {
      take_x();
      if (want >= 0) {
        prefetch_x(want, a.units + static_cast<size_t>(want) * kUnitInts);
        want = -1;
      }
    }
    const TileOut out{row0, mc, cc.pt};
    // refill source: tile t + kDepth (the last tile again near the end; unused)
    const uint4* qnx;
    const uint8_t* snx;
    tile_src(rc, qnx, snx);
    if (rt + 1 < t1) {
      ++rt;
      advance(rc);
    }
    f32x4_t accA = {0, 0, 0, 0}, accB = {0, 0, 0, 0}, biasA = {0, 0, 0, 0}, biasB = {0, 0, 0, 0};
    // the scale of chunk j is applied after the products of chunk j + 1 are
    // issued, so that the matrix-core latency is covered
    Prod pp;
    Coef pk;
#pragma unroll
    for (int j = 0; j < kSlot; ++j) {
      const int c = wave + kWaves * j;
      Slot& s = sl[hf * kSlot + j];
      const Decoded d = decode_slot<G, BITS>(s);
      load_slot<G, BITS>(s, qnx, snx, min(c, nc - 1));
      Prod p;
      if (FULL || c < nc) p = chunk_mfma<G, false>(d, xa[j][0], xa[j][1], xa[j][0], xa[j][1]);
      if (j > 0 && (FULL || c - kWaves < nc)) {
        float s0[4], s1[4];
        sums_of(j - 1, 0, s0);
        sums_of(j - 1, kHalves - 1, s1);
        chunk_scale<G>(pp, pk, s0, s1, accA, accB, biasA, biasB);
      }
      pp = p;
      pk = coef_of(d);
    }
    if (FULL || wave + kWaves * (kSlot - 1) < nc) {
      float s0[4], s1[4];
      sums_of(kSlot - 1, 0, s0);
      sums_of(kSlot - 1, kHalves - 1, s1);
      chunk_scale<G>(pp, pk, s0, s1, accA, accB, biasA, biasB);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      red[pb][hf][wave][0][i][lane] = fmaf(kQScale, accA[i], biasA[i]);
      red[pb][hf][wave][1][i][lane] = fmaf(kQScale, accB[i], biasB[i]);
    }
    advance(cc);
    return out;
  };
  // after the barrier: thread (tile tt, row m, column n) sums the wave
  // slices of gate and up in wave order and applies SwiGLU
  auto reduce = [&](const int pb, const TileOut& o0, const TileOut& o1, const int ntiles) {
    // int8: the thread's indices are formed here; hoisted to the kernel's
    // start they would stay live across the main loop and spill (int4 keeps
    // the compiler's placement, which does not spill)
    int tr = tid;
    if constexpr (BITS == 8) asm volatile("" : "+v"(tr));
    const int tt = tr >> 8, m = (tr >> 4) & 15, nn = tr & 15;
    if (tt < ntiles) {
      const TileOut& o = tt == 0 ? o0 : o1;
      const int src = nn + 16 * (m >> 2), e = m & 3;
      float ga = 0.0f, up = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        ga += red[pb][tt][w][0][e][src];
        up += red[pb][tt][w][1][e][src];
      }
      // silu(g) * u with the hardware exp2 and reciprocal (relative error a
      // few ulp, far inside the block's tolerance)
      const float hv = ga * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * ga)) * up;
      // operand-ready fp16 of h * f, f = 1/16 on the columns the down
      // projection's B operand carries as q * 2^-20 (column 16 pt + nn); int8:
      // f = 1, stored at the permuted column h8_col
      const bool sc = BITS == 4 && (nn & 2) != 0;
      const float hf_v = sc ? hv * 0.0625f : hv;
      const uint32_t hi = f32_to_f16_bits(hf_v);
      float hs = f16_bits_f32(hi);
      hs = sc ? hs * 16.0f : hs;
      // sum over the 16 columns of this row of the tile (one 16-lane DPP row)
      hs = __uint_as_float(dpp_row_sum(__float_as_uint(hs)));
      if (m < o.mc) {
        if ((hi & 0x7C00u) == 0x7C00u) atomicOr(a.status, kStatusF16Range);   // h outside the fp16 range
        const int col = BITS == 8 ? h8_col(nn) : nn;
        const size_t off = static_cast<size_t>(o.row0 + m) * a.hstride + 16 * o.pt + col;
        h16[off] = static_cast<uint16_t>(hi);
        if (nn == 0) a.hsum[static_cast<size_t>(o.row0 + m) * hs_stride + o.pt] = hs;
      }
    }
  };
  // pairs of tiles: both slot groups, one barrier, then the shared reduction
  // (buffers alternate, so the next pair's partials never overwrite a pair
  // that is still being reduced)
  int tb = t0, pb = 0;
  for (; tb + 2 <= t1; tb += 2, pb ^= 1) {
    const TileOut o0 = compute(tb, Half<0>{}, pb);
    const TileOut o1 = compute(tb + 1, Half<1>{}, pb);
    __syncthreads();
    reduce(pb, o0, o1, 2);
  }
  if (tb < t1) {
    const TileOut o0 = compute(tb, Half<0>{}, pb);
    __syncthreads();
    reduce(pb, o0, o0, 1);
  }
}

// ---------------------------------------------------------------------------
// down projection.  Tiles are down pair-tiles (32 output rows); a step takes 4
// consecutive tiles of one unit (quad), tile q4 = wave % 4, and the two waves
// w, w + 4 split the reduction (chunks w / 4 + 2 j).  h (operand-ready fp16)
// of the unit's rows is staged in LDS, in one of two buffers: a
// workgroup's range spans at most two units at the batch shapes, and both
// are staged before the first weight loads, so the switch to the second unit
// waits for nothing (a third unit, possible at other shapes, is staged at its
// switch).  The second wave's partial goes through LDS; the first adds it and
// stores yrow (unweighted, fp32).
// ---------------------------------------------------------------------------
template <int G, int BITS, bool FULL>
__global__ __launch_bounds__(512) void k_down_tiles(FfnArgs a) {
  constexpr int NQ = BITS / 4;   // 16-byte weight loads per lane and chunk
  // quads whose weights are in flight.  Two, not more: every workgroup
  // issues its first kDepth quads at once, and the memory system serves all
  // of them interleaved, so a workgroup's first quad is complete only when
  // nearly the whole chip-wide burst has arrived; a deeper start only delays
  // the first products (measured: first quad done at 8.3 us with 2 in
  // flight, 12 us with 4), while the steady state is paced by the products.
  constexpr int kDepth = 2;
  constexpr int kHalves = G == 32 ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint16_t hsh[2][kSub * kGroupedMaxInter];
  __shared__ float red[2][4][8][65];
  __shared__ __attribute__((aligned(16))) float cs[2][kGroupedMaxInter / 32][kSub];   // 32-column sums of h
  __shared__ int urow[2][kSub];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kb = lane >> 4;
  const int q4 = wave & 3, kh = wave >> 2;
  const int H = FULL ? kGroupedMaxH : a.H, n_pairs = H / 32;
  const int qpu = (n_pairs + 3) / 4;   // quads per unit
  // reduction width of a unit's expert (I or I_s)
  auto inter_of = [&](int expert) { return FULL ? kGroupedMaxInter : (expert < 0 ? a.Is : a.I); };
  const int n_units = load_uniform(a.n_units) + load_uniform(a.n_units + 1);
  const int Q = n_units * qpu, lw = logical_wg();
  const int s0 = static_cast<int>((static_cast<long long>(lw) * Q) >> kGridTilesLog2);
  const int s1 = static_cast<int>((static_cast<long long>(lw + 1) * Q) >> kGridTilesLog2);
  if (s0 >= s1) return;
  const uint16_t* h16 = reinterpret_cast<const uint16_t*>(a.h);
  const int hs_stride = a.hstride / 16;
  int xu = s0 / qpu;
  const UnitHdr hd0 = unit_hdr(a.units, xu);
  int row0 = hd0.row0, mc = hd0.mc;
  const int ex0 = hd0.expert;
  int su = xu;
  const uint8_t* sblob = expert_blob(a, ex0);
  int sI = inter_of(ex0);
  // weights of this wave's tile of quad q (pair-tile clamped to the last one)
  auto tile_src = [&](int q, const uint4*& qb, const uint8_t*& sb, int& ncq) {
    const int u = q / qpu;
    const int pt = FULL ? (q - u * qpu) * 4 + q4 : min((q - u * qpu) * 4 + q4, n_pairs - 1);
    if (u != su) {
      const UnitHdr hd = unit_hdr(a.units, u);
      su = u;
      sblob = expert_blob(a, hd.expert);
      sI = inter_of(hd.expert);
    }
    ncq = sI / 64;
    qb = reinterpret_cast<const uint4*>(sblob + blob_d_q(H, sI, BITS)) + static_cast<size_t>(pt) * ncq * 64 * NQ + lane;
    sb = sblob + blob_d_s(H, sI, G, BITS) + (static_cast<size_t>(pt) * (sI / G) * 16 + n) * 8;
  };
  // stage h of a unit's rows (direct-to-LDS) and fetch the sums of
  // h over 16-column blocks; the 32-column sums are stored afterwards, so
  // that loads issued in between stay in flight (kSub * inter / 32 <= 512:
  // one sum per thread)
  static_assert(kSub * (kGroupedMaxInter / 32) <= 512, "one column sum per thread");
  // urow[b] must hold the unit's rows (and be visible) before the call
  auto stage_issue = [&](int b, int r0, int mcu, int Iu, float& p0, float& p1) {
    stage_rows(h16, urow[b], mcu, a.hstride, Iu, hsh[b], wave, lane);
    const int m = tid & (kSub - 1), j = tid >> 4;
    p0 = p1 = 0.0f;
    if (j < Iu / 32 && m < mcu) {
      const float* hs = a.hsum + static_cast<size_t>(r0 + m) * hs_stride + 2 * j;
      p0 = hs[0];
      p1 = hs[1];
    }
  };
  auto stage_finish = [&](int b, int Iu, float p0, float p1) {
    const int m = tid & (kSub - 1), j = tid >> 4;
    if (j < Iu / 32) cs[b][j][m] = p0 + p1;
  };
  int nc = sI / 64, upr = sI / 8;
  // unit u uses buffer (u - u_first) & 1; the second unit of the range (if
  // any) is staged right away
  const int u_first = xu;
  int hb = 0;
  const bool two = (s1 - 1) / qpu > u_first;
  const UnitHdr hd1 = two ? unit_hdr(a.units, u_first + 1) : hd0;
  const int I1 = inter_of(hd1.expert);
  if (tid < kSub) {
    urow[0][tid] = row0 + tid;
    urow[1][tid] = hd1.row0 + tid;
  }
  __syncthreads();
  float hp0, hp1, hq0 = 0.0f, hq1 = 0.0f;
  stage_issue(0, row0, mc, sI, hp0, hp1);
  if (two) stage_issue(1, hd1.row0, hd1.mc, I1, hq0, hq1);
  asm volatile("" ::: "memory");
  Slot sl[kDepth * kSlot];
#pragma unroll
  for (int hf = 0; hf < kDepth; ++hf) {
    const uint4* qb;
    const uint8_t* sb;
    int ncq;
    tile_src(min(s0 + hf, s1 - 1), qb, sb, ncq);
#pragma unroll
    for (int j = 0; j < kSlot; ++j) load_slot<G, BITS>(sl[hf * kSlot + j], qb, sb, FULL ? kh + 2 * j : min(kh + 2 * j, ncq - 1));
  }
  // the weight loads just issued may stay in flight; the staging before them may not
  staged_barrier<kDepth * kSlot * kLoadsPerSlot<G, BITS>>();
  stage_finish(0, nc * 64, hp0, hp1);
  if (two) stage_finish(1, I1, hq0, hq1);
  staged_barrier<kDepth * kSlot * kLoadsPerSlot<G, BITS>>();
  auto process = [&](const int q, auto hfc) {
    constexpr int hf = decltype(hfc)::value;
    const int u = q / qpu;
    const int pt = (q - u * qpu) * 4 + q4;
    if (u != xu) {
      const UnitHdr hd = unit_hdr(a.units, u);
      const int Iu = inter_of(hd.expert);
      hb = (u - u_first) & 1;
      if (u > u_first + 1) {
        // not staged yet: wait until the readers of unit u - 2 (same buffer)
        // are done, then stage and wait for it
        __syncthreads();
        if (tid < kSub) urow[hb][tid] = hd.row0 + tid;
        __syncthreads();
        float p0, p1;
        stage_issue(hb, hd.row0, hd.mc, Iu, p0, p1);
        stage_finish(hb, Iu, p0, p1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
      xu = u;
      row0 = hd.row0;
      mc = hd.mc;
      nc = Iu / 64;
      upr = Iu / 8;
    }
    const uint4* qnx;
    const uint8_t* snx;
    int ncn;
    tile_src(min(q + kDepth, s1 - 1), qnx, snx, ncn);
    const uint16_t* ha0 = &hsh[hb][(n * upr + (kb ^ (n & 7))) * 8];
    const uint16_t* ha1 = &hsh[hb][(n * upr + ((kb + 4) ^ (n & 7))) * 8];
    const float(*csb)[kSub] = cs[hb];
    f32x4_t accA = {0, 0, 0, 0}, accB = {0, 0, 0, 0}, biasA = {0, 0, 0, 0}, biasB = {0, 0, 0, 0};
    // the scale of chunk j is applied after the products of chunk j + 1 are
    // issued (matrix-core latency)
    Prod pp;
    Coef pk;
    float pcs0[4], pcs1[4];
#pragma unroll
    for (int j = 0; j < kSlot; ++j) {
      const int c = kh + 2 * j;
      Slot& s = sl[hf * kSlot + j];
      const Decoded d = decode_slot<G, BITS>(s);
      load_slot<G, BITS>(s, qnx, snx, FULL ? c : min(c, ncn - 1));
      Prod p;
      float cs0[4], cs1[4];
      if (FULL || c < nc) {
        const uint4 h0 = *reinterpret_cast<const uint4*>(ha0 + 64 * c);
        const uint4 h1 = *reinterpret_cast<const uint4*>(ha1 + 64 * c);
        const float4 c0 = *reinterpret_cast<const float4*>(&csb[2 * c][4 * kb]);
        const float4 c1 = *reinterpret_cast<const float4*>(&csb[2 * c + 1][4 * kb]);
        if constexpr (G == 32) {
          cs0[0] = c0.x; cs0[1] = c0.y; cs0[2] = c0.z; cs0[3] = c0.w;
          cs1[0] = c1.x; cs1[1] = c1.y; cs1[2] = c1.z; cs1[3] = c1.w;
        } else {
          cs0[0] = c0.x + c1.x; cs0[1] = c0.y + c1.y; cs0[2] = c0.z + c1.z; cs0[3] = c0.w + c1.w;
          cs1[0] = cs0[0]; cs1[1] = cs0[1]; cs1[2] = cs0[2]; cs1[3] = cs0[3];
        }
        p = chunk_mfma<G, false>(d, h0, h1, h0, h1);
      }
      if (j > 0 && (FULL || c - 2 < nc)) chunk_scale<G>(pp, pk, pcs0, pcs1, accA, accB, biasA, biasB);
      pp = p;
      pk = coef_of(d);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pcs0[i] = cs0[i];
        pcs1[i] = cs1[i];
      }
    }
    if (FULL || kh + 2 * (kSlot - 1) < nc) chunk_scale<G>(pp, pk, pcs0, pcs1, accA, accB, biasA, biasB);
    (void)kHalves;
    constexpr int rb = hf & 1;
    if (kh == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        red[rb][q4][i][lane] = fmaf(kQScale, accA[i], biasA[i]);
        red[rb][q4][4 + i][lane] = fmaf(kQScale, accB[i], biasB[i]);
      }
    }
    __syncthreads();
    if (kh == 0 && (FULL || pt < n_pairs)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * kb + i;
        if (m < mc) {
          float* yr = a.yrow + static_cast<size_t>(row0 + m) * H + 32 * pt;
          yr[n] = fmaf(kQScale, accA[i], biasA[i]) + red[rb][q4][i][lane];
          yr[16 + n] = fmaf(kQScale, accB[i], biasB[i]) + red[rb][q4][4 + i][lane];
        }
      }
    }
  };
  int sb0 = s0;
  for (; sb0 + kDepth <= s1; sb0 += kDepth) {
    process(sb0, Half<0>{});
    process(sb0 + 1, Half<1>{});
  }
  if (sb0 < s1) process(sb0, Half<0>{});
}

// the family's largest shape, for which the down kernel drops its bounds
// tests (FULL: every chunk and pair-tile index it forms is in range)
static bool full_shape(const FfnArgs& a) {
  return a.H == kGroupedMaxH && a.I == kGroupedMaxInter && (a.Is == kGroupedMaxInter || a.Is == 0);
}

// 16 waves where that form needs no more than its 128 registers per lane
// (bf16 activations, int4, group 64 or 128, the full shape); 8 elsewhere.
template <int A, int G, int B>
static void launch_gateup_t(const FfnArgs& a, hipStream_t s) {
  const bool full = a.H == kGroupedMaxH;
  if constexpr (A == 2 && B == 4 && G >= 64) {
    if (full) {
      hipLaunchKernelGGL((k_gateup_tiles<A, G, B, true, 16>), dim3(kGridTiles), dim3(1024), 0, s, a);
      return;
    }
  } else {
    if (full) {
      hipLaunchKernelGGL((k_gateup_tiles<A, G, B, true, 8>), dim3(kGridTiles), dim3(512), 0, s, a);
      return;
    }
  }
  hipLaunchKernelGGL((k_gateup_tiles<A, G, B, false, 8>), dim3(kGridTiles), dim3(512), 0, s, a);
}

hipError_t launch_gateup_grouped(int act, const FfnArgs& a, hipStream_t s) {
#define GU_G(A_, B_)                                   \
  do {                                                 \
    if (a.G == 32) launch_gateup_t<A_, 32, B_>(a, s);  \
    else if (a.G == 64) launch_gateup_t<A_, 64, B_>(a, s); \
    else launch_gateup_t<A_, 128, B_>(a, s);           \
  } while (0)
  if (a.bits == 8) {
    if (act == 2) GU_G(2, 8);
    else GU_G(1, 8);
  } else {
    if (act == 2) GU_G(2, 4);
    else GU_G(1, 4);
  }
#undef GU_G
  return hipGetLastError();
}

hipError_t launch_down_grouped(const FfnArgs& a, hipStream_t s) {
  const bool full = full_shape(a);
#define DN_LAUNCH(G_, B_)                                                                            \
  do {                                                                                               \
    if (full) hipLaunchKernelGGL((k_down_tiles<G_, B_, true>), dim3(kGridTiles), dim3(512), 0, s, a); \
    else hipLaunchKernelGGL((k_down_tiles<G_, B_, false>), dim3(kGridTiles), dim3(512), 0, s, a);     \
  } while (0)
  if (a.bits == 8) {
    // group 32 with int8 keeps the generic form (the FULL one needs scratch)
    if (a.G == 32) hipLaunchKernelGGL((k_down_tiles<32, 8, false>), dim3(kGridTiles), dim3(512), 0, s, a);
    else if (a.G == 64) DN_LAUNCH(64, 8);
    else DN_LAUNCH(128, 8);
  } else {
    if (a.G == 32) DN_LAUNCH(32, 4);
    else if (a.G == 64) DN_LAUNCH(64, 4);
    else DN_LAUNCH(128, 4);
  }
#undef DN_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
