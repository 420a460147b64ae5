// Batched grouped-GEMM family on the gfx950 matrix cores.
//
// When a batch routes many tokens to the same experts, each expert's weights
// are streamed for all of its tokens together: the rows of the batch are
// bucketed by expert (stable counting sort), and work items of up to 16 of one
// expert's token rows are multiplied by a slice of that expert's weights with
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
// split into bf16 hi + lo pairs (four MFMAs).  Activations are exact in the
// operand type; the SwiGLU output h enters the down projection as a hi + lo
// bf16 pair (h = hi + lo to 16 significant bits).
//
// Operand layout of v_mfma_f32_16x16x32 (64 lanes, lane l: n = l % 16,
// kb = l / 16): A lane holds row m = n, k = 8kb..8kb+7; B lane holds column n,
// k = 8kb..8kb+7; C lane holds rows 4kb..4kb+3 of column n.  The expert blob
// stores each lane's B values contiguously (see the public header), so one
// 16-byte load per lane fetches the B operands of two 16-row tiles for a
// 64-column chunk.
//
// Scheduling.  Both kernels are persistent: workgroup w runs work items
// w, w + grid, ... of the list built by the bucketing kernel (longest units
// first; sub-items of one unit on one XCD).  Each wave streams its weight
// chunks through kPF register slots; the refills issued while the last chunks
// of an item are processed already fetch the next item's first chunks, and the
// next item's descriptor and token ids are loaded during the current item, so
// the weight stream does not stop between items.  An item's activations are
// staged in LDS once, with direct global-to-LDS loads.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int kSub = kSubTokens;
constexpr int kPF = 16;                              // gate/up weight chunks in flight per wave
constexpr int kPFD = 2 * kGroupedMaxInter / 64;      // down: a whole item's stream (two pair-tiles)
constexpr int kGridGU = 1024;                        // persistent grids (multiples of 8)
constexpr int kGridD = 1024;

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

// 16-byte global -> LDS copy by the active lanes of a wave; lane i writes
// 16 bytes at lds_base + 16 i (lds_base is wave-uniform).
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void_ptr)(lds_base), 16, 0, 0);
}

// Staged tile of 16 rows: 16-byte unit (m, u8) (columns 8*u8..8*u8+7 of row m)
// sits at m*upr + (u8 ^ (m & 7)), so the 16 lanes reading one column block of
// the 16 rows hit different banks.
__device__ __forceinline__ int unit_pos(int m, int u8, int upr) { return m * upr + (u8 ^ (m & 7)); }

// Marks a weight slot's decoded operands and scales as computed here: the
// compiler may not sink the decoding below the slot's refill (a later memory
// access), which would keep the old and the new slot contents live together.
__device__ __forceinline__ void consumed(uint4& a, uint4& b, uint4& c, uint4& d, float& s0, float& s1) {
  asm volatile("" : "+v"(a.x), "+v"(a.y), "+v"(a.z), "+v"(a.w), "+v"(b.x), "+v"(b.y), "+v"(b.z), "+v"(b.w) : : "memory");
  asm volatile("" : "+v"(c.x), "+v"(c.y), "+v"(c.z), "+v"(c.w), "+v"(d.x), "+v"(d.y), "+v"(d.z), "+v"(d.w), "+v"(s0),
               "+v"(s1) : : "memory");
}

struct Item {
  int row0, mc, block, expert;
};
__device__ __forceinline__ Item decode_item(int4 w) { return Item{w.x, w.y & 0xFF, w.y >> 8, w.z}; }

__device__ __forceinline__ const uint8_t* item_blob(const FfnArgs& a, int expert) {
  return expert < 0 ? a.shared : a.experts + (a.offsets ? a.offsets[expert] : static_cast<uint64_t>(expert) * a.stride);
}

__device__ __forceinline__ int row_token(const FfnArgs& a, int row) {
  const int tk = a.T * a.K;
  return row < tk ? a.tok_sorted[row] : row - tk;
}

// Bias MFMA B operands for groups g0 + 8kb + 0..7 of the lane's rows:
// (b - 16 s) of tile A and tile B as hi/lo bf16 (zero beyond ng).
struct BiasRaw {
  uint2 v[8];
};
__device__ __forceinline__ BiasRaw bias_load(const uint8_t* ssec, int p, int ng, int g0, int n, int kb) {
  BiasRaw r;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int g = min(g0 + 8 * kb + j, ng - 1);
    r.v[j] = *reinterpret_cast<const uint2*>(ssec + ((static_cast<uint64_t>(p) * ng + g) * 16 + n) * 8);
  }
  return r;
}
__device__ __forceinline__ void bias_operands(const BiasRaw& r, int ng, int g0, int kb, uint4& ah, uint4& al,
                                              uint4& bh, uint4& bl) {
  uint32_t vah[4], val[4], vbh[4], vbl[4];
#pragma unroll
  for (int j2 = 0; j2 < 4; ++j2) {
    uint32_t h2[2][2], l2[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = 2 * j2 + h;
      const bool in = g0 + 8 * kb + j < ng;
      const float ba = in ? fmaf(-16.0f, f16_bits_to_f32(r.v[j].x & 0xFFFFu), f16_bits_to_f32(r.v[j].x >> 16)) : 0.0f;
      const float bb = in ? fmaf(-16.0f, f16_bits_to_f32(r.v[j].y & 0xFFFFu), f16_bits_to_f32(r.v[j].y >> 16)) : 0.0f;
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

// A operand of the bias MFMA: group sums of row n, groups g0 + 8kb + 0..7, hi/lo.
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
// gate/up + SwiGLU.  Item block b = 64 rows of I; wave w owns gate/up pair-tile
// p = 4b + w, i.e. weight chunks p*nc .. p*nc + nc - 1 of the GU section.
// Output: h as hi and lo bf16 planes.
// ---------------------------------------------------------------------------
// NCT > 0: the hidden size is 64*NCT (compile-time chunk count, refills run into
// the next item when NCT % kPF == 0); NCT == 0: any hidden size up to the
// family's maximum, slots reloaded per item.
template <int ACT, int G, int NCT>
__global__ __launch_bounds__(256) void k_gateup_grouped(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[kSub * kGroupedMaxH];
  __shared__ float gsum[kSub][kGroupedMaxH / 32 + 1];
  __shared__ int tok[kSub];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kb = lane >> 4;
  const int H = NCT > 0 ? 64 * NCT : a.H;
  const int nc = H / 64, ng = H / G, upr = H / 8;
  const int n_work = a.n_work[0];
  const int hplane = (a.T * a.K + (a.Is > 0 ? a.T : 0)) * a.hstride;
  uint16_t* h_hi = reinterpret_cast<uint16_t*>(a.h);
  uint16_t* h_lo = h_hi + hplane;
  int wi = blockIdx.x;
  if (wi >= n_work) return;
  Item it = decode_item(a.work_gu[wi]);
  const uint8_t* blob = item_blob(a, it.expert);
  int p = 4 * it.block + wave;
  const uint4* qblk = reinterpret_cast<const uint4*>(blob) + static_cast<size_t>(p) * nc * 64;
  const uint8_t* ssec = blob + blob_gu_s(H, it.expert < 0 ? a.Is : a.I);
  // weight stream: slot u holds the chunk c with c % kPF == u
  uint4 qn[kPF];
  uint2 sn[kPF];
#pragma unroll
  for (int u = 0; u < kPF; ++u) {
    const int c = min(u, nc - 1);
    qn[u] = qblk[static_cast<size_t>(c) * 64 + lane];
    sn[u] = *reinterpret_cast<const uint2*>(ssec + ((static_cast<uint64_t>(p) * ng + (64 * c) / G) * 16 + n) * 8);
  }
  int tok_next = (tid < it.mc) ? row_token(a, it.row0 + tid) : 0;
  // the refills run into the next item only when its chunks land in the slots
  // they are read from (c % kPF), i.e. when an item has a multiple of kPF chunks
  static_assert(NCT == 0 || NCT % kPF == 0, "compile-time chunk count must fill whole slot blocks");
  constexpr bool cross = NCT > 0;
  bool first = true;
  while (true) {
    if (!cross && !first) {
#pragma unroll
      for (int u = 0; u < kPF; ++u) {
        const int c = min(u, nc - 1);
        qn[u] = qblk[static_cast<size_t>(c) * 64 + lane];
        sn[u] = *reinterpret_cast<const uint2*>(ssec + ((static_cast<uint64_t>(p) * ng + (64 * c) / G) * 16 + n) * 8);
      }
    }
    first = false;
    // ---- item setup: tokens, next descriptor, activation staging, bias operands
    __syncthreads();                  // previous item's LDS readers are done
    if (tid < it.mc) tok[tid] = tok_next;
    const int wi2 = wi + gridDim.x;
    const bool has_next = wi2 < n_work;
    const int4 w2 = has_next ? a.work_gu[wi2] : make_int4(0, 0, 0, 0);
    const int nbias = (ng + 31) / 32;
    BiasRaw braw[kGroupedMaxH / 32 / 32];
#pragma unroll
    for (int gb = 0; gb < kGroupedMaxH / 32 / 32; ++gb)
      if (gb < nbias) braw[gb] = bias_load(ssec, p, ng, 32 * gb, n, kb);
    __syncthreads();                  // tok visible
    for (int op = wave; op * 64 < kSub * upr; op += 4) {
      const int u = op * 64 + lane;
      const int m = u / upr, ph = u - m * upr;
      if (m < it.mc) dma16(a.x + static_cast<size_t>(tok[m]) * H + 8 * (ph ^ (m & 7)), &xs[op * 64 * 8]);
    }
    __builtin_amdgcn_s_waitcnt(0);    // this wave's direct-to-LDS loads have landed
    __syncthreads();
    for (int idx = tid; idx < kSub * ng; idx += 256) {
      const int m = idx / ng, g = idx - m * ng;
      float s = 0.0f;
      if (m < it.mc) {
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
    f32x4_t bsg = {0, 0, 0, 0}, bsu = {0, 0, 0, 0};
#pragma unroll
    for (int gb = 0; gb < kGroupedMaxH / 32 / 32; ++gb) {
      if (gb < nbias) {
        uint4 sh, sl, bah, bal, bbh, bbl;
        sum_operands(&gsum[0][0], kGroupedMaxH / 32 + 1, ng, 32 * gb, n, kb, sh, sl);
        bias_operands(braw[gb], ng, 32 * gb, kb, bah, bal, bbh, bbl);
        bsg = bias_mfma(sh, sl, bah, bal, bsg);
        bsu = bias_mfma(sh, sl, bbh, bbl, bsu);
      }
    }
    // ---- next item's weight addresses (its first chunks are fetched by the refills)
    const Item it2 = decode_item(w2);
    const uint8_t* blob2 = has_next ? item_blob(a, it2.expert) : blob;
    const int p2 = has_next ? 4 * it2.block + wave : p;
    const uint4* qblk2 = reinterpret_cast<const uint4*>(blob2) + static_cast<size_t>(p2) * nc * 64;
    const uint8_t* ssec2 = has_next ? blob2 + blob_gu_s(H, it2.expert < 0 ? a.Is : a.I) : ssec;
    // (without a next item these point at this item's own first chunks: the
    // refills then repeat loads of valid memory and are never read)
    // ---- main loop: blocks of kPF chunks; within a block chunk cb + u sits in
    // slot u and is replaced by chunk cb + kPF + u, or, past the item's end,
    // by the next item's chunk u (cross) / this item's last chunk (repeat, unused)
    f32x4_t accg = {0, 0, 0, 0}, accu = {0, 0, 0, 0}, pg = {0, 0, 0, 0}, pu = {0, 0, 0, 0};
    // A operand of chunk c: unit (n, 8c + kb) = lane base + 8c units (the XOR
    // swizzle only touches the low 3 bits, which 8c leaves free)
    const uint16_t* xa0 = &xs[(n * upr + (kb ^ (n & 7))) * 8];
    const uint16_t* xa1 = &xs[(n * upr + ((kb + 4) ^ (n & 7))) * 8];
    const uint8_t* srow = ssec + (static_cast<uint64_t>(p) * ng * 16 + n) * 8;   // scales of (p, group 0, n)
    const uint8_t* srow2 = ssec2 + (static_cast<uint64_t>(p2) * ng * 16 + n) * 8;
#pragma unroll 1
    for (int cb = 0; cb < nc; cb += kPF) {
      const bool nxt = cross && cb + kPF >= nc;
      const uint4* qsrc = nxt ? qblk2 : qblk;
      const uint8_t* ssrc = nxt ? srow2 : srow;
      const int cr = nxt ? 0 : cb + kPF;
#pragma unroll
      for (int u = 0; u < kPF; ++u) {
        const int c = cb + u;
        if (cross || c < nc) {
          const uint4 q = qn[u];
          const uint2 sr = sn[u];
          uint4 bg0 = word_operand<ACT>(q.x), bg1 = word_operand<ACT>(q.y);
          uint4 bu0 = word_operand<ACT>(q.z), bu1 = word_operand<ACT>(q.w);
          float sg = f16_bits_to_f32(sr.x & 0xFFFFu), su = f16_bits_to_f32(sr.y & 0xFFFFu);
          // the slot is fully consumed before its refill is issued, so the refill
          // lands in the same registers (no copies, no early waits at the back-edge)
          consumed(bg0, bg1, bu0, bu1, sg, su);
          {
            const int cn = cross ? cr + u : min(cr + u, nc - 1);
            qn[u] = qsrc[static_cast<size_t>(cn) * 64 + lane];
            sn[u] = *reinterpret_cast<const uint2*>(ssrc + static_cast<size_t>((64 * cn) / G) * 128);
          }
          const uint4 a0 = *reinterpret_cast<const uint4*>(xa0 + 64 * c);
          const uint4 a1 = *reinterpret_cast<const uint4*>(xa1 + 64 * c);
          if constexpr (G == 32) {
            const uint2 sr1 = *reinterpret_cast<const uint2*>(srow + static_cast<size_t>(2 * c + 1) * 128);
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
            // G = 128 spans chunks c, c + 1 (c even; cb is a multiple of kPF, which is even)
            if (G == 64 || (u & 1)) {
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
    // tokens of the next item (read during this item's tail)
    if (has_next) tok_next = (tid < it2.mc) ? row_token(a, it2.row0 + tid) : 0;
    // ---- SwiGLU; lane holds tokens 4kb..4kb+3 of column n of pair-tile p
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * kb + i;
      if (m < it.mc) {
        const float ga = fmaf(16.0f, accg[i], bsg[i]);
        const float up = fmaf(16.0f, accu[i], bsu[i]);
        const float hv = ga / (1.0f + expf(-ga)) * up;
        uint32_t hi, lo;
        split_bf16(hv, hi, lo);
        const size_t o = static_cast<size_t>(it.row0 + m) * a.hstride + 16 * p + n;
        h_hi[o] = static_cast<uint16_t>(hi);
        h_lo[o] = static_cast<uint16_t>(lo);
      }
    }
    if (!has_next) break;
    wi = wi2;
    it = it2;
    blob = blob2;
    p = p2;
    qblk = qblk2;
    ssec = ssec2;
  }
}

// ---------------------------------------------------------------------------
// down projection.  Item block b = 256 output rows; wave w owns the two down
// pair-tiles p0 = 8b + 2w and p0 + 1 (64 rows).  Its weight stream is chunk j
// = (pair-tile p0 + j / nc, chunk j % nc), j < 2 nc <= kPFD, so an item's whole
// stream sits in the kPFD slots: slot j is refilled with the next item's chunk
// j as soon as it is consumed, and the next item's weights are in flight while
// this one computes.  Reads h (hi/lo planes) of its tokens.
// ---------------------------------------------------------------------------
// NJT > 0: every expert (routed and shared) streams NJT chunks (inter = 32 NJT,
// compile-time tile split); NJT == 0: any inter up to the family's maximum.
template <int G, int NJT>
__global__ __launch_bounds__(256) void k_down_grouped(FfnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t hsh[kSub * kGroupedMaxInter];
  __shared__ __attribute__((aligned(16))) uint16_t hsl[kSub * kGroupedMaxInter];
  __shared__ float gsum[kSub][kGroupedMaxInter / 32 + 1];
  static_assert(NJT == 0 || (NJT <= kPFD && NJT % 2 == 0), "stream must fit the slots");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kb = lane >> 4;
  const int H = a.H;
  const int n_pairs = H / 32;
  const int n_work = a.n_work[1];
  const int hplane = (a.T * a.K + (a.Is > 0 ? a.T : 0)) * a.hstride;
  const uint16_t* h_hi = reinterpret_cast<const uint16_t*>(a.h);
  const uint16_t* h_lo = h_hi + hplane;
  int wi = blockIdx.x;
  if (wi >= n_work) return;
  Item it = decode_item(a.work_d[wi]);
  const uint8_t* blob = item_blob(a, it.expert);
  int I = it.expert < 0 ? a.Is : a.I;
  int p0 = 8 * it.block + 2 * wave;
  // weights of pair-tile pp (clamped to the last pair-tile of H) of a blob
  auto qtile = [&](const uint8_t* bl, int Ii, int pp) -> const uint4* {
    return reinterpret_cast<const uint4*>(bl + blob_d_q(H, Ii)) +
           static_cast<size_t>(min(pp, n_pairs - 1)) * (Ii / 64) * 64 + lane;
  };
  auto stile = [&](const uint8_t* bl, int Ii, int pp) -> const uint8_t* {
    return bl + blob_d_s(H, Ii, G) + (static_cast<uint64_t>(min(pp, n_pairs - 1)) * (Ii / G) * 16 + n) * 8;
  };
  // stream chunk u of the item (blob, Ii, pair-tiles pp0, pp0 + 1); u past the
  // stream's end repeats its last chunk (loaded, never used)
  auto load_chunk = [&](const uint8_t* bl, int Ii, int pp0, int u, uint4& q, uint2& sc) {
    const int nci = NJT > 0 ? NJT / 2 : Ii / 64;
    const int j = NJT > 0 ? u : min(u, 2 * nci - 1);
    const int t = j >= nci ? 1 : 0, c = j - t * nci;
    q = qtile(bl, Ii, pp0 + t)[static_cast<size_t>(c) * 64];
    sc = *reinterpret_cast<const uint2*>(stile(bl, Ii, pp0 + t) + static_cast<size_t>((64 * c) / G) * 128);
  };
  uint4 qn[kPFD];
  uint2 sn[kPFD];
#pragma unroll
  for (int u = 0; u < kPFD; ++u) load_chunk(blob, I, p0, u, qn[u], sn[u]);
  while (true) {
    const int nc = NJT > 0 ? NJT / 2 : I / 64;
    const int ng = 64 * nc / G, upr = 8 * nc;
    const uint8_t* dsec = blob + blob_d_s(H, I, G);
    __syncthreads();
    const int wi2 = wi + gridDim.x;
    const bool has_next = wi2 < n_work;
    const int4 w2 = has_next ? a.work_d[wi2] : make_int4(0, 0, 0, 0);
    const bool v0 = p0 < n_pairs, v1 = p0 + 1 < n_pairs;
    BiasRaw braw[2];
    braw[0] = bias_load(dsec, min(p0, n_pairs - 1), ng, 0, n, kb);
    braw[1] = bias_load(dsec, min(p0 + 1, n_pairs - 1), ng, 0, n, kb);
    for (int op = wave; op * 64 < kSub * upr; op += 4) {
      const int u = op * 64 + lane;
      const int m = u / upr, ph = u - m * upr;
      if (m < it.mc) {
        const size_t src = static_cast<size_t>(it.row0 + m) * a.hstride + 8 * (ph ^ (m & 7));
        dma16(h_hi + src, &hsh[op * 64 * 8]);
        dma16(h_lo + src, &hsl[op * 64 * 8]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int idx = tid; idx < kSub * ng; idx += 256) {
      const int m = idx / ng, g = idx - m * ng;
      float s = 0.0f;
      if (m < it.mc) {
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
    f32x4_t bias[4];
    {
      uint4 sh, sl;
      sum_operands(&gsum[0][0], kGroupedMaxInter / 32 + 1, ng, 0, n, kb, sh, sl);
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        uint4 bah, bal, bbh, bbl;
        bias_operands(braw[t2], ng, 0, kb, bah, bal, bbh, bbl);
        bias[2 * t2] = bias_mfma(sh, sl, bah, bal, f32x4_t{0, 0, 0, 0});
        bias[2 * t2 + 1] = bias_mfma(sh, sl, bbh, bbl, f32x4_t{0, 0, 0, 0});
      }
    }
    // the refills fetch the next item's stream (this item's again when there is none)
    const Item it2 = decode_item(w2);
    const uint8_t* blob2 = has_next ? item_blob(a, it2.expert) : blob;
    const int I2 = has_next ? (it2.expert < 0 ? a.Is : a.I) : I;
    const int p02 = has_next ? 8 * it2.block + 2 * wave : p0;
    f32x4_t acc[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
    f32x4_t pa = {0, 0, 0, 0}, pb = {0, 0, 0, 0};
    const uint16_t* ha0 = &hsh[(n * upr + (kb ^ (n & 7))) * 8];
    const uint16_t* ha1 = &hsh[(n * upr + ((kb + 4) ^ (n & 7))) * 8];
    const uint16_t* la0 = &hsl[(n * upr + (kb ^ (n & 7))) * 8];
    const uint16_t* la1 = &hsl[(n * upr + ((kb + 4) ^ (n & 7))) * 8];
    const uint8_t* st0 = stile(blob, I, p0);
    const uint8_t* st1 = stile(blob, I, p0 + 1);
#pragma unroll
    for (int u = 0; u < (NJT > 0 ? NJT : kPFD); ++u) {
      if (NJT > 0 || u < 2 * nc) {
        const uint4 q = qn[u];
        const uint2 sr = sn[u];
        uint4 ba0 = word_operand<2>(q.x), ba1 = word_operand<2>(q.y);
        uint4 bb0 = word_operand<2>(q.z), bb1 = word_operand<2>(q.w);
        float sa = f16_bits_to_f32(sr.x & 0xFFFFu), sb = f16_bits_to_f32(sr.y & 0xFFFFu);
        consumed(ba0, ba1, bb0, bb1, sa, sb);
        load_chunk(blob2, I2, p02, u, qn[u], sn[u]);
        const int t2 = u >= nc ? 1 : 0;  // which pair-tile of the wave
        const int c = u - t2 * nc;
        const uint4 h0 = *reinterpret_cast<const uint4*>(ha0 + 64 * c);
        const uint4 h1 = *reinterpret_cast<const uint4*>(ha1 + 64 * c);
        const uint4 l0 = *reinterpret_cast<const uint4*>(la0 + 64 * c);
        const uint4 l1 = *reinterpret_cast<const uint4*>(la1 + 64 * c);
        f32x4_t ra, rb;  // scaled products of this chunk (or chunk pair)
        bool flush = true;
        if constexpr (G == 32) {
          const uint2 sr1 = *reinterpret_cast<const uint2*>((t2 ? st1 : st0) + static_cast<size_t>(2 * c + 1) * 128);
          const float sa1 = f16_bits_to_f32(sr1.x & 0xFFFFu), sb1 = f16_bits_to_f32(sr1.y & 0xFFFFu);
          const f32x4_t z = {0, 0, 0, 0};
          const f32x4_t x0 = mfma<2>(l0, ba0, mfma<2>(h0, ba0, z));
          const f32x4_t y0 = mfma<2>(l0, bb0, mfma<2>(h0, bb0, z));
          const f32x4_t x1 = mfma<2>(l1, ba1, mfma<2>(h1, ba1, z));
          const f32x4_t y1 = mfma<2>(l1, bb1, mfma<2>(h1, bb1, z));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ra[i] = fmaf(sa1, x1[i], sa * x0[i]);
            rb[i] = fmaf(sb1, y1[i], sb * y0[i]);
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
          // G = 128 spans chunks c, c + 1 (nc is even then, so c and u agree in parity)
          flush = G == 64 || (u & 1);
          ra = pa;
          rb = pb;
        }
        if (flush) {
          if (NJT > 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              acc[2 * t2][i] = G == 32 ? acc[2 * t2][i] + ra[i] : fmaf(sa, ra[i], acc[2 * t2][i]);
              acc[2 * t2 + 1][i] = G == 32 ? acc[2 * t2 + 1][i] + rb[i] : fmaf(sb, rb[i], acc[2 * t2 + 1][i]);
            }
          } else {
            // tile chosen at run time: update both accumulator pairs by select
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float na = G == 32 ? (t2 ? acc[2][i] : acc[0][i]) + ra[i]
                                       : fmaf(sa, ra[i], t2 ? acc[2][i] : acc[0][i]);
              const float nb = G == 32 ? (t2 ? acc[3][i] : acc[1][i]) + rb[i]
                                       : fmaf(sb, rb[i], t2 ? acc[3][i] : acc[1][i]);
              acc[0][i] = t2 ? acc[0][i] : na;
              acc[2][i] = t2 ? na : acc[2][i];
              acc[1][i] = t2 ? acc[1][i] : nb;
              acc[3][i] = t2 ? nb : acc[3][i];
            }
          }
          // pin the scaling here: otherwise every chunk's products stay live
          // in their own registers until the end of the stream
          asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
          pa = f32x4_t{0, 0, 0, 0};
          pb = f32x4_t{0, 0, 0, 0};
        }
        // keep each chunk's LDS reads next to its products (hoisting all of
        // them costs more registers than the latency they would hide)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      if (t2 == 0 ? v0 : v1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 4 * kb + i;
          if (m < it.mc) {
            float* yr = a.yrow + static_cast<size_t>(it.row0 + m) * H + 32 * (p0 + t2);
            yr[n] = fmaf(16.0f, acc[2 * t2][i], bias[2 * t2][i]);
            yr[16 + n] = fmaf(16.0f, acc[2 * t2 + 1][i], bias[2 * t2 + 1][i]);
          }
        }
      }
    }
    if (!has_next) break;
    wi = wi2;
    it = it2;
    blob = blob2;
    I = I2;
    p0 = p02;
  }
}

static int grid_cap(int upper, int cap) { return upper < cap ? (upper > 0 ? upper : 1) : cap; }

hipError_t launch_gateup_grouped(int act, const FfnArgs& a, hipStream_t s) {
  const int grid = grid_cap(work_upper(a.I / 64, a.Is / 64, a.T, a.K, a.E), kGridGU);
#define GU_LAUNCH(A_, G_)                                                                   \
  do {                                                                                      \
    if (a.H == 2048) hipLaunchKernelGGL((k_gateup_grouped<A_, G_, 32>), dim3(grid), dim3(256), 0, s, a); \
    else hipLaunchKernelGGL((k_gateup_grouped<A_, G_, 0>), dim3(grid), dim3(256), 0, s, a);           \
  } while (0)
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
  const int nb = (a.H + kDownBlockRows - 1) / kDownBlockRows;
  const int grid = grid_cap(work_upper(nb, a.Is > 0 ? nb : 0, a.T, a.K, a.E), kGridD);
  const bool i512 = a.I == 512 && (a.Is == 0 || a.Is == 512);
#define D_LAUNCH(G_)                                                                     \
  do {                                                                                   \
    if (i512) hipLaunchKernelGGL((k_down_grouped<G_, kPFD>), dim3(grid), dim3(256), 0, s, a); \
    else hipLaunchKernelGGL((k_down_grouped<G_, 0>), dim3(grid), dim3(256), 0, s, a);        \
  } while (0)
  if (a.G == 32) D_LAUNCH(32);
  else if (a.G == 64) D_LAUNCH(64);
  else D_LAUNCH(128);
#undef D_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
