// Internal launch functions of the MoE kernels (host side).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "blob_copy.h"

namespace moe {

constexpr int kMaxH = 8192;        // hidden size limit (router keeps a row in registers)
constexpr int kMaxInter = 4096;    // intermediate size limit (down GEMV stages h in LDS)
constexpr int kMaxExperts = 1024;  // top-k holds E/64 logits per lane; bucketing uses one workgroup
constexpr int kMaxTopK = 64;       // one selected expert per lane
constexpr int kRouterMfmaMinTokens = 16;  // router GEMM on the matrix cores from this batch size
constexpr int kRouterMaxParts = 4;        // hidden-dimension slices of the matrix-core router
constexpr int kRouterWaves = 4;           // waves per matrix-core router workgroup
constexpr int kRouterBatch = 8;           // 32-column steps whose loads a router wave issues together

// Routed rows of a batch: row j < T*K is (token j/K, rank j%K) in slot order,
// or the j-th row of the expert-sorted order in the grouped family; rows
// T*K + t (t < T) are the shared expert's.
struct FfnArgs {
  const uint16_t* x;          // [T][H] activations
  const int32_t* topk_idx;    // [T][K]
  const uint8_t* experts;     // routed blob base
  uint64_t stride;            // blob stride when offsets == nullptr
  const uint64_t* offsets;    // [E] byte offsets or nullptr
  const uint8_t* shared;      // shared blob or nullptr
  float* h;                   // grouped: h as fp16 [rows][hstride], operand-ready;
                              // GEMV: partial (gate, up) sums [kGemvSplit][rows][hstride][2] fp32
  float* yrow;                // [rows][H] per-row expert outputs (unweighted)
  // grouped family
  const int32_t* units;       // [n_units][kUnitInts] unit records (see UnitPlan)
  const int32_t* n_units;     // [2] shared units, routed units
  float* hsum;                // [rows][hstride/16] sums of h over 16-column blocks
  int T, H, K, I, Is, G, E;
  int hstride;                // max(I, Is)
  int bits;                   // expert weight width, 4 or 8
  // GEMV family with top-K fused into gate/up (route_part != nullptr): every
  // routed row's workgroups select the token's experts from the router's
  // logit slices themselves; one workgroup per token (the last rank's,
  // pair-tile 0, split 0) writes the selection to sel_idx (== topk_idx),
  // sel_w, sel_gamma
  const float* route_part;    // [route_nparts][T][E+1]
  const float* route_bias;    // [E] or nullptr (also nullptr when the slices hold it)
  int route_nparts;
  int32_t* sel_idx;
  float* sel_w;
  float* sel_gamma;
  // status word of the call (workspace): with status_reset the GEMV gate/up
  // kernel clears it (the grouped family clears it in the bucketing kernel);
  // the grouped gate/up kernel sets kStatusF16Range when an activation or a
  // SwiGLU output does not fit its fp16 matrix-core operand
  uint32_t* status;
  int status_reset;
  // GEMV gate/up of a streamed FFN (the slot pool's misses copied by the
  // kernel's first workgroups; stream.first.list == nullptr: none)
  StreamCopy stream;
};
constexpr uint32_t kStatusF16Range = 1u;
constexpr uint32_t kStatusStreamWait = 2u;   // a streamed gate/up row gave up waiting for its copy

// Units of the grouped family, written by the bucketing kernel.  A unit is up
// to 16 rows of one expert: the shared expert's units come first (rows
// T*K + 16u .. , tokens 16u ..), then every routed expert in ascending index,
// its sorted rows cut into runs of 16.  Record = kUnitInts int32:
// {row0, mc, expert (-1 = shared), 0, token[0..15]} (tokens beyond mc unset).
constexpr int kUnitInts = 20;
struct UnitPlan {
  int32_t* units;
  int32_t* n_units;
  int T, K;
  int shared;                 // 1 when the layer has a shared expert
  uint32_t* status_reset;     // non-null: the call's status word, cleared here
};
// The grouped kernels run kGridTiles workgroups (one per CU, a multiple of 8).
// Logical workgroup w takes the contiguous part [w L / W, (w+1) L / W) of the
// list of all L tiles (W = kGridTiles, a power of two).
constexpr int kGridTiles = 256;
constexpr int kGemvSplit = 2;   // GEMV gate/up: hidden-dimension splits per pair-tile
constexpr int kGridTilesLog2 = 8;
constexpr int kSubTokens = 16;
// limits of the grouped family (larger shapes use the GEMV family)
constexpr int kGroupedMaxH = 2048;
constexpr int kGroupedMaxInter = 512;
inline int max_units(int T, int K, int E, bool shared) {
  const int rows = T * K;
  const int n_act = rows < E ? rows : E;
  return n_act + rows / kSubTokens + (shared ? (T + kSubTokens - 1) / kSubTokens : 0);
}

// Router logits.  The matrix-core path (T >= kRouterMfmaMinTokens) splits
// the hidden dimension into n_part slices (n_part <= kRouterMaxParts) and
// writes unbiased partial sums part[p][t][row] of all E+1 rows (row E, the
// shared gate, from vector-unit products).  The per-row path writes finished
// logits of all E+1 rows (bias included) as a single part.
struct RouterParts {
  int n_part;
  bool biased;   // bias already added
};
hipError_t launch_router_logits(int act, const uint16_t* x, const uint16_t* wr, const float* bias, float* part,
                                int T, int H, int E, hipStream_t s, RouterParts* out);
// Router of a layer after the first in a decode-sized stack with the
// previous layer's combine, residual and normalisation folded in (the GEMV
// family's rows yrow [T*K + T][H], weights w [T][K], gamma [T]):
// r_dst = r_src + y, x_out = rne(r_dst / rms(r_dst)), y_out = y (optional),
// logits of x_out as launch_router_logits writes them (one biased part).
// r_dst must differ from r_src.  Fits for T * H <= 32768 (x of every token
// in LDS) and T below the matrix-core router's size.
inline bool router_combine_fits(int T, int H) {
  return T >= 1 && T < kRouterMfmaMinTokens && static_cast<long long>(T) * H <= 32768;
}
hipError_t launch_router_combine(int act, const uint16_t* wr, const float* bias, float* logits, int T, int H, int E,
                                 int K, bool has_shared, const float* yrow, const float* w, const float* gamma,
                                 const float* r_src, float* r_dst, uint16_t* x_out, float* y_out, hipStream_t s,
                                 RouterParts* out);
// Top-K over z[t][e] = sum_p part[p][t][e] (p ascending) + bias[e] (bias may
// be null); the shared-gate logit is column E, summed the same way.  Writes
// the selection, the renormalised weights, the shared gate (when gamma is
// non-null) and, when logits is non-null, the logits themselves.
hipError_t launch_topk(const float* part, int n_part, const float* bias, int T, int E, int K, int32_t* idx, float* w,
                       float* gamma, float* logits, hipStream_t s);
hipError_t launch_permute(const int32_t* idx, int n, int E, int32_t* off, int32_t* perm, int32_t* inv,
                          const UnitPlan* plan, hipStream_t s);

hipError_t launch_gateup_gemv(int act, const FfnArgs& a, hipStream_t s);
hipError_t launch_down_gemv(const FfnArgs& a, hipStream_t s);
hipError_t launch_gateup_grouped(int act, const FfnArgs& a, hipStream_t s);
hipError_t launch_down_grouped(const FfnArgs& a, hipStream_t s);

// y[t] = sum_k w[t,k] yrow[row(t,k)] + gamma[t] yrow[T*K+t]; row(t,k) = inv ? inv[t*K+k] : t*K+k.
// With r != nullptr also the stack epilogue (r = r_in + y, r_in == nullptr
// meaning r itself; x_next = rne(r / rms(r))).
hipError_t launch_combine(int act, const float* yrow, const int32_t* inv, const float* w, const float* gamma,
                          int T, int K, int H, bool has_shared, float* y, float* r, uint16_t* x_next,
                          hipStream_t s, const float* r_in = nullptr);
hipError_t launch_epilogue(int act, const float* y, float* r, uint16_t* x_next, int T, int H, hipStream_t s);

}  // namespace moe
