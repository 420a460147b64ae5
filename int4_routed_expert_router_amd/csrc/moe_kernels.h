// Internal launch functions of the MoE kernels (host side).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxH = 8192;        // hidden size limit (router keeps a row in registers)
constexpr int kMaxInter = 4096;    // intermediate size limit (down GEMV stages h in LDS)
constexpr int kMaxExperts = 1024;  // top-k holds E/64 logits per lane; bucketing uses one workgroup
constexpr int kMaxTopK = 64;       // one selected expert per lane
constexpr int kRouterMfmaMinTokens = 16;  // router GEMM on the matrix cores from this batch size

// Routed rows of a batch: row j < T*K is (token j/K, rank j%K) in slot order,
// or the r-th row of the expert-sorted order in the grouped family; rows
// T*K + t (t < T) are the shared expert's.
struct FfnArgs {
  const uint16_t* x;          // [T][H] activations
  const int32_t* topk_idx;    // [T][K]
  const uint8_t* experts;     // routed blob base
  uint64_t stride;            // blob stride when offsets == nullptr
  const uint64_t* offsets;    // [E] byte offsets or nullptr
  const uint8_t* shared;      // shared blob or nullptr
  float* h;                   // [rows][hstride] SwiGLU activations
  float* yrow;                // [rows][H] per-row expert outputs (unweighted)
  // grouped family
  const int32_t* perm;        // [T*K] sorted row -> slot t*K+k
  const int32_t* expert_off;  // [E+1]
  const int32_t* active;      // active experts, most tokens first
  const int32_t* n_active;    // [1]
  const int32_t* tok_sorted;  // [T*K] token of each sorted row
  const int4* work_gu;        // gate/up work items (see WorkLists)
  const int4* work_d;         // down work items
  const int32_t* n_work;      // [2] number of gate/up and down work items
  int T, H, K, I, Is, G, E;
  int hstride;                // max(I, Is)
};

// Work lists of the grouped kernels, built by the bucketing kernel.  A unit
// is (expert, block of output rows); it splits into sub-items of up to 16
// tokens.  Item = int4 {row0, mc | block << 8, expert (-1 = shared), 0}: rows
// row0..row0+mc-1 of the row space (sorted routed rows, then T*K + t for the
// shared expert).  Units run longest first (shared, then experts by
// descending token count).  When the blocks per unit are a multiple of 8,
// item index = 8 * position + block % 8 with the sub-items of a unit at
// consecutive positions, so a persistent grid whose size is a multiple of 8
// runs them on one XCD.
struct WorkLists {
  int32_t* tok_sorted;
  int4* work_gu;
  int4* work_d;
  int32_t* n_work;
  int T, K;
  int nb_gu, nb_gu_s;   // gate/up blocks (64 rows of I) per routed / shared unit
  int nb_d, nb_d_s;     // down blocks (256 rows of H) per routed / shared unit
};
constexpr int kSubTokens = 16;
constexpr int kDownBlockRows = 256;
// limits of the grouped family (larger shapes use the GEMV family)
constexpr int kGroupedMaxH = 2048;
constexpr int kGroupedMaxInter = 512;
inline int work_upper(int nb, int nb_s, int T, int K, int E) {
  const int rows = T * K;
  const int n_act = rows < E ? rows : E;
  return nb * ((rows + kSubTokens - 1) / kSubTokens + n_act) + nb_s * ((T + kSubTokens - 1) / kSubTokens);
}

hipError_t launch_router_logits(int act, const uint16_t* x, const uint16_t* wr, const float* bias, float* logits,
                                int T, int H, int E, hipStream_t s);
hipError_t launch_topk(const float* logits, int T, int E, int K, int32_t* idx, float* w, float* gamma,
                       hipStream_t s);
hipError_t launch_permute(const int32_t* idx, int n, int E, int32_t* off, int32_t* perm, int32_t* inv,
                          int32_t* active, int32_t* n_active, const WorkLists* wl, hipStream_t s);

hipError_t launch_gateup_gemv(int act, const FfnArgs& a, hipStream_t s);
hipError_t launch_down_gemv(const FfnArgs& a, hipStream_t s);
hipError_t launch_gateup_grouped(int act, const FfnArgs& a, hipStream_t s);
hipError_t launch_down_grouped(const FfnArgs& a, hipStream_t s);

// y[t] = sum_k w[t,k] yrow[row(t,k)] + gamma[t] yrow[T*K+t]; row(t,k) = inv ? inv[t*K+k] : t*K+k.
// With r != nullptr also the stack epilogue (r += y; x_next = rne(r / rms(r))).
hipError_t launch_combine(int act, const float* yrow, const int32_t* inv, const float* w, const float* gamma,
                          int T, int K, int H, bool has_shared, float* y, float* r, uint16_t* x_next,
                          hipStream_t s);
hipError_t launch_epilogue(int act, const float* y, float* r, uint16_t* x_next, int T, int H, hipStream_t s);

}  // namespace moe
