// C ABI of the MoE library: validation, workspace layout, kernel sequencing.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "devpool.h"
#include "moe_common.h"
#include "moe.h"
#include "moe_kernels.h"
#include "moe_slotpool.h"

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}
moe_status ok() {
  g_err[0] = '\0';
  return MOE_OK;
}
moe_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}
// Prefixes the current message with "<what> <layer>: " (the message is
// copied first: it lives in the buffer being written).
moe_status fail_layer(moe_status code, const char* what, int layer) {
  char msg[sizeof(g_err)];
  snprintf(msg, sizeof(msg), "%s", g_err);
  return fail(code, "%s %d: %s", what, layer, msg);
}

struct KernelTimer {
  std::vector<hipEvent_t> begin, end;
  int kind = 0;
};
thread_local KernelTimer g_timer;

hipError_t timer_mark(bool at_begin, int kind, int layer, hipStream_t s) {
  if (layer < 0 || kind != g_timer.kind || layer >= static_cast<int>(g_timer.begin.size())) return hipSuccess;
  return hipEventRecord(at_begin ? g_timer.begin[layer] : g_timer.end[layer], s);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// weight_bits 0 means 4 (a zero-initialised descriptor describes int4 experts)
int wbits(const moe_layer_desc* d) { return d->weight_bits == 8 ? 8 : 4; }
using moe::blob_size;

bool grouped_fits(const moe_layer_desc* d);

moe_status check_desc(const moe_layer_desc* d) {
  if (!d) return fail(MOE_EINVAL, "desc is NULL");
  const int H = d->hidden, E = d->n_experts, K = d->top_k, I = d->inter, Is = d->shared_inter, G = d->group_size;
  if (H < 64 || H > moe::kMaxH || H % 64) return fail(MOE_ESHAPE, "hidden=%d must be a multiple of 64 in [64, %d]", H, moe::kMaxH);
  if (E < 1 || E > moe::kMaxExperts) return fail(MOE_ESHAPE, "n_experts=%d must be in [1, %d]", E, moe::kMaxExperts);
  if (K < 1 || K > E || K > moe::kMaxTopK) return fail(MOE_ESHAPE, "top_k=%d must be in [1, min(E, %d)]", K, moe::kMaxTopK);
  if (I < 64 || I > moe::kMaxInter || I % 64) return fail(MOE_ESHAPE, "inter=%d must be a multiple of 64 in [64, %d]", I, moe::kMaxInter);
  if (Is != 0 && (Is < 64 || Is > moe::kMaxInter || Is % 64))
    return fail(MOE_ESHAPE, "shared_inter=%d must be 0 or a multiple of 64 in [64, %d]", Is, moe::kMaxInter);
  if (G != 32 && G != 64 && G != 128) return fail(MOE_ESHAPE, "group_size=%d must be 32, 64 or 128", G);
  if (H % G || I % G || (Is && Is % G)) return fail(MOE_ESHAPE, "group_size=%d must divide hidden, inter and shared_inter", G);
  if (d->act_dtype != MOE_F16 && d->act_dtype != MOE_BF16) return fail(MOE_EINVAL, "act_dtype=%d is not MOE_F16/MOE_BF16", d->act_dtype);
  if (d->path < MOE_PATH_AUTO || d->path > MOE_PATH_GROUPED) return fail(MOE_EINVAL, "path=%d is not a MOE_PATH_*", d->path);
  if (d->weight_bits != 0 && d->weight_bits != 4 && d->weight_bits != 8)
    return fail(MOE_ESHAPE, "weight_bits=%d must be 4 (or 0) or 8", d->weight_bits);
  if (d->path == MOE_PATH_GROUPED && !grouped_fits(d))
    return fail(MOE_ESHAPE, "the grouped family needs hidden <= %d and inter, shared_inter <= %d", moe::kGroupedMaxH,
                moe::kGroupedMaxInter);
  return MOE_OK;
}

moe_status check_weights(const moe_layer_desc* d, const moe_layer_weights* w) {
  if (!w) return fail(MOE_EINVAL, "weights is NULL");
  if (!w->router_w || !aligned(w->router_w, 16)) return fail(MOE_EINVAL, "router_w must be a 16-byte aligned device pointer");
  if (!w->experts || !aligned(w->experts, 256)) return fail(MOE_EINVAL, "experts must be a 256-byte aligned device pointer");
  if (!w->expert_offset) {
    if (w->expert_stride % 256 || w->expert_stride < blob_size(d->hidden, d->inter, d->group_size, wbits(d)))
      return fail(MOE_EINVAL, "expert_stride=%llu must be a multiple of 256 and >= %llu",
                  (unsigned long long)w->expert_stride,
                  (unsigned long long)blob_size(d->hidden, d->inter, d->group_size, wbits(d)));
  }
  if (d->shared_inter > 0 && (!w->shared || !aligned(w->shared, 256)))
    return fail(MOE_EINVAL, "shared blob must be a 256-byte aligned device pointer when shared_inter > 0");
  return MOE_OK;
}

size_t al(size_t v) { return (v + 255) & ~size_t(255); }

struct Ws {
  size_t logits, idx, w, gamma, off, perm, inv, units, nunits, h, hsum, yrow, pre, status, rres, total;
};

Ws layout(const moe_layer_desc* d, int T) {
  const size_t E = d->n_experts, K = d->top_k, H = d->hidden;
  const size_t hstride = d->inter > d->shared_inter ? d->inter : d->shared_inter;
  const size_t rows = T * K + (d->shared_inter ? T : 0);
  Ws s{};
  size_t o = 0;
  s.logits = o; o += al(moe::kRouterMaxParts * T * (E + 1) * 4);   // router partial sums
  s.idx = o; o += al(T * K * 4);
  s.w = o; o += al(T * K * 4);
  s.gamma = o; o += al(T * 4);
  s.off = o; o += al((E + 1) * 4);
  s.perm = o; o += al(T * K * 4);
  s.inv = o; o += al(T * K * 4);
  s.units = o; o += al(4ull * moe::kUnitInts * moe::max_units(T, d->top_k, d->n_experts, d->shared_inter > 0));
  s.nunits = o; o += al(16);
  // grouped: fp16 h (2 B per element); GEMV: splits of fp32 (gate, up)
  s.h = o; o += al(rows * hstride * 4 * 2 * moe::kGemvSplit);
  s.hsum = o; o += al(rows * (hstride / 16) * 4);
  s.yrow = o; o += al(rows * H * 4);
  s.pre = o; o += al(T * K * 8 + T * 4);   // pre-gated selection: idx, w, gamma
  s.status = o; o += al(4);                 // status word of the last call (MOE_FLAG_*)
  s.rres = o; o += al(static_cast<size_t>(T) * H * 4);   // second residual buffer of decode stacks
  s.total = o;
  return s;
}

template <class T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

moe_status check_ws(const moe_layer_desc* d, int T, void* ws, size_t ws_bytes, Ws& L) {
  L = layout(d, T);
  if (!ws || !aligned(ws, 256)) return fail(MOE_EINVAL, "workspace must be a 256-byte aligned device pointer");
  if (ws_bytes < L.total) return fail(MOE_EWORKSPACE, "workspace of %zu bytes < required %zu", ws_bytes, L.total);
  return MOE_OK;
}

bool grouped_fits(const moe_layer_desc* d) {
  return d->hidden <= moe::kGroupedMaxH && d->inter <= moe::kGroupedMaxInter &&
         d->shared_inter <= moe::kGroupedMaxInter;
}

bool use_grouped(const moe_layer_desc* d, int T) {
  if (d->path == MOE_PATH_GEMV) return false;
  if (d->path == MOE_PATH_GROUPED) return true;
  return static_cast<long long>(T) * d->top_k > MOE_GEMV_MAX_ROWS && grouped_fits(d);
}

// The router kernel alone: its logit slices go to part.
moe_status do_router(const moe_layer_desc* d, const moe_layer_weights* w, const void* x, int T, float* part,
                     hipStream_t s, int layer, moe::RouterParts* rp) {
  hipError_t e = timer_mark(true, MOE_TIME_ROUTER, layer, s);
  *rp = moe::RouterParts{1, true};
  if (e == hipSuccess)
    e = moe::launch_router_logits(d->act_dtype, static_cast<const uint16_t*>(x), w->router_w, w->router_bias, part, T,
                                  d->hidden, d->n_experts, s, rp);
  if (e == hipSuccess) e = timer_mark(false, MOE_TIME_ROUTER, layer, s);
  if (e != hipSuccess) return hip_fail(e, "router kernel launch");
  return MOE_OK;
}

moe_status do_route(const moe_layer_desc* d, const moe_layer_weights* w, const void* x, int T, int32_t* idx,
                    float* tw, float* gamma, float* part, float* logits_out, hipStream_t s, int layer = -1) {
  moe::RouterParts rp{};
  moe_status st = do_router(d, w, x, T, part, s, layer, &rp);
  if (st) return st;
  hipError_t e = moe::launch_topk(part, rp.n_part, rp.biased ? nullptr : w->router_bias, T, d->n_experts, d->top_k,
                                  idx, tw, gamma, logits_out, s);
  if (e != hipSuccess) return hip_fail(e, "top-k kernel launch");
  return MOE_OK;
}

// Top-K fused into the batch-1 gate/up GEMV: the router's slices and the
// buffers the selection is written to.
struct FusedTopk {
  const float* part;
  moe::RouterParts rp;
  int32_t* idx;
  float* w;
  float* gamma;
};

bool fuse_topk(const moe_layer_desc* d, int T) { return !use_grouped(d, T) && d->n_experts <= 512; }

// Decode-sized stacks (GEMV family, batches below the matrix-core router's
// size): the combine, residual and normalisation of layer l run inside the
// router of layer l + 1 (launch_router_combine), and one combine follows the
// last layer, so a layer is three launches (router, gate/up with the top-K,
// down).  The residual alternates between the caller's r and a workspace
// buffer (layer l's input residual in buffer l & 1); the last combine
// writes the caller's r.
bool fold_combine(const moe_layer_desc* d, int T) {
  return !use_grouped(d, T) && moe::router_combine_fits(T, d->hidden);
}

// The previous layer's outputs that the next router combines.
struct PrevLayer {
  const float* w;
  const float* gamma;
  const float* r_src;
  float* r_dst;
  float* y_out;
};

moe_status do_router_combine(const moe_layer_desc* d, const moe_layer_weights* w, int T, float* part,
                             const float* yrow, const PrevLayer& pv, void* x_out, hipStream_t s, int layer,
                             moe::RouterParts* rp) {
  hipError_t e = timer_mark(true, MOE_TIME_ROUTER, layer, s);
  if (e == hipSuccess)
    e = moe::launch_router_combine(d->act_dtype, w->router_w, w->router_bias, part, T, d->hidden, d->n_experts,
                                   d->top_k, d->shared_inter > 0, yrow, pv.w, pv.gamma, pv.r_src, pv.r_dst,
                                   static_cast<uint16_t*>(x_out), pv.y_out, s, rp);
  if (e == hipSuccess) e = timer_mark(false, MOE_TIME_ROUTER, layer, s);
  if (e != hipSuccess) return hip_fail(e, "router + combine kernel launch");
  return MOE_OK;
}

// reset_status: this FFN is the first of the call, so its first kernel clears
// the call's status word (the grouped gate/up kernel may then set it)
// skip_combine: leave the expert rows in the workspace for the next layer's
// router (fold_combine).
moe_status do_ffn(const moe_layer_desc* d, const moe_layer_weights* w, const void* x, int T, const int32_t* idx,
                  const float* tw, const float* gamma, float* y, float* r, void* x_next, void* ws, const Ws& L,
                  hipStream_t s, bool reset_status, int layer = -1, const FusedTopk* fz = nullptr,
                  bool skip_combine = false, const moe::StreamCopy* streamed = nullptr) {
  moe::FfnArgs a{};
  // a streamed FFN's copies run in the GEMV gate/up kernel
  if (streamed != nullptr && (use_grouped(d, T) || fz != nullptr))
    return fail(MOE_EINVAL, "a streamed FFN needs the GEMV family without the fused top-K");
  if (streamed != nullptr) a.stream = *streamed;
  a.status = at<uint32_t>(ws, L.status);
  a.x = static_cast<const uint16_t*>(x);
  a.topk_idx = idx;
  a.experts = w->experts;
  a.stride = w->expert_stride;
  a.offsets = w->expert_offset;
  a.shared = w->shared;
  a.h = at<float>(ws, L.h);
  a.yrow = at<float>(ws, L.yrow);
  a.T = T;
  a.H = d->hidden;
  a.K = d->top_k;
  a.I = d->inter;
  a.Is = d->shared_inter;
  a.G = d->group_size;
  a.E = d->n_experts;
  a.hstride = d->inter > d->shared_inter ? d->inter : d->shared_inter;
  a.bits = wbits(d);
  if (fz != nullptr) {
    a.route_part = fz->part;
    a.route_bias = fz->rp.biased ? nullptr : w->router_bias;
    a.route_nparts = fz->rp.n_part;
    a.sel_idx = fz->idx;
    a.sel_w = fz->w;
    a.sel_gamma = fz->gamma;
  }
  const int32_t* inv = nullptr;
  hipError_t e;
  if (use_grouped(d, T)) {
    a.units = at<int32_t>(ws, L.units);
    a.n_units = at<int32_t>(ws, L.nunits);
    a.hsum = at<float>(ws, L.hsum);
    moe::UnitPlan plan{};
    plan.units = at<int32_t>(ws, L.units);
    plan.n_units = at<int32_t>(ws, L.nunits);
    plan.T = T;
    plan.K = d->top_k;
    plan.shared = d->shared_inter > 0 ? 1 : 0;
    plan.status_reset = reset_status ? a.status : nullptr;
    e = moe::launch_permute(idx, T * d->top_k, d->n_experts, at<int32_t>(ws, L.off), at<int32_t>(ws, L.perm),
                            at<int32_t>(ws, L.inv), &plan, s);
    if (e != hipSuccess) return hip_fail(e, "permute kernel launch");
    e = timer_mark(true, MOE_TIME_GATEUP, layer, s);
    if (e == hipSuccess) e = moe::launch_gateup_grouped(d->act_dtype, a, s);
    if (e == hipSuccess) e = timer_mark(false, MOE_TIME_GATEUP, layer, s);
    if (e != hipSuccess) return hip_fail(e, "grouped gate/up kernel launch");
    e = timer_mark(true, MOE_TIME_DOWN, layer, s);
    if (e == hipSuccess) e = moe::launch_down_grouped(a, s);
    if (e == hipSuccess) e = timer_mark(false, MOE_TIME_DOWN, layer, s);
    if (e != hipSuccess) return hip_fail(e, "grouped down kernel launch");
    inv = at<int32_t>(ws, L.inv);
  } else {
    a.status_reset = reset_status ? 1 : 0;
    e = timer_mark(true, MOE_TIME_GATEUP, layer, s);
    if (e == hipSuccess) e = moe::launch_gateup_gemv(d->act_dtype, a, s);
    if (e == hipSuccess) e = timer_mark(false, MOE_TIME_GATEUP, layer, s);
    if (e != hipSuccess) return hip_fail(e, "gate/up GEMV kernel launch");
    e = timer_mark(true, MOE_TIME_DOWN, layer, s);
    if (e == hipSuccess) e = moe::launch_down_gemv(a, s);
    if (e == hipSuccess) e = timer_mark(false, MOE_TIME_DOWN, layer, s);
    if (e != hipSuccess) return hip_fail(e, "down GEMV kernel launch");
  }
  if (skip_combine) return MOE_OK;
  e = moe::launch_combine(d->act_dtype, a.yrow, inv, tw, gamma, T, d->top_k, d->hidden, d->shared_inter > 0, y, r,
                          static_cast<uint16_t*>(x_next), s);
  if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  return MOE_OK;
}

}  // namespace

namespace moe {
moe_status set_error(moe_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}
}  // namespace moe

struct moe_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

extern "C" {

const char* moe_last_error(void) { return g_err; }

const char* moe_version(void) { return "int4_routed_expert_router_amd 0.1 (gfx950)"; }

uint64_t moe_blob_bytes_q(int32_t hidden, int32_t inter, int32_t group_size, int32_t bits) {
  if (hidden <= 0 || inter <= 0 || hidden % 64 || inter % 64) return 0;
  if ((group_size != 32 && group_size != 64 && group_size != 128) || hidden % group_size || inter % group_size)
    return 0;
  if (bits != 4 && bits != 8) return 0;
  return blob_size(hidden, inter, group_size, bits);
}

uint64_t moe_blob_bytes(int32_t hidden, int32_t inter, int32_t group_size) {
  return moe_blob_bytes_q(hidden, inter, group_size, 4);
}

moe_status moe_pack_expert_q(int32_t H, int32_t I, int32_t G, int32_t bits, const uint8_t* gate_q,
                             const uint16_t* gate_s, const uint16_t* gate_b, const uint8_t* up_q,
                             const uint16_t* up_s, const uint16_t* up_b, const uint8_t* down_q,
                             const uint16_t* down_s, const uint16_t* down_b, uint8_t* blob_out) {
  if (moe_blob_bytes_q(H, I, G, bits) == 0)
    return fail(MOE_ESHAPE, "bad blob shape H=%d I=%d G=%d bits=%d", H, I, G, bits);
  if (!gate_q || !gate_s || !gate_b || !up_q || !up_s || !up_b || !down_q || !down_s || !down_b || !blob_out)
    return fail(MOE_EINVAL, "NULL pointer");
  const size_t nq = static_cast<size_t>(I) * H;
  if (bits == 4)
    for (size_t i = 0; i < nq; ++i)
      if ((gate_q[i] | up_q[i] | down_q[i]) > 15) return fail(MOE_EINVAL, "q value above 15 at element %zu", i);
  memset(blob_out, 0, blob_size(H, I, G, bits));
  // value sections, for pair-tile p, chunk c, lane l = 16 kb + n, tile, half ks
  // and value j (column 64c + 32ks + 8kb + j): int4 puts it in nibble
  // (j>>1) + 4(j&1) of word 2 tile + ks of the lane's 16 bytes in a 1 KiB
  // block; int8 puts it in byte 8 ks + j of the lane's 16 bytes in plane
  // `tile` of a 2 KiB block
  auto pack_section = [&](uint8_t* sec, int n_pairs, int in_dim, const uint8_t* qa, int row_a0_stride,
                          const uint8_t* qb, bool gu) {
    const int nc = in_dim / 64;
    for (int p = 0; p < n_pairs; ++p)
      for (int c = 0; c < nc; ++c)
        for (int l = 0; l < 64; ++l) {
          const int n = l % 16, kb = l / 16;
          for (int wd = 0; wd < 4; ++wd) {
            const int tile = wd >> 1, ks = wd & 1;
            int row;
            const uint8_t* q;
            if (gu) {
              row = 16 * p + n;
              q = tile ? qb : qa;
            } else {
              row = 32 * p + 16 * tile + n;
              q = qa;
            }
            const uint8_t* src = q + static_cast<size_t>(row) * in_dim + 64 * c + 32 * ks + 8 * kb;
            if (bits == 8) {
              memcpy(sec + (static_cast<size_t>(p) * nc + c) * 2048 + 1024 * tile + 16 * l + 8 * ks, src, 8);
              continue;
            }
            uint32_t word = 0;
            for (int j = 0; j < 8; ++j) word |= static_cast<uint32_t>(src[j]) << (4 * ((j >> 1) + 4 * (j & 1)));
            uint8_t* dst = sec + (static_cast<size_t>(p) * nc + c) * 1024 + 16 * l + 4 * wd;
            memcpy(dst, &word, 4);
          }
        }
    (void)row_a0_stride;
  };
  pack_section(blob_out, I / 16, H, gate_q, 0, up_q, true);
  pack_section(blob_out + static_cast<size_t>(I) * H * bits / 4, H / 32, I, down_q, 0, nullptr, false);
  auto pack_scales = [&](uint8_t* sec, int n_pairs, int in_dim, const uint16_t* sa, const uint16_t* ba,
                         const uint16_t* sb_, const uint16_t* bb, bool gu) {
    const int ng = in_dim / G;
    for (int p = 0; p < n_pairs; ++p)
      for (int g = 0; g < ng; ++g)
        for (int n = 0; n < 16; ++n) {
          uint16_t v[4];
          if (gu) {
            const size_t r = static_cast<size_t>(16 * p + n) * ng + g;
            v[0] = sa[r];
            v[1] = ba[r];
            v[2] = sb_[r];
            v[3] = bb[r];
          } else {
            const size_t ra = static_cast<size_t>(32 * p + n) * ng + g;
            const size_t rb = static_cast<size_t>(32 * p + 16 + n) * ng + g;
            v[0] = sa[ra];
            v[1] = ba[ra];
            v[2] = sa[rb];
            v[3] = ba[rb];
          }
          memcpy(sec + ((static_cast<size_t>(p) * ng + g) * 16 + n) * 8, v, 8);
        }
  };
  const size_t gu_s = 3ull * I * H * bits / 8, d_s = gu_s + 8ull * I * H / G;
  pack_scales(blob_out + gu_s, I / 16, H, gate_s, gate_b, up_s, up_b, true);
  pack_scales(blob_out + d_s, H / 32, I, down_s, down_b, nullptr, nullptr, false);
  return ok();
}

moe_status moe_pack_expert(int32_t H, int32_t I, int32_t G, const uint8_t* gate_q, const uint16_t* gate_s,
                           const uint16_t* gate_b, const uint8_t* up_q, const uint16_t* up_s, const uint16_t* up_b,
                           const uint8_t* down_q, const uint16_t* down_s, const uint16_t* down_b,
                           uint8_t* blob_out) {
  return moe_pack_expert_q(H, I, G, 4, gate_q, gate_s, gate_b, up_q, up_s, up_b, down_q, down_s, down_b, blob_out);
}

moe_status moe_workspace_bytes(const moe_layer_desc* d, int32_t n_tokens, size_t* bytes) {
  moe_status st = check_desc(d);
  if (st) return st;
  if (n_tokens < 0) return fail(MOE_ESHAPE, "n_tokens=%d < 0", n_tokens);
  if (!bytes) return fail(MOE_EINVAL, "bytes is NULL");
  *bytes = layout(d, n_tokens).total;
  return ok();
}

moe_status moe_workspace_status(const moe_layer_desc* d, int32_t n_tokens, size_t* offset) {
  moe_status st = check_desc(d);
  if (st) return st;
  if (n_tokens < 0) return fail(MOE_ESHAPE, "n_tokens=%d < 0", n_tokens);
  if (!offset) return fail(MOE_EINVAL, "offset is NULL");
  *offset = layout(d, n_tokens).status;
  return ok();
}

moe_status moe_route(const moe_layer_desc* d, const moe_layer_weights* w, const void* x, int32_t T,
                     int32_t* topk_idx, float* topk_w, float* shared_gate, float* logits_or_null, void* ws,
                     size_t ws_bytes, moe_stream stream) {
  moe_status st = check_desc(d);
  if (st) return st;
  if ((st = check_weights(d, w))) return st;
  if (T < 0) return fail(MOE_ESHAPE, "n_tokens=%d < 0", T);
  if (T == 0) return ok();
  if (!x || !aligned(x, 16)) return fail(MOE_EINVAL, "x must be a 16-byte aligned device pointer");
  if (!topk_idx || !topk_w) return fail(MOE_EINVAL, "topk_idx and topk_w are required");
  Ws L;
  if ((st = check_ws(d, T, ws, ws_bytes, L))) return st;
  float* gamma = shared_gate ? shared_gate : at<float>(ws, L.gamma);
  st = do_route(d, w, x, T, topk_idx, topk_w, gamma, at<float>(ws, L.logits), logits_or_null,
                reinterpret_cast<hipStream_t>(stream));
  return st ? st : ok();
}

moe_status moe_permute(const moe_layer_desc* d, const int32_t* topk_idx, int32_t T, int32_t* expert_off,
                       int32_t* perm, int32_t* inv_or_null, void* ws, size_t ws_bytes, moe_stream stream) {
  moe_status st = check_desc(d);
  if (st) return st;
  if (T < 0) return fail(MOE_ESHAPE, "n_tokens=%d < 0", T);
  if (T == 0) return ok();
  if (!topk_idx || !expert_off || !perm) return fail(MOE_EINVAL, "topk_idx, expert_off and perm are required");
  Ws L;
  if ((st = check_ws(d, T, ws, ws_bytes, L))) return st;
  hipError_t e = moe::launch_permute(topk_idx, T * d->top_k, d->n_experts, expert_off, perm, inv_or_null, nullptr,
                                     reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "permute kernel launch");
  return ok();
}

moe_status moe_expert_ffn(const moe_layer_desc* d, const moe_layer_weights* w, const void* x, int32_t T,
                          const int32_t* topk_idx, const float* topk_w, const float* shared_gate, float* y,
                          void* ws, size_t ws_bytes, moe_stream stream) {
  moe_status st = check_desc(d);
  if (st) return st;
  if ((st = check_weights(d, w))) return st;
  if (T < 0) return fail(MOE_ESHAPE, "n_tokens=%d < 0", T);
  if (T == 0) return ok();
  if (!x || !aligned(x, 16)) return fail(MOE_EINVAL, "x must be a 16-byte aligned device pointer");
  if (!topk_idx || !topk_w || !y) return fail(MOE_EINVAL, "topk_idx, topk_w and y are required");
  if (d->shared_inter > 0 && !shared_gate) return fail(MOE_EINVAL, "shared_gate is required when shared_inter > 0");
  Ws L;
  if ((st = check_ws(d, T, ws, ws_bytes, L))) return st;
  st = do_ffn(d, w, x, T, topk_idx, topk_w, shared_gate, y, nullptr, nullptr, ws, L,
              reinterpret_cast<hipStream_t>(stream), true);
  return st ? st : ok();
}

moe_status moe_layer_forward(const moe_layer_desc* d, const moe_layer_weights* w, const void* x, int32_t T,
                             float* y, int32_t* idx_out, float* w_out, float* gamma_out, void* ws,
                             size_t ws_bytes, moe_stream stream) {
  moe_status st = check_desc(d);
  if (st) return st;
  if ((st = check_weights(d, w))) return st;
  if (T < 0) return fail(MOE_ESHAPE, "n_tokens=%d < 0", T);
  if (T == 0) return ok();
  if (!x || !aligned(x, 16)) return fail(MOE_EINVAL, "x must be a 16-byte aligned device pointer");
  if (!y) return fail(MOE_EINVAL, "y is required");
  Ws L;
  if ((st = check_ws(d, T, ws, ws_bytes, L))) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int32_t* idx = idx_out ? idx_out : at<int32_t>(ws, L.idx);
  float* tw = w_out ? w_out : at<float>(ws, L.w);
  float* gamma = gamma_out ? gamma_out : at<float>(ws, L.gamma);
  if (fuse_topk(d, T)) {
    FusedTopk fz{at<float>(ws, L.logits), {}, idx, tw, gamma};
    if ((st = do_router(d, w, x, T, at<float>(ws, L.logits), s, -1, &fz.rp))) return st;
    if ((st = do_ffn(d, w, x, T, idx, tw, gamma, y, nullptr, nullptr, ws, L, s, true, -1, &fz))) return st;
    return ok();
  }
  if ((st = do_route(d, w, x, T, idx, tw, gamma, at<float>(ws, L.logits), nullptr, s))) return st;
  if ((st = do_ffn(d, w, x, T, idx, tw, gamma, y, nullptr, nullptr, ws, L, s, true))) return st;
  return ok();
}

moe_status moe_stack_epilogue(const moe_layer_desc* d, int32_t T, const float* y, float* r, void* x_next,
                              moe_stream stream) {
  moe_status st = check_desc(d);
  if (st) return st;
  if (T < 0) return fail(MOE_ESHAPE, "n_tokens=%d < 0", T);
  if (T == 0) return ok();
  if (!y || !r || !x_next) return fail(MOE_EINVAL, "y, r and x_next are required");
  hipError_t e = moe::launch_epilogue(d->act_dtype, y, r, static_cast<uint16_t*>(x_next), T, d->hidden,
                                      reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "epilogue kernel launch");
  return ok();
}

static moe_status stack_enqueue(const moe_layer_desc* d, const moe_layer_weights* layers, int32_t L_, const void* x0,
                                int32_t T, float* r, void* x_buf, void* x_all, float* y_all, int32_t* idx_all,
                                float* w_all, float* gamma_all, void* ws, size_t ws_bytes, hipStream_t s) {
  moe_status st = check_desc(d);
  if (st) return st;
  if (L_ < 0 || (L_ > 0 && !layers)) return fail(MOE_EINVAL, "bad layer array");
  if (T < 0) return fail(MOE_ESHAPE, "n_tokens=%d < 0", T);
  if (T == 0 || L_ == 0) return ok();
  if (!x0 || !aligned(x0, 16) || !r || !x_buf || !aligned(x_buf, 16))
    return fail(MOE_EINVAL, "x0, r and x_buf are required (16-byte aligned)");
  for (int l = 0; l < L_; ++l)
    if ((st = check_weights(d, &layers[l]))) return fail_layer(st, "layer", l);
  Ws L;
  if ((st = check_ws(d, T, ws, ws_bytes, L))) return st;
  const size_t TH = static_cast<size_t>(T) * d->hidden, TK = static_cast<size_t>(T) * d->top_k;
  const bool fold = fold_combine(d, T);
  if (fold && !aligned(r, 16)) return fail(MOE_EINVAL, "r must be 16-byte aligned");
  float* rbuf[2] = {r, at<float>(ws, L.rres)};
  const float* prev_w = nullptr;
  const float* prev_gamma = nullptr;
  for (int l = 0; l < L_; ++l) {
    const void* xl = (l == 0) ? x0 : x_buf;
    int32_t* idx = idx_all ? idx_all + l * TK : at<int32_t>(ws, L.idx);
    float* tw = w_all ? w_all + l * TK : at<float>(ws, L.w);
    float* gamma = gamma_all ? gamma_all + static_cast<size_t>(l) * T : at<float>(ws, L.gamma);
    float* y = y_all ? y_all + l * TH : nullptr;
    if (fold) {
      // router (layers after the first also combine the previous layer into
      // r and form this layer's x in x_buf), gate/up with the top-K, down
      FusedTopk fz{at<float>(ws, L.logits), {}, idx, tw, gamma};
      if (l == 0) {
        if ((st = do_router(d, &layers[l], xl, T, at<float>(ws, L.logits), s, l, &fz.rp))) return st;
      } else {
        const PrevLayer pv{prev_w, prev_gamma, rbuf[(l - 1) & 1], rbuf[l & 1], y_all ? y_all + (l - 1) * TH : nullptr};
        if ((st = do_router_combine(d, &layers[l], T, at<float>(ws, L.logits), at<float>(ws, L.yrow), pv, x_buf, s, l,
                                    &fz.rp)))
          return st;
      }
      if (x_all) {
        hipError_t e = hipMemcpyAsync(static_cast<uint16_t*>(x_all) + l * TH, xl, TH * 2, hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "x capture copy");
      }
      if (fuse_topk(d, T)) {
        if ((st = do_ffn(d, &layers[l], xl, T, idx, tw, gamma, y, nullptr, nullptr, ws, L, s, l == 0, l, &fz, true)))
          return st;
      } else {
        hipError_t e = moe::launch_topk(fz.part, fz.rp.n_part, fz.rp.biased ? nullptr : layers[l].router_bias, T,
                                        d->n_experts, d->top_k, idx, tw, gamma, nullptr, s);
        if (e != hipSuccess) return hip_fail(e, "top-k kernel launch");
        if ((st = do_ffn(d, &layers[l], xl, T, idx, tw, gamma, y, nullptr, nullptr, ws, L, s, l == 0, l, nullptr,
                         true)))
          return st;
      }
      prev_w = tw;
      prev_gamma = gamma;
      continue;
    }
    if (x_all) {
      hipError_t e = hipMemcpyAsync(static_cast<uint16_t*>(x_all) + l * TH, xl, TH * 2, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return hip_fail(e, "x capture copy");
    }
    if (fuse_topk(d, T)) {
      FusedTopk fz{at<float>(ws, L.logits), {}, idx, tw, gamma};
      if ((st = do_router(d, &layers[l], xl, T, at<float>(ws, L.logits), s, l, &fz.rp))) return st;
      if ((st = do_ffn(d, &layers[l], xl, T, idx, tw, gamma, y, r, x_buf, ws, L, s, l == 0, l, &fz))) return st;
      continue;
    }
    if ((st = do_route(d, &layers[l], xl, T, idx, tw, gamma, at<float>(ws, L.logits), nullptr, s, l))) return st;
    if ((st = do_ffn(d, &layers[l], xl, T, idx, tw, gamma, y, r, x_buf, ws, L, s, l == 0, l))) return st;
  }
  if (fold) {   // the last layer's combine, residual and next input
    hipError_t e = moe::launch_combine(d->act_dtype, at<float>(ws, L.yrow), nullptr, prev_w, prev_gamma, T, d->top_k,
                                       d->hidden, d->shared_inter > 0, y_all ? y_all + (L_ - 1) * TH : nullptr, r,
                                       static_cast<uint16_t*>(x_buf), s, rbuf[(L_ - 1) & 1]);
    if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  }
  return MOE_OK;
}

moe_status moe_stack_forward(const moe_layer_desc* d, const moe_layer_weights* layers, int32_t n_layers,
                             const void* x0, int32_t T, float* r, void* x_buf, void* x_all, float* y_all,
                             int32_t* idx_all, float* w_all, float* gamma_all, void* ws, size_t ws_bytes,
                             moe_stream stream) {
  moe_status st = stack_enqueue(d, layers, n_layers, x0, T, r, x_buf, x_all, y_all, idx_all, w_all, gamma_all, ws,
                                ws_bytes, reinterpret_cast<hipStream_t>(stream));
  return st ? st : ok();
}

moe_status moe_stack_graph_create(const moe_layer_desc* d, const moe_layer_weights* layers, int32_t n_layers,
                                  const void* x0, int32_t T, float* r, void* x_buf, void* x_all, float* y_all,
                                  int32_t* idx_all, float* w_all, float* gamma_all, void* ws, size_t ws_bytes,
                                  moe_stream capture_stream, moe_graph** out) {
  if (!out) return fail(MOE_EINVAL, "out is NULL");
  if (!capture_stream) return fail(MOE_EINVAL, "graph capture needs a non-NULL stream");
  *out = nullptr;
  hipStream_t s = reinterpret_cast<hipStream_t>(capture_stream);
  hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return hip_fail(e, "hipStreamBeginCapture");
  moe_status st = stack_enqueue(d, layers, n_layers, x0, T, r, x_buf, x_all, y_all, idx_all, w_all, gamma_all, ws,
                                ws_bytes, s);
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(s, &g);
  if (st) {
    if (g) hipGraphDestroy(g);
    return st;
  }
  if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
  hipGraphExec_t ex = nullptr;
  e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    hipGraphDestroy(g);
    return hip_fail(e, "hipGraphInstantiate");
  }
  moe_graph* mg = new (std::nothrow) moe_graph;
  if (!mg) {
    hipGraphExecDestroy(ex);
    hipGraphDestroy(g);
    return fail(MOE_ENOMEM, "graph handle allocation");
  }
  mg->graph = g;
  mg->exec = ex;
  *out = mg;
  return ok();
}

moe_status moe_pool_decode_step(const moe_layer_desc* d, const moe_layer_weights* layers, int32_t L_,
                                moe_slotpool* pool, uint64_t step, const void* x0, float* r, void* x_buf,
                                int32_t* idx_host, int32_t* idx_log, int32_t pregate, void* ws, size_t ws_bytes,
                                moe_stream compute) {
  moe_status st = check_desc(d);
  if (st) return st;
  if (!pool) return fail(MOE_EINVAL, "pool is NULL");
  if (L_ < 0 || (L_ > 0 && !layers)) return fail(MOE_EINVAL, "bad layer array");
  if (pregate < 0) return fail(MOE_EINVAL, "pregate=%d < 0", pregate);
  if (!x0 || !aligned(x0, 16) || !r || !x_buf || !aligned(x_buf, 16) || !idx_host)
    return fail(MOE_EINVAL, "x0, r, x_buf (16-byte aligned) and idx_host are required");
  moe_slotpool_config pc{};
  if ((st = slotpool_get_config(pool, &pc))) return st;
  if (pc.flags & MOE_POOL_HOST_ONLY) return fail(MOE_EINVAL, "the pool makes no device copies (MOE_POOL_HOST_ONLY)");
  if (pc.n_layers < L_ || pc.n_experts != d->n_experts)
    return fail(MOE_ESHAPE, "pool of %d layers x %d experts does not fit %d layers x %d experts", pc.n_layers,
                pc.n_experts, L_, d->n_experts);
  if (pc.blob_bytes < blob_size(d->hidden, d->inter, d->group_size, wbits(d)))
    return fail(MOE_ESHAPE, "pool blobs of %llu bytes are smaller than the layer's", (unsigned long long)pc.blob_bytes);
  if (L_ == 0) return ok();
  Ws L;
  if ((st = check_ws(d, 1, ws, ws_bytes, L))) return st;
  const int K = d->top_k, H = d->hidden;
  const uint64_t S = static_cast<uint64_t>(pc.slots_per_layer), E = static_cast<uint64_t>(pc.n_experts);
  auto pooled = [&](int l) {
    moe_layer_weights w = layers[l];
    w.experts = pc.device_slab + static_cast<uint64_t>(l) * S * pc.blob_stride;
    w.expert_stride = pc.blob_stride;
    w.expert_offset = pc.device_offsets + static_cast<uint64_t>(l) * E;
    return w;
  };
  for (int l = 0; l < L_; ++l) {
    moe_layer_weights w = pooled(l);
    if ((st = check_weights(d, &w))) return fail_layer(st, "layer", l);
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(compute);
  int32_t* idx = at<int32_t>(ws, L.idx);
  float* tw = at<float>(ws, L.w);
  float* gamma = at<float>(ws, L.gamma);
  int32_t* pidx = at<int32_t>(ws, L.pre);
  float* pw = at<float>(ws, L.pre + static_cast<size_t>(K) * 4);
  float* pg = at<float>(ws, L.pre + static_cast<size_t>(K) * 8);
  const size_t xbytes = static_cast<size_t>(H) * 2;
  // decode-sized: the router of layer l > 0 also combines layer l - 1 (see
  // fold_combine), forming x of layer l in slot (l - 1) & 1 of x_buf
  const bool fold = fold_combine(d, 1);
  if (fold && !aligned(r, 16)) return fail(MOE_EINVAL, "r must be 16-byte aligned");
  float* rbuf[2] = {r, at<float>(ws, L.rres)};
  for (int l = 0; l < L_; ++l) {
    void* xslot = static_cast<char*>(x_buf) + ((l - 1) & 1) * xbytes;
    const void* xl = (l == 0) ? x0 : xslot;
    void* xn = static_cast<char*>(x_buf) + (l & 1) * xbytes;
    const moe_layer_weights w = pooled(l);
    if (fold && l > 0) {
      // tw and gamma still hold layer l - 1's values: the top-K below rewrites them
      moe::RouterParts rp{};
      const PrevLayer pv{tw, gamma, rbuf[(l - 1) & 1], rbuf[l & 1], nullptr};
      if ((st = do_router_combine(d, &w, 1, at<float>(ws, L.logits), at<float>(ws, L.yrow), pv, xslot, s, -1, &rp)))
        return st;
      hipError_t e = moe::launch_topk(at<float>(ws, L.logits), rp.n_part, rp.biased ? nullptr : w.router_bias, 1,
                                      d->n_experts, K, idx, tw, gamma, nullptr, s);
      if (e != hipSuccess) return hip_fail(e, "top-k kernel launch");
    } else if ((st = do_route(d, &w, xl, 1, idx, tw, gamma, at<float>(ws, L.logits), nullptr, s))) {
      return st;
    }
    hipError_t e = hipMemcpyAsync(idx_host, idx, K * 4, hipMemcpyDeviceToHost, s);
    const bool pre = pregate > 0 && l + 1 < L_;
    const int n_pre = pregate < K ? pregate : K;   // the highest-ranked predictions
    if (pre && e == hipSuccess) {
      const moe_layer_weights wn = pooled(l + 1);
      if ((st = do_route(d, &wn, xl, 1, pidx, pw, pg, at<float>(ws, L.logits), nullptr, s))) return st;
      e = hipMemcpyAsync(idx_host + K, pidx, K * 4, hipMemcpyDeviceToHost, s);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "index read-back");
    if (idx_log) {   // [l][0] the selection, [l][1] the prediction for layer l + 1 (-1: none)
      int32_t* lg = idx_log + static_cast<size_t>(l) * 2 * K;
      memcpy(lg, idx_host, K * 4);
      for (int k = 0; k < K; ++k) lg[K + k] = (pre && k < n_pre) ? idx_host[K + k] : -1;
    }
    if ((st = slotpool_acquire(pool, l, idx_host, K, step, compute, nullptr, nullptr, nullptr)))
      return fail_layer(st, "acquire, layer", l);
    if (pre && (st = slotpool_prefetch(pool, l + 1, idx_host + K, n_pre, step, compute, nullptr, nullptr, nullptr,
                                       nullptr)))
      return fail_layer(st, "prefetch, layer", l + 1);
    if ((st = do_ffn(d, &w, xl, 1, idx, tw, gamma, nullptr, fold ? nullptr : r, fold ? nullptr : xn, ws, L, s,
                     l == 0, -1, nullptr, fold)))
      return st;
    if ((st = slotpool_release(pool, l, compute))) return fail_layer(st, "release, layer", l);
  }
  if (fold) {
    hipError_t e = moe::launch_combine(d->act_dtype, at<float>(ws, L.yrow), nullptr, tw, gamma, 1, K, H,
                                       d->shared_inter > 0, nullptr, r,
                                       reinterpret_cast<uint16_t*>(static_cast<char*>(x_buf) + ((L_ - 1) & 1) * xbytes),
                                       s, rbuf[(L_ - 1) & 1]);
    if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  }
  return ok();
}

static moe_status pool_dev_enqueue(const moe_layer_desc* d, const moe_layer_weights* layers, int32_t L_,
                                   moe_devpool* pool, const void* x0, float* r, void* x_buf, int32_t* trace,
                                   void* ws, size_t ws_bytes, hipStream_t s) {
  moe_status st = check_desc(d);
  if (st) return st;
  if (!pool) return fail(MOE_EINVAL, "pool is NULL");
  if (L_ < 0 || (L_ > 0 && !layers)) return fail(MOE_EINVAL, "bad layer array");
  if (!x0 || !aligned(x0, 16) || !r || !aligned(r, 16) || !x_buf || !aligned(x_buf, 16))
    return fail(MOE_EINVAL, "x0, r and x_buf are required (16-byte aligned)");
  const moe_slotpool_config& pc = moe::devpool_config(pool);
  if (pc.n_layers < L_ || pc.n_experts != d->n_experts)
    return fail(MOE_ESHAPE, "pool of %d layers x %d experts does not fit %d layers x %d experts", pc.n_layers,
                pc.n_experts, L_, d->n_experts);
  if (d->top_k > pc.slots_per_layer || d->top_k > 64)
    return fail(MOE_ESHAPE, "top_k=%d exceeds the pool's %d slots per layer (or 64)", d->top_k, pc.slots_per_layer);
  if (pc.blob_bytes < blob_size(d->hidden, d->inter, d->group_size, wbits(d)))
    return fail(MOE_ESHAPE, "pool blobs of %llu bytes are smaller than the layer's", (unsigned long long)pc.blob_bytes);
  if (L_ == 0) return MOE_OK;
  Ws L;
  if ((st = check_ws(d, 1, ws, ws_bytes, L))) return st;
  const int K = d->top_k, H = d->hidden;
  const uint64_t S = static_cast<uint64_t>(pc.slots_per_layer), E = static_cast<uint64_t>(pc.n_experts);
  auto pooled = [&](int l) {
    moe_layer_weights w = layers[l];
    w.experts = pc.device_slab + static_cast<uint64_t>(l) * S * pc.blob_stride;
    w.expert_stride = pc.blob_stride;
    w.expert_offset = pc.device_offsets + static_cast<uint64_t>(l) * E;
    return w;
  };
  for (int l = 0; l < L_; ++l) {
    moe_layer_weights w = pooled(l);
    if ((st = check_weights(d, &w))) return fail_layer(st, "layer", l);
  }
  int32_t* idx = at<int32_t>(ws, L.idx);
  float* tw = at<float>(ws, L.w);
  float* gamma = at<float>(ws, L.gamma);
  const size_t xbytes = static_cast<size_t>(H) * 2;
  const bool fold = fold_combine(d, 1);
  float* rbuf[2] = {r, at<float>(ws, L.rres)};
  for (int l = 0; l < L_; ++l) {
    void* xslot = static_cast<char*>(x_buf) + ((l - 1) & 1) * xbytes;
    const void* xl = (l == 0) ? x0 : xslot;
    void* xn = static_cast<char*>(x_buf) + (l & 1) * xbytes;
    const moe_layer_weights w = pooled(l);
    moe::RouterParts rp{};
    if (fold && l > 0) {
      // tw and gamma still hold layer l - 1's values: the selection below rewrites them
      const PrevLayer pv{tw, gamma, rbuf[(l - 1) & 1], rbuf[l & 1], nullptr};
      if ((st = do_router_combine(d, &w, 1, at<float>(ws, L.logits), at<float>(ws, L.yrow), pv, xslot, s, -1, &rp)))
        return st;
    } else if ((st = do_router(d, &w, xl, 1, at<float>(ws, L.logits), s, -1, &rp))) {
      return st;
    }
    // the pool's policy kernel selects the token's experts itself (the top-K
    // kernel's code) and then acquires them
    const moe::DevRoute rt{at<float>(ws, L.logits), rp.n_part, rp.biased ? nullptr : w.router_bias, tw, gamma};
    // GEMV family: the misses are copied by the gate/up kernel's first
    // workgroups, the gate/up sections first (a missed row's products wait
    // for its expert's), then the down sections, so the products overlap the
    // copies and no separate copy launch is paid.  The grouped family (a
    // forced path) copies with the copy kernel after the acquire.
    const bool streamed = !use_grouped(d, 1);
    moe::StreamCopy sc = moe::devpool_stream_copy(pool, l);
    {
      const int I = d->inter, G = d->group_size, bits = wbits(d);
      sc.first.off[0] = 0;
      sc.first.len[0] = moe::blob_d_q(H, I, bits);
      sc.first.off[1] = moe::blob_gu_s(H, I, bits);
      sc.first.len[1] = moe::blob_d_s(H, I, G, bits) - moe::blob_gu_s(H, I, bits);
      sc.second.off[0] = moe::blob_d_q(H, I, bits);
      sc.second.len[0] = moe::blob_gu_s(H, I, bits) - moe::blob_d_q(H, I, bits);
      sc.second.off[1] = moe::blob_d_s(H, I, G, bits);
      sc.second.len[1] = pc.blob_bytes - moe::blob_d_s(H, I, G, bits);
    }
    hipError_t e = moe::devpool_enqueue_acquire(pool, l, idx, K, l == L_ - 1,
                                                trace ? trace + static_cast<size_t>(l) * K * 3 : nullptr, s, &rt,
                                                !streamed);
    if (e != hipSuccess) return hip_fail(e, "pool acquire launch");
    if ((st = do_ffn(d, &w, xl, 1, idx, tw, gamma, nullptr, fold ? nullptr : r, fold ? nullptr : xn, ws, L, s,
                     l == 0, -1, nullptr, fold, streamed ? &sc : nullptr)))
      return st;
  }
  if (fold) {
    hipError_t e = moe::launch_combine(d->act_dtype, at<float>(ws, L.yrow), nullptr, tw, gamma, 1, K, H,
                                       d->shared_inter > 0, nullptr, r,
                                       reinterpret_cast<uint16_t*>(static_cast<char*>(x_buf) + ((L_ - 1) & 1) * xbytes),
                                       s, rbuf[(L_ - 1) & 1]);
    if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  }
  return MOE_OK;
}

moe_status moe_pool_decode_step_dev(const moe_layer_desc* d, const moe_layer_weights* layers, int32_t L_,
                                    moe_devpool* pool, const void* x0, float* r, void* x_buf, int32_t* trace,
                                    void* ws, size_t ws_bytes, moe_stream stream) {
  moe_status st = pool_dev_enqueue(d, layers, L_, pool, x0, r, x_buf, trace, ws, ws_bytes,
                                   reinterpret_cast<hipStream_t>(stream));
  return st ? st : ok();
}

moe_status moe_pool_graph_create(const moe_layer_desc* d, const moe_layer_weights* layers, int32_t L_,
                                 moe_devpool* pool, const void* x0, float* r, void* x_buf, int32_t* trace, void* ws,
                                 size_t ws_bytes, moe_stream capture_stream, moe_graph** out) {
  if (!out) return fail(MOE_EINVAL, "out is NULL");
  if (!capture_stream) return fail(MOE_EINVAL, "graph capture needs a non-NULL stream");
  *out = nullptr;
  hipStream_t s = reinterpret_cast<hipStream_t>(capture_stream);
  hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return hip_fail(e, "hipStreamBeginCapture");
  moe_status st = pool_dev_enqueue(d, layers, L_, pool, x0, r, x_buf, trace, ws, ws_bytes, s);
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(s, &g);
  if (st) {
    if (g) hipGraphDestroy(g);
    return st;
  }
  if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
  hipGraphExec_t ex = nullptr;
  e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    hipGraphDestroy(g);
    return hip_fail(e, "hipGraphInstantiate");
  }
  moe_graph* mg = new (std::nothrow) moe_graph;
  if (!mg) {
    hipGraphExecDestroy(ex);
    hipGraphDestroy(g);
    return fail(MOE_ENOMEM, "graph handle allocation");
  }
  mg->graph = g;
  mg->exec = ex;
  *out = mg;
  return ok();
}

moe_status moe_stack_set_kernel_events(void* const* begin, void* const* end, int32_t n_layers, int32_t kind) {
  if (n_layers < 0 || (n_layers > 0 && (!begin || !end))) return fail(MOE_EINVAL, "bad event arrays");
  if (kind < MOE_TIME_GATEUP || kind > MOE_TIME_ROUTER) return fail(MOE_EINVAL, "kind=%d is not a MOE_TIME_*", kind);
  g_timer.begin.assign(n_layers, nullptr);
  g_timer.end.assign(n_layers, nullptr);
  for (int l = 0; l < n_layers; ++l) {
    if (!begin[l] || !end[l]) return fail(MOE_EINVAL, "NULL event for layer %d", l);
    g_timer.begin[l] = static_cast<hipEvent_t>(begin[l]);
    g_timer.end[l] = static_cast<hipEvent_t>(end[l]);
  }
  g_timer.kind = kind;
  return ok();
}

moe_status moe_graph_launch(moe_graph* g, moe_stream stream) {
  if (!g) return fail(MOE_EINVAL, "graph is NULL");
  hipError_t e = hipGraphLaunch(g->exec, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hipGraphLaunch");
  return ok();
}

void moe_graph_destroy(moe_graph* g) {
  if (!g) return;
  if (g->exec) hipGraphExecDestroy(g->exec);
  if (g->graph) hipGraphDestroy(g->graph);
  delete g;
}

}  // extern "C"
