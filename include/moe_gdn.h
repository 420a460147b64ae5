/*
 * moe_gdn.h - Gated DeltaNet single-token recurrence (the step that runs
 * beside the MoE block).
 *
 * Three quarters of the layers of the models this library serves use Gated
 * DeltaNet linear attention with a fixed-size recurrent state instead of a
 * growing KV cache (page "Show HN: Run an 80B Qwen in 4.3 GB of RAM on a Mac
 * and a 35B on an iPhone", how-it-works list).  The pages give no formula;
 * this is the published gated delta rule (Yang, Kautz and Hatamizadeh,
 * "Gated Delta Networks: Improving Mamba2 with Delta Rule", ICLR 2025), one
 * decode token per sequence, per value head h with key head
 * hk = h / (v_heads / k_heads):
 *
 *   k^ = k[hk] / sqrt(|k[hk]|^2 + 1e-6)
 *   q^ = q_scale * q[hk] / sqrt(|q[hk]|^2 + 1e-6)
 *   alpha = exp(g[h]),   b = beta[h]
 *   S' = alpha S + b (v[h] - alpha S k^) k^T          (S: [d_v][d_k])
 *   o[h] = S' q^
 *
 * Buffers (device, caller-owned):
 *   q, k:   [B][k_heads][d_k]  act_dtype, 8-byte aligned
 *   v:      [B][v_heads][d_v]  act_dtype, 2-byte aligned
 *   g, beta:[B][v_heads]       fp32 (g <= 0 is the log of the decay)
 *   state:  [B][v_heads][d_v][d_k] fp32, 16-byte aligned, updated in place
 *   o:      [B][v_heads][d_v]  fp32
 * Products and sums are fp32 in a fixed order (bitwise repeatable); the
 * state stays fp32.  Only the given stream is used.
 */
#ifndef MOE_AMD_MOE_GDN_H
#define MOE_AMD_MOE_GDN_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Shape of one Gated DeltaNet layer step.
 *   batch:      B in [0, 65535] (0 is a no-op)
 *   k_heads:    >= 1
 *   v_heads:    a multiple of k_heads, <= 1024
 *   head_k_dim: 128
 *   head_v_dim: a multiple of 16, 16..256
 *   act_dtype:  MOE_F16 or MOE_BF16 (q, k, v) */
typedef struct {
  int32_t batch, k_heads, v_heads, head_k_dim, head_v_dim, act_dtype;
} moe_gdn_desc;

/* One token of the recurrence for every sequence and value head.  MOE_ESHAPE
 * for unsupported sizes, MOE_EINVAL for NULL or misaligned pointers or a bad
 * act_dtype; nothing is enqueued then. */
moe_status moe_gdn_step(const moe_gdn_desc* desc, const void* q, const void* k, const void* v, const float* g,
                        const float* beta, float q_scale, float* state, float* o, moe_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_AMD_MOE_GDN_H */
