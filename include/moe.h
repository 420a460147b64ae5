/*
 * moe.h - C ABI of the MI355X (gfx950) int4 routed-expert MoE library.
 *
 * The operation is the sparse Mixture-of-Experts block of a Qwen3-Next-style
 * hybrid model (the model family named in the intro of the page "Show HN:
 * Run an 80B Qwen in 4.3 GB of RAM on a Mac and a 35B on an iPhone"): every
 * token is routed to K of E experts (10 of 512 for the 80B, 8 of 256 for the
 * 35B; same page, how-it-works list), whose weights are 4-bit affine
 * group-quantised (that page's what-was-built list), and a shared expert that
 * stays resident (how-it-works list) is added on top.  For x of T tokens:
 *
 *   z[t,e]   = sum_h x[t,h] * Wr[e,h] + beta[e]                  (e < E)
 *   z_s[t]   = sum_h x[t,h] * Wr[E,h]                            (shared gate)
 *   S_t      = K largest z[t,.], ordered by (z desc, expert index asc)
 *   w[t,k]   = exp(z[t,S_tk] - z[t,S_t0]) / sum_j exp(z[t,S_tj] - z[t,S_t0])
 *   gamma[t] = 1 / (1 + exp(-z_s[t]))
 *   FFN_e(x) = Wd_e (silu(Wg_e x) * (Wu_e x)),  silu(a) = a / (1 + exp(-a))
 *   y[t]     = sum_k w[t,k] FFN_{S_tk}(x[t]) + gamma[t] FFN_shared(x[t])
 *
 * with W[r,c] = s[r, c/G] * q[r,c] + b[r, c/G], q in 0..15 (or 0..255 for
 * int8 experts, the pages' other affine width: same what-was-built list),
 * fp16 s and b, groups of G columns along each matrix's input dimension.
 *
 * Conventions (all functions):
 *  - Every buffer is caller-owned.  Pointers named "device" are device
 *    addresses (HBM, e.g. torch tensors' data_ptr()); "host" pointers are
 *    ordinary host memory.  The library never allocates device memory; the
 *    slot pool allocates host metadata and HIP events only.
 *  - Device work is only enqueued on the given HIP stream; functions return
 *    before it runs.  Kernel faults surface at the caller's synchronisation.
 *  - Errors: a negative moe_status and a thread-local message
 *    (moe_last_error).  Nothing throws across the ABI.  A call that fails
 *    validation enqueues nothing.  n_tokens == 0 is a valid no-op.
 *  - Floating-point results are deterministic: every reduction has a fixed
 *    order, so the same inputs give bitwise identical outputs.
 */
#ifndef MOE_AMD_MOE_H
#define MOE_AMD_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* moe_stream; /* a hipStream_t; NULL = default stream */

typedef int32_t moe_status;
#define MOE_OK          0
#define MOE_EINVAL     -1 /* NULL required pointer, bad enum, misaligned pointer */
#define MOE_ESHAPE     -2 /* unsupported sizes (see moe_layer_desc) */
#define MOE_EWORKSPACE -3 /* ws_bytes < moe_workspace_bytes() */
#define MOE_EHIP       -4 /* a HIP call failed; message carries hipGetErrorString */
#define MOE_EPOOLFULL  -5 /* more misses than free or evictable slots */
#define MOE_EBUSY      -6 /* evicting a pinned slot */
#define MOE_ENOMEM     -7 /* host allocation failed */

enum { MOE_F16 = 1, MOE_BF16 = 2 };

/* Kernel family for the expert FFN. AUTO picks the batched grouped-GEMM
 * (matrix-core) family when the batch has more than MOE_GEMV_MAX_ROWS
 * routed rows (T*K) and the shape fits it (hidden <= 2048, inter and
 * shared_inter <= 512), the per-row GEMV family otherwise.  Asking for
 * GROUPED with a shape beyond those limits is MOE_ESHAPE.
 *
 * Range of the grouped family: its matrix-core operands are fp16, so every
 * activation x and every SwiGLU output h must round to a finite fp16 value
 * (|v| < 65520; bf16 activations are exact in fp16 inside that range).  A
 * value outside it (or a non-finite input) makes that call's results
 * invalid; the call then sets MOE_FLAG_F16_RANGE in its status word (see
 * moe_workspace_status).  The GEMV family has no such limit (bf16 and fp16
 * activations enter its products exactly; h is fp32). */
enum { MOE_PATH_AUTO = 0, MOE_PATH_GEMV = 1, MOE_PATH_GROUPED = 2 };
#define MOE_GEMV_MAX_ROWS 32

/* Shape of one MoE layer.
 *   hidden H:        multiple of 64, 64..8192
 *   n_experts E:     1..1024
 *   top_k K:         1..min(E, 64)
 *   inter I:         multiple of 64, 64..4096 (routed experts)
 *   shared_inter:    0 (no shared expert) or a multiple of 64, 64..4096
 *   group_size G:    32, 64 or 128, dividing H, I and shared_inter
 *   act_dtype:       MOE_F16 or MOE_BF16 (dtype of x); y is always fp32
 *   path:            MOE_PATH_*
 *   weight_bits:     4 (or 0, the same) for int4 experts, 8 for int8 experts
 *                    (routed and shared alike), on either kernel family. */
typedef struct {
  int32_t hidden, n_experts, top_k, inter, shared_inter, group_size;
  int32_t act_dtype;
  int32_t path;
  int32_t weight_bits;
} moe_layer_desc;

/* Weights of one layer (device addresses, caller-owned, read-only).
 *   router_w:      [E+1][H] fp16 bits, row-major; row E is the shared-gate
 *                  vector (no bias on it).  16-byte aligned.
 *   router_bias:   [E] fp32, or NULL for none.
 *   experts:       base of the routed expert blobs; expert e's blob starts at
 *                  experts + (expert_offset ? expert_offset[e] : e*expert_stride).
 *                  Blob starts must be 256-byte aligned.
 *   expert_stride: bytes between consecutive blobs when expert_offset is NULL
 *                  (>= moe_blob_bytes_q(H, I, G, weight_bits), multiple of 256).
 *   expert_offset: [E] uint64 byte offsets (device) or NULL.  Only entries of
 *                  selected experts are read (the slot pool keeps them valid).
 *   shared:        blob of the shared expert (inter = shared_inter), or NULL
 *                  when shared_inter == 0. */
typedef struct {
  const uint16_t* router_w;
  const float* router_bias;
  const uint8_t* experts;
  uint64_t expert_stride;
  const uint64_t* expert_offset;
  const uint8_t* shared;
} moe_layer_weights;

/* Fixed-stride expert blob (the pages pack every routed expert at a fixed
 * stride so one fetch is one read: Show HN page, how-it-works list).  The
 * byte layout is this library's own, tiled for 64-lane wavefronts:
 *
 *   section  offset               size       contents
 *   GU_Q     0                    I*H        gate/up nibbles
 *   D_Q      I*H                  H*I/2      down nibbles
 *   GU_S     3*I*H/2              8*I*H/G    gate/up fp16 scale, bias
 *   D_S      3*I*H/2 + 8*I*H/G    4*H*I/G    down fp16 scale, bias
 *
 * Matrices: gate, up [I][H] and down [H][I] (rows = outputs, columns =
 * inputs).  A pair-tile joins two 16-row tiles: GU pair-tile p (p < I/16) has
 * tile A = gate rows 16p..16p+15 and tile B = up rows 16p..16p+15; D
 * pair-tile p (p < H/32) has tile A = down rows 32p..32p+15 and tile B = down
 * rows 32p+16..32p+31.  The input dimension is cut into chunks of 64
 * columns; chunk c of pair-tile p is the 1024-byte block number
 * p*(in_dim/64) + c of its section.  In a block, lane l (n = l%16,
 * kb = l/16) owns bytes 16l..16l+15 = four little-endian 32-bit words:
 *   word 0: tile A row n, columns 64c +      8kb + j,  j = 0..7
 *   word 1: tile A row n, columns 64c + 32 + 8kb + j
 *   word 2: tile B row n, columns 64c +      8kb + j
 *   word 3: tile B row n, columns 64c + 32 + 8kb + j
 * and value j of a word occupies bits [4p, 4p+4), p = (j>>1) + 4*(j&1).
 * Scale sections: for pair-tile p, group g (< in_dim/G), n < 16, the eight
 * bytes at ((p*(in_dim/G) + g)*16 + n)*8 hold fp16 [s_A, b_A, s_B, b_B] of
 * row n of tiles A and B.
 *
 * int8 experts double the value sections (GU_Q 2*I*H bytes at 0, D_Q I*H
 * bytes at 2*I*H) and move the scale sections to 3*I*H and 3*I*H + 8*I*H/G
 * (same contents).  A chunk is then a 2048-byte block of two 1024-byte
 * planes, tile A first; in each plane lane l owns the 16 bytes at 16l: the 8
 * values of columns 64c + 8kb + j, then the 8 of columns 64c + 32 + 8kb + j,
 * one byte per value in order j = 0..7.
 *
 * moe_blob_bytes: size of an int4 blob; moe_blob_bytes_q: of a blob of
 * weight_bits 4 or 8.  Both return 0 for unsupported sizes. */
uint64_t moe_blob_bytes(int32_t hidden, int32_t inter, int32_t group_size);
uint64_t moe_blob_bytes_q(int32_t hidden, int32_t inter, int32_t group_size, int32_t weight_bits);

/* Host-side packer: raw tensors -> one blob (host buffer of
 * moe_blob_bytes_q() bytes).  q arrays hold one value per byte (0..15 for
 * weight_bits 4, 0..255 for 8), row-major: gate_q, up_q [I][H], down_q
 * [H][I]; scale and bias arrays are fp16 bits, row-major [rows][in_dim/G].
 * Returns MOE_ESHAPE for bad sizes or widths, MOE_EINVAL for NULL pointers
 * or int4 q values above 15.  moe_pack_expert is the int4 packer. */
moe_status moe_pack_expert_q(int32_t hidden, int32_t inter, int32_t group_size, int32_t weight_bits,
                             const uint8_t* gate_q, const uint16_t* gate_s, const uint16_t* gate_b,
                             const uint8_t* up_q, const uint16_t* up_s, const uint16_t* up_b,
                             const uint8_t* down_q, const uint16_t* down_s, const uint16_t* down_b,
                             uint8_t* blob_out);
moe_status moe_pack_expert(int32_t hidden, int32_t inter, int32_t group_size,
                           const uint8_t* gate_q, const uint16_t* gate_s, const uint16_t* gate_b,
                           const uint8_t* up_q, const uint16_t* up_s, const uint16_t* up_b,
                           const uint8_t* down_q, const uint16_t* down_s, const uint16_t* down_b,
                           uint8_t* blob_out);

/* Device workspace needed by moe_route / moe_expert_ffn / moe_layer_forward
 * and the stack calls for n_tokens tokens (256-byte aligned base). */
moe_status moe_workspace_bytes(const moe_layer_desc* desc, int32_t n_tokens, size_t* bytes);

/* Status word of a call.  moe_expert_ffn, moe_layer_forward,
 * moe_stack_forward (and its graphs), moe_pool_decode_step and
 * moe_pool_decode_step_dev (and its graphs) clear a uint32 status word
 * inside the workspace at their start (in their first FFN kernel) and their
 * kernels set flags in it:
 *   MOE_FLAG_F16_RANGE    a grouped-family operand (an activation or a
 *                         SwiGLU output) fell outside the fp16 range: the
 *                         outputs of the call are not valid (run such inputs
 *                         with MOE_PATH_GEMV).
 *   MOE_FLAG_STREAM_WAIT  a streamed decode's gate/up product gave up
 *                         waiting (about 0.1 s) for its expert's copy: the
 *                         outputs of the call are not valid.
 * moe_workspace_status returns the byte offset of the word in a workspace
 * laid out for (desc, n_tokens); read it (device memory) after the call's
 * stream has been synchronised.  Calls that overlap on one workspace race on
 * it, as they do on the rest of the workspace. */
#define MOE_FLAG_F16_RANGE 1u
#define MOE_FLAG_STREAM_WAIT 2u
moe_status moe_workspace_status(const moe_layer_desc* desc, int32_t n_tokens, size_t* offset);

/* Router GEMV (shared-gate row fused), top-K with lower-index tie-break,
 * renormalised weights and sigmoid shared gate (the routing step of the
 * how-it-works list).  x: device [T][H] act_dtype (16-byte aligned rows).
 * Outputs (device): topk_idx [T][K] int32 in rank order, topk_w [T][K]
 * fp32, shared_gate [T] fp32 (may be NULL when shared_inter == 0),
 * logits_or_null [T][E+1] fp32 (column E = shared-gate logit).  Logits are
 * fp32 sums of exact products in a fixed order (for batches of 16+ tokens,
 * up to 4 hidden-dimension slices added in slice order, then the bias);
 * selection and weights use those fp32 values. */
moe_status moe_route(const moe_layer_desc* desc, const moe_layer_weights* w, const void* x,
                     int32_t n_tokens, int32_t* topk_idx, float* topk_w, float* shared_gate,
                     float* logits_or_null, void* ws, size_t ws_bytes, moe_stream stream);

/* Token-to-expert bucketing (batched path; exposed for tests): stable
 * counting sort of the T*K routed rows by expert.  Outputs (device):
 * expert_off [E+1] int32 exclusive prefix sums of per-expert counts;
 * perm [T*K] int32, perm[r] = t*K + k of the r-th row in (expert, t, k)
 * order; inv_or_null [T*K] int32 the inverse permutation.  A row whose
 * expert index lies outside [0, E) is dropped: it is not counted, perm holds
 * only the expert_off[E] placed rows, and its inv entry is -1. */
moe_status moe_permute(const moe_layer_desc* desc, const int32_t* topk_idx, int32_t n_tokens,
                       int32_t* expert_off, int32_t* perm, int32_t* inv_or_null,
                       void* ws, size_t ws_bytes, moe_stream stream);

/* Expert FFNs and combine for given routing: y [T][H] fp32 (device) =
 * sum_k topk_w[t,k] FFN_{topk_idx[t,k]}(x_t) + shared_gate[t] FFN_shared(x_t),
 * summed in rank order, shared term last.  shared_gate may be NULL only when
 * shared_inter == 0.  An index outside [0, E) selects no expert (that term is
 * zero). */
moe_status moe_expert_ffn(const moe_layer_desc* desc, const moe_layer_weights* w, const void* x,
                          int32_t n_tokens, const int32_t* topk_idx, const float* topk_w,
                          const float* shared_gate, float* y, void* ws, size_t ws_bytes,
                          moe_stream stream);

/* The whole block, bit for bit the results of moe_route then
 * moe_expert_ffn.  On the GEMV family with E <= 512 the top-K selection runs
 * inside the gate/up kernel instead of a launch of its own.  Optional device
 * outputs topk_idx_or_null [T][K], topk_w_or_null [T][K],
 * shared_gate_or_null [T]. */
moe_status moe_layer_forward(const moe_layer_desc* desc, const moe_layer_weights* w, const void* x,
                             int32_t n_tokens, float* y, int32_t* topk_idx_or_null,
                             float* topk_w_or_null, float* shared_gate_or_null,
                             void* ws, size_t ws_bytes, moe_stream stream);

/* moe_layer_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same call, bit for bit the same results, with its
 * workspace in a static device array of MOE_STATIC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends.  It calls no
 * allocating routine.  A batch whose workspace (moe_workspace_bytes) exceeds
 * the array returns MOE_EWORKSPACE.  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (other streams or threads)
 * race on it; calls ordered on one stream do not.  The status word of the
 * call (moe_workspace_status) sits in the array and is not readable here. */
#define MOE_STATIC_SCRATCH_BYTES (32u << 20)
moe_status moe_layer_forward_static(const moe_layer_desc* desc, const moe_layer_weights* w, const void* x,
                                    int32_t n_tokens, float* y, int32_t* topk_idx_or_null,
                                    float* topk_w_or_null, float* shared_gate_or_null, moe_stream stream);

/* Chaining step between MoE layers of a stack (a pre-norm residual stand-in;
 * the pages do not describe the layers between MoE blocks):
 *   r[t] += y[t];  x_next[t] = round_rne(r[t] / sqrt(mean(r[t]^2) + 1e-6))
 * r, y: device [T][H] fp32; x_next: device [T][H] act_dtype. */
moe_status moe_stack_epilogue(const moe_layer_desc* desc, int32_t n_tokens, const float* y,
                              float* r, void* x_next, moe_stream stream);

/* A stack of n_layers MoE layers with distinct weights (host array of
 * per-layer weight descriptors).  Layer 0 reads x0; each later layer reads
 * the previous epilogue's x_next (held in x_buf, device [T][H] act_dtype).
 * r (device [T][H] fp32) must hold the initial residual (x0 as fp32) on
 * entry and holds the final residual on exit.  Optional per-layer captures
 * (device, NULL to skip): x_all [L][T][H] act_dtype (each layer's input),
 * y_all [L][T][H] fp32, idx_all [L][T][K], w_all [L][T][K], gamma_all [L][T]. */
moe_status moe_stack_forward(const moe_layer_desc* desc, const moe_layer_weights* layers,
                             int32_t n_layers, const void* x0, int32_t n_tokens, float* r,
                             void* x_buf, void* x_all, float* y_all, int32_t* idx_all,
                             float* w_all, float* gamma_all, void* ws, size_t ws_bytes,
                             moe_stream stream);

/* A captured HIP graph of moe_stack_forward (same arguments, fixed at
 * capture): one launch replays the whole stack with no host work per layer.
 * The stream passed to create must not be the NULL stream; the graph is
 * captured on it (nothing runs) and may later be launched on any stream. */
typedef struct moe_graph moe_graph;
moe_status moe_stack_graph_create(const moe_layer_desc* desc, const moe_layer_weights* layers,
                                  int32_t n_layers, const void* x0, int32_t n_tokens, float* r,
                                  void* x_buf, void* x_all, float* y_all, int32_t* idx_all,
                                  float* w_all, float* gamma_all, void* ws, size_t ws_bytes,
                                  moe_stream capture_stream, moe_graph** out);
moe_status moe_graph_launch(moe_graph* g, moe_stream stream);
void moe_graph_destroy(moe_graph* g);

/* Optional timing of one kernel per layer inside moe_stack_forward and
 * graphs captured by moe_stack_graph_create on this thread: when set,
 * begin[l] and end[l] (hipEvent_t handles created by the caller with timing
 * enabled) are recorded on the stream right before and right after layer l's
 * kernel of the chosen kind (MOE_TIME_*).  n_layers = 0 disables it.  The
 * setting is read when the stack is enqueued or captured.  The events stay
 * owned by the caller and are only borrowed: they must remain valid while
 * the setting is in force on this thread (until it is cleared with
 * n_layers = 0), until every stack call enqueued with them has run, and for
 * the whole life of any graph captured with them (each replay records into
 * them). */
enum { MOE_TIME_GATEUP = 0, MOE_TIME_DOWN = 1, MOE_TIME_ROUTER = 2 };
moe_status moe_stack_set_kernel_events(void* const* begin, void* const* end, int32_t n_layers, int32_t kind);

/* Thread-local description of the last error on this thread (valid until
 * the next call on the thread); "" when the last call succeeded. */
const char* moe_last_error(void);

/* Library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_AMD_MOE_H */
