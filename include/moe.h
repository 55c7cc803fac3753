/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts layer forward library
 * (libmoe_mi355x.so).
 *
 * The layer is the MoE block of the Nemotron 3 hybrid Mamba-Transformer stack, which takes the
 * place of the FFN: a learned router sends every token to k of E routable experts (6 of 128 in
 * Nano) ["NVIDIA AI发布了Nemotron 3：一款混合Mamba Transformer MoE堆栈", section
 * "混合Mamba Transformer MoE架构"], expert selection is balanced aux-loss-free in the DeepSeek
 * style ["Nemotron 3 Nano：開放高效的 MoE 混合 Mamba-Transformer 智能體推理模型", section 2.2],
 * and the selected experts' outputs are combined with the router's weights ["Nemotron 3 Nano:
 * Open, Efficient Mixture-of-Experts Hybrid Mamba-Transformer Model for Agentic Reasoning",
 * section "技术框架"]. LatentMoE projects tokens from H to a latent width l, runs
 * E' = E*H/l experts with k' = k*H/l there and projects back, while router and shared expert stay
 * in H ["NVIDIA Nemotron 3: Efficient and Open Intelligence", section 2.2 and Figure 3b].
 *
 * What one call computes, per token t (x_t is row t of x):
 *   logits  z = x_t W_r^T                                   (fp32 accumulation)
 *   scores  s = sigmoid(z)                                  (fp32, evaluated in double, rounded)
 *   keys    s + b  -> idx = k largest keys, descending; equal keys: lower expert index first
 *   gates   g_j = s[idx_j] / sum_j s[idx_j]                 (unbiased scores, sum 1)
 *   u       = x_t, or x_t W_in^T rounded to bf16 (LatentMoE)
 *   expert  f_e(u) = relu(u W_up[e]^T)^2 W_down[e]^T        (squared-ReLU, no gate, no bias)
 *   routed  r = sum_j g_j f_{idx_j}(u)                      (fixed j order: deterministic)
 *   y_t     = r, or r W_out^T (LatentMoE);  y_t += relu(x_t Ws_up^T)^2 Ws_down^T if I_shared > 0
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers to row-major, contiguous arrays, 16-byte aligned, owned
 *     by the caller. The library never allocates, frees or synchronises on the call path; scratch
 *     comes from the caller's workspace (size from moe_workspace_size).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null stream).
 *   - Return value: MOE_OK (0) or a negative moe_status; nothing is launched on an error found
 *     before launch. MOE_ERR_HIP reports a failed launch (hipGetLastError after enqueueing).
 *   - State and thread safety: the library keeps, per device and for the life of the process,
 *     one side stream and three events, created on the first call that needs them (the decode
 *     path of a layer with a shared expert and 8- or 4-bit experts forks the shared expert onto
 *     that stream and joins it back before the combine). Calls that use it hold a per-device
 *     lock while they enqueue, so concurrent host threads may call on different streams; their
 *     side-stream work then runs one call after another in lock order. Concurrent calls need
 *     different workspaces and outputs. The launch trace (moe_trace_*) is process-wide and not
 *     for concurrent calls.
 *   - Dimension rules: H, I, I_shared and latent are multiples of 16; 1 <= k <= E <= 1024,
 *     k <= 64; T >= 0 (T == 0 is a no-op that returns MOE_OK). MOE_MXFP4 / MOE_MXFP8 experts
 *     also need D (H, or latent) and I to be multiples of 32 (else MOE_ERR_INVALID_ARG).
 *   - Size rule (bf16 activations): the matrix-core GEMMs use 32-bit operand offsets, so each
 *     of x [T,H], h [T*k,I] (one byte per element for 8- and 4-bit experts, else two), the
 *     shared expert's [T,I_shared], the latent rows [T,latent] and each weight matrix (W_r, one
 *     expert's W_up or W_down, Ws_up, Ws_down, W_in, W_out) must span less than 2 GiB; the
 *     backward pass also needs [T*k, D] in bf16 under 2 GiB. Larger shapes return
 *     MOE_ERR_INVALID_ARG (split T over several calls).
 *   - Expert weights of 8 or 4 bits (MOE_FP8_E4M3, MOE_MXFP4, MOE_MXFP8): the expert input rows
 *     and the rows of h = relu(u W_up^T)^2 (rounded to bf16) are quantised per row to e4m3 with
 *     scale amax / 448 before they meet the weights, as in "Nemotron 3 Nano：開放高效的 MoE 混合
 *     Mamba-Transformer 智能體推理模型", section 4 (FP8 expert weights). MOE_MXFP4 / MOE_MXFP8
 *     run on the decode (stream) path only, whatever T is; MOE_PATH_GROUPED is unsupported for
 *     them.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Expert-weight formats beyond the activation type (expert weights only, with MOE_BF16
 * activations). MOE_MXFP4 / MOE_MXFP8 are the OCP Microscaling (MX v1.0) formats: blocks of 32
 * consecutive elements along K (the input width of each projection) share one E8M0 scale
 * 2^(code - 127); the elements are E2M1 (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives;
 * two per byte, element 2i in the low nibble of byte i) or E4M3. They are the gfx950-native
 * counterpart of the micro-block scaled FP4 of "NVIDIA Nemotron 3: Efficient and Open
 * Intelligence", section 2.4. Scale code 255 (NaN) is not supported: a block carrying it makes
 * its outputs undefined. */
typedef enum {
  MOE_F32 = 0,      /* IEEE binary32 */
  MOE_BF16 = 1,     /* bfloat16 */
  MOE_FP8_E4M3 = 2, /* OCP 8-bit E4M3 (fn: max 448, no inf) with fp32 per-output-channel scales */
  MOE_MXFP4 = 3,    /* OCP MXFP4: E2M1 elements, E8M0 scale per 32 along K */
  MOE_MXFP8 = 4     /* OCP MXFP8: E4M3 elements, E8M0 scale per 32 along K */
} moe_dtype_t;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,  /* null required pointer, misaligned pointer, bad dimension */
  MOE_ERR_UNSUPPORTED = -2,  /* dtype / shape / path combination not provided */
  MOE_ERR_WORKSPACE = -3,    /* workspace missing or smaller than moe_workspace_size */
  MOE_ERR_HIP = -4           /* a HIP launch failed */
} moe_status;

/* desc.flags */
#define MOE_PATH_AUTO 0u         /* stream path when the mean expert load T*k/E is <= 8, or for
                                    MXFP4 / MXFP8 experts */
#define MOE_PATH_GROUPED 1u      /* grouped MFMA GEMMs with a device-built tile list (prefill) */
#define MOE_PATH_STREAM 2u       /* read each touched expert's weights once (decode): bf16,
                                    e4m3, MXFP4 and MXFP8 experts */
#define MOE_PATH_MASK 3u
#define MOE_ROUTING_GIVEN 4u     /* routing->idx and routing->gates are INPUTS: skip the router */
#define MOE_SAVED_IN_WORKSPACE 8u /* moe_layer_backward only: the workspace holds what
                                    moe_layer_forward_train saved; skip the recompute */
#define MOE_WGRAD_BF16 16u       /* moe_layer_backward: dW_up, dW_down, dWs_up and dWs_down are
                                    written in bf16 (moe_layer_forward_train ignores it; the
                                    inference calls reject it with MOE_ERR_INVALID_ARG) */

typedef struct {
  int32_t T;           /* tokens */
  int32_t H;           /* hidden width */
  int32_t E;           /* routed experts (E' for LatentMoE) */
  int32_t k;           /* experts per token (k' for LatentMoE) */
  int32_t I;           /* expert inner width */
  int32_t I_shared;    /* shared-expert inner width; 0 = no shared expert */
  int32_t latent;      /* 0 = plain MoE; else the latent width l (latent_moe_forward only) */
  moe_dtype_t act_dtype;    /* x, y, W_r, shared expert, W_in, W_out: MOE_F32 or MOE_BF16 */
  moe_dtype_t expert_dtype; /* W_up, W_down: act_dtype, or MOE_FP8_E4M3 with act MOE_BF16 */
  uint32_t flags;
} moe_desc_t;

/* D below is the width the routed experts read and write: H, or latent for LatentMoE. */
typedef struct {
  const void *x;        /* [T, H]  act_dtype */
  const void *W_r;      /* [E, H]  act_dtype (router / gating network, always in H) */
  const float *b;       /* [E]     fp32 selection bias (enters the keys, never the gates) */
  const void *W_up;     /* [E, I, D] expert_dtype (MOE_MXFP4: [E, I, D / 2] bytes) */
  const void *W_down;   /* [E, D, I] expert_dtype (MOE_MXFP4: [E, D, I / 2] bytes) */
  const void *s_up;     /* MOE_FP8_E4M3: [E, I] fp32 per-output-channel scales;
                           MOE_MXFP4 / MOE_MXFP8: [E, I, D / 32] uint8 E8M0 block scales;
                           otherwise unused */
  const void *s_down;   /* MOE_FP8_E4M3: [E, D] fp32; MOE_MXFP4 / MOE_MXFP8: [E, D, I / 32] uint8 */
  const void *Ws_up;    /* [I_shared, H] act_dtype, or NULL when I_shared == 0 */
  const void *Ws_down;  /* [H, I_shared] act_dtype, or NULL when I_shared == 0 */
  const void *W_in;     /* [latent, H] act_dtype (LatentMoE only) */
  const void *W_out;    /* [H, latent] act_dtype (LatentMoE only) */
} moe_weights_t;

/* Optional routing record. Any non-NULL member is written (or, for idx and gates under
 * MOE_ROUTING_GIVEN, read) by the layer call. */
typedef struct {
  int32_t *idx;      /* [T, k]  selected experts, descending key order */
  float *gates;      /* [T, k]  gate weights */
  int32_t *counts;   /* [E]     pairs per expert */
  int32_t *offsets;  /* [E + 1] exclusive prefix sum of counts, offsets[E] = T*k */
  int32_t *perm;     /* [T*k]   token of each pair, grouped by expert, tokens ascending */
  int32_t *pos;      /* [T, k]  row of pair (t, j) in that grouped order (inverse of perm) */
  float *logits;     /* [T, E]  router logits */
} moe_routing_t;

/* Bytes of workspace moe_layer_forward / latent_moe_forward need for this descriptor (the path
 * is resolved from desc->flags exactly as the forward call resolves it). */
int32_t moe_workspace_size(const moe_desc_t *desc, size_t *bytes);

/* Plain MoE layer forward (desc->latent must be 0). y: [T, H] act_dtype.
 * routing may be NULL unless MOE_ROUTING_GIVEN is set. */
int32_t moe_layer_forward(const moe_desc_t *desc, const moe_weights_t *w, void *y, void *ws,
                          size_t ws_bytes, moe_routing_t *routing, void *stream);

/* LatentMoE layer forward (desc->latent = l > 0, W_in and W_out required): experts run in the
 * latent width, their gated sum is projected back with W_out, and the shared expert (if any) is
 * added in H. y: [T, H] act_dtype. */
int32_t latent_moe_forward(const moe_desc_t *desc, const moe_weights_t *w, void *y, void *ws,
                           size_t ws_bytes, moe_routing_t *routing, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): moe_layer_forward, or latent_moe_forward when
 * desc->latent > 0, with no workspace argument. Its scratch is a library-owned device array of
 * MOE_STATIC_WORKSPACE_BYTES (64 MiB) per GPU, held until the process ends: enough for decode
 * calls (a Nano layer at T = 64 needs about 7 MB). A descriptor whose moe_workspace_size exceeds
 * it returns MOE_ERR_WORKSPACE before anything is launched. The call allocates nothing; its first
 * call on each device does that device's set-up (looks up the array's address, creates the side
 * stream of the narrow decode path), so make that first call outside graph capture. Every call
 * on one GPU shares that GPU's array: calls that overlap on one GPU (other streams, other host
 * threads) race and must be serialised by the caller. Results are those of moe_layer_forward /
 * latent_moe_forward bit for bit; arguments and other errors as there. */
#define MOE_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
int32_t moe_layer_forward_static(const moe_desc_t *desc, const moe_weights_t *w, void *y,
                                 moe_routing_t *routing, void *stream);

/* Router alone (steps logits -> scores -> top-k -> gates). If `logits` is non-NULL it is used as
 * the fp32 router logits [T, E] and x / W_r are ignored; otherwise logits are computed from
 * x [T, H] and W_r [E, H] (dtype `dt`) into `logits_out` [T, E], which is then required.
 * Writes idx [T, k] and gates [T, k]. */
int32_t moe_route(const float *logits, const void *x, const void *W_r, const float *b, int32_t T,
                  int32_t H, int32_t E, int32_t k, moe_dtype_t dt, int32_t *idx, float *gates,
                  float *logits_out, void *stream);

/* Workspace bytes moe_dispatch needs. */
int32_t moe_dispatch_workspace_size(int32_t T, int32_t E, int32_t k, size_t *bytes);

/* Dispatch alone: from idx [T, k] (values in [0, E), distinct per token) build counts [E],
 * offsets [E + 1], perm [T*k] and pos [T, k] as described in moe_routing_t. The order is stable
 * and deterministic (no atomics decide it). */
int32_t moe_dispatch(const int32_t *idx, int32_t T, int32_t E, int32_t k, int32_t *counts,
                     int32_t *offsets, int32_t *perm, int32_t *pos, void *ws, size_t ws_bytes,
                     void *stream);

/* Aux-loss-free load balancing step ("Nemotron 3 Nano：開放高效的 MoE 混合 Mamba-Transformer
 * 智能體推理模型", section 2.2, training hyper-parameters: DeepSeek's auxiliary-loss-free
 * balancing). The routing bias of every expert moves by a fixed step toward its target load:
 *   b[e] <- fp32(b[e] + gamma * sign(target[e] - counts[e]))        (sign(0) = 0)
 * counts [E] int32 (device): pairs routed to each expert, e.g. moe_routing_t.counts of a forward
 * call. target [E] fp32 (device) or NULL for the mean load sum(counts) / E (compared exactly in
 * integers). b [E] fp32 (device) is updated in place. Only the bias changes: gates never use it.
 * Errors: MOE_ERR_INVALID_ARG for E < 1 or a NULL counts / b. Asynchronous on `stream`. */
int32_t moe_bias_update(const int32_t *counts, const float *target, int32_t E, float gamma,
                        float *b, void *stream);

/* ---- Backward pass (training) of the MoE layer and of LatentMoE.
 * Gradients of a scalar loss given dy = dLoss/dy [T, H] (device, act dtype), for the forward that
 * moe_layer_forward / latent_moe_forward compute ("NVIDIA Nemotron 3: Efficient and Open
 * Intelligence", section 2.2; "Nemotron 3 Nano: Open, Efficient Mixture-of-Experts Hybrid
 * Mamba-Transformer Model for Agentic Reasoning", section "技术框架"). The top-k selection is
 * piecewise constant, so it is held at the forward's choice and the gradient reaches the router
 * through the gate weights only:
 *   g_j = s_j / sum_m s_m with s = sigmoid(x W_r^T) over the selected experts;
 *   dz_{e_j} = (dg_j - sum_m g_m dg_m) / sum_m s_m * s_j (1 - s_j), dg_j = <dY, Y_j>, where Y_j is
 *   expert e_j's output and dY the gradient reaching the experts' gated sum (dy, or for LatentMoE
 *   dy W_out, rounded to bf16). The routing bias b only steers the selection: no gradient.
 * The squared ReLU's derivative is 2 relu(a). Every gradient is written (not accumulated) in
 * fp32, row-major, with D = H (or latent); under MOE_WGRAD_BF16 the expert weight gradients
 * dW_up, dW_down, dWs_up and dWs_down are written in bf16 instead, each element the fp32 result
 * rounded to nearest even (the same sums, half the bytes stored):
 *   dx [T, H], dW_r [E, H], dW_up [E, I, D], dW_down [E, D, I], dWs_up [I_s, H], dWs_down [H, I_s]
 *   (when I_shared > 0), dW_in [latent, H] and dW_out [H, latent] (LatentMoE); all required when
 *   they apply.
 * Supported: act_dtype = expert_dtype = MOE_BF16, routing computed inside (flags:
 * path bits ignored, MOE_ROUTING_GIVEN not accepted) -- else MOE_ERR_UNSUPPORTED. Without
 * MOE_SAVED_IN_WORKSPACE the call first recomputes the forward's routing and expert activations
 * from x; with it, it reads them from the workspace, where moe_layer_forward_train (same
 * descriptor apart from that flag, same weights and x) left them. Either way the weights are
 * read in place as stored (the products that need them K-major stage them through transposing
 * LDS reads; nothing is copied), and the call never overwrites the saved part, so several
 * backward calls (e.g. for several dy) may follow one moe_layer_forward_train. Pointers: 16-byte
 * aligned device memory owned by the caller. Workspace: moe_backward_workspace_size bytes.
 * Asynchronous on `stream`; nothing is allocated or synchronised. Results are deterministic (no
 * atomics) and identical with or without the saved activations. */
typedef struct {
  float *dx;
  float *dW_r;
  void *dW_up;      /* fp32, or bf16 under MOE_WGRAD_BF16; so are the next three */
  void *dW_down;
  void *dWs_up;
  void *dWs_down;
  float *dW_in;     /* LatentMoE only: [latent, H] */
  float *dW_out;    /* LatentMoE only: [H, latent] */
} moe_grads_t;

int32_t moe_backward_workspace_size(const moe_desc_t *desc, size_t *bytes);
/* Training forward: y [T, H] exactly as moe_layer_forward (latent_moe_forward when latent > 0)
 * computes it on MOE_PATH_GROUPED (bit for bit), keeping the routing and expert activations
 * moe_layer_backward reads in `ws` (moe_backward_workspace_size bytes). Same support, arguments
 * and errors as moe_layer_backward (MOE_SAVED_IN_WORKSPACE must not be set). */
int32_t moe_layer_forward_train(const moe_desc_t *desc, const moe_weights_t *weights, void *y,
                                void *ws, size_t ws_bytes, void *stream);
int32_t moe_layer_backward(const moe_desc_t *desc, const moe_weights_t *weights, const void *dy,
                           moe_grads_t *grads, void *ws, size_t ws_bytes, void *stream);

/* Static text for a status code. */
const char *moe_status_str(int32_t code);

/* ---- Diagnostics: per-launch timing with HIP events (process-wide; not for concurrent calls).
 * moe_trace_enable(capacity, filter) creates 2*capacity events up front (its only allocation;
 * capacity 0 disables tracing and destroys them). While enabled, every kernel launch of a layer
 * call whose trace name starts with `filter` (NULL or "" = all) is bracketed by two events
 * recorded on the call's stream, until `capacity` launches are recorded. Trace names are
 * "<kernel>:<role>", e.g. "stream:up", "gemm_bf16_sqrelu:routed_up", "dispatch:all".
 * The events are timing-only (created with hipEventDisableSystemFence): recording one adds no
 * cache write-back or invalidate to the stream, so tracing changes the traced work's timing as
 * little as possible; they order nothing, and a reader must synchronise the stream (or device)
 * before moe_trace_read(i, name, ms) returns record i. */
int32_t moe_trace_enable(int32_t capacity, const char *filter);
int32_t moe_trace_count(void);
int32_t moe_trace_read(int32_t i, const char **name, float *ms);
void moe_trace_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
