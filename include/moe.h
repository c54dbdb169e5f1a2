/*
 * moe.h — C ABI of the sigmoid-routed mixture-of-experts FFN layer for MI355X (gfx950).
 *
 * One layer of the Kimi K2 / DeepSeek-V3 mixture of experts, as the equations of
 * "Kimi K2 · Transformer blocks" (MoE transformer block, "Mixture of experts") give it:
 *
 *   z = x W_r^T                       router logits            [T, E]
 *   s = sigmoid(z)                    scores
 *   sel(t) = top_k(s + b)             selection on biased scores (bias only here)
 *   G_i = alpha * s_i / sum_{j in sel} s_j   on sel(t), 0 elsewhere (alpha = 2.827 on K2)
 *   E_i = (silu(x W1_i^T) * (x W3_i^T)) W2_i^T   SwiGLU expert
 *   y_routed = sum_i G_i E_i ;  y_shared = same SwiGLU with the shared expert's weights
 *   out = y_routed + y_shared
 *
 * and the routing notes of "nnterp encyclopedia · kimi_k2" ("The mixture of experts":
 * all experts eligible, each gate the selected expert's sigmoid score with the bias left
 * out, renormalised and scaled so the gates of a token sum to alpha).
 *
 * Conventions for every entry point
 *   - All array pointers are DEVICE pointers; `dims` is a host pointer.  bf16 arrays are
 *     passed as uint16_t bit patterns (bfloat16, round-to-nearest-even).
 *   - Matrices are row-major and stored [out, in] (the input dimension contiguous):
 *       x      [T, d]       bf16        w_router [E, d]    fp32     bias [E] fp32
 *       w1, w3 [E, I, d]    bf16        w2       [E, d, I] bf16
 *       ws1, ws3 [Is, d]    bf16        ws2      [d, Is]   bf16     (shared expert)
 *   - Row p of the "grouped" order: the T*k (token, slot) pairs sorted by expert, expert 0
 *     first; inside an expert's segment tokens ascend.  Slot id = t*k + slot.
 *   - The caller owns all memory.  The library allocates nothing and never synchronises
 *     the host; all work is queued on `stream` (a hipStream_t; NULL = the default stream).
 *     Concurrent calls need their own workspace.  (The one exception, moe_forward_noalloc,
 *     works in a device array the library holds instead of a workspace.)
 *   - No result depends on an earlier call.  The routing of up to 512 tokens over more
 *     than 16 experts counts, per block of 16 tokens, the router workgroups that have
 *     finished, in a small counter array the library holds on each GPU (zero at load, and
 *     back to zero at the end of every routing launch).  Each workspace address is given
 *     its own slot of 1024; a workspace keeps its slot while it is among the 1024 most
 *     recently used on that GPU, and, once a call on it has been captured into a graph, until
 *     moe_workspace_release.  So calls that may overlap, having their own workspaces, never
 *     share counters; capturing calls on more than 1024 unreleased workspaces of one GPU
 *     fails with MOE_EHIP.
 *   - Every output is fully overwritten.  tokens == 0 is a valid no-op.
 *   - Errors are status codes, checked on the host BEFORE anything is launched:
 *       MOE_EINVAL       null / misaligned (16 B) pointer, impossible dims
 *       MOE_EUNSUPPORTED dims this library does not handle (d, I not multiples of 64,
 *                        top_k > 8, E > 1024, Is not 0 or I, x or one weight matrix
 *                        of 2 GiB or more, T above 2^23)
 *       MOE_EWORKSPACE   ws_bytes smaller than moe_workspace_bytes()
 *       MOE_EHIP         a kernel launch failed (device faults surface at the caller's
 *                        next synchronisation, as usual for asynchronous work)
 *       MOE_ESCRATCH     moe_forward_noalloc only: dims need more than its fixed scratch
 *   - Deterministic: the same inputs give bit-identical outputs (no float atomics).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Layer shape.  K2: d_model 7168, n_experts 384, top_k 8, d_expert 2048, d_shared 2048,
 * routed_scale 2.827 ("nnterp encyclopedia · kimi_k2", section "Config"). */
typedef struct moe_dims {
  int64_t tokens;      /* T >= 0 (batch x positions flattened: the layer is per token) */
  int32_t d_model;     /* d, multiple of 64 */
  int32_t n_experts;   /* E in [1, 1024] */
  int32_t top_k;       /* k in [1, min(8, E)] */
  int32_t d_expert;    /* I, multiple of 64 */
  int32_t d_shared;    /* Is: 0 (no shared expert) or equal to d_expert */
  float routed_scale;  /* alpha, finite */
} moe_dims;

typedef enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = 1,
  MOE_EUNSUPPORTED = 2,
  MOE_EWORKSPACE = 3,
  MOE_EHIP = 4,
  MOE_ESCRATCH = 5
} moe_status;

/* Human-readable name of a status code (static string). */
const char* moe_status_str(int status);

/* Bytes of device workspace every entry point below accepts for these dims (one size
 * serves them all).  Host only; launches nothing.
 * After moe_forward, moe_forward_block, moe_forward_fp8 or moe_forward_latent returns (and
 * its work has completed), the workspace begins with that call's routing and permutation,
 * each array starting at the next multiple of 256 bytes, in this order:
 *   topk_idx [T, k] int32, topk_w [T, k] fp32, counts [E] int32, offsets [E+1] int32,
 *   perm_rows [T*k] int32, inv_perm [T*k] int32
 * with the meanings of moe_route and moe_permute.  The rest of the workspace is opaque. */
moe_status moe_workspace_bytes(const moe_dims* dims, size_t* bytes);

/* Router ("Kimi K2 · Transformer blocks", MoE equations z, s, E_sel, G_i).
 *   topk_idx [T, k] int32  chosen experts per token, descending biased score, ties to
 *                          the lower expert index
 *   topk_w   [T, k] fp32   gates alpha * s / sum(s over the chosen), same order
 *   logits   [T, E] fp32   z, or NULL (not written)
 *   ws                     workspace (required)
 * z keeps fp32 accuracy: w_router is split exactly into three bf16 parts whose products
 * with the bf16 x are exact; their sums (fp32 accumulation) are added in fp64 and
 * rounded to fp32.  The selection compares fp32 scores fl(sigmoid(z) + b). */
moe_status moe_route(const moe_dims* dims, const uint16_t* x, const float* w_router,
                     const float* bias, int32_t* topk_idx, float* topk_w, float* logits,
                     void* ws, size_t ws_bytes, void* stream);

/* Token permutation ("Kimi K3 · Latent up-projection", moe_infer: count tokens per
 * expert, group the slots by expert, each expert's rows a contiguous segment).
 *   counts   [E]    int32  rows per expert
 *   offsets  [E+1]  int32  exclusive scan of counts (offsets[E] = number of valid slots)
 *   perm_rows[T*k]  int32  perm_rows[p] = slot id (t*k + slot) of grouped row p
 *   inv_perm [T*k]  int32  inv_perm[t*k + slot] = its grouped row
 * Entries of topk_idx outside [0, E), or repeating an earlier slot of the same token,
 * are dropped: not counted, inv_perm = -1, and the tail perm_rows[offsets[E]..T*k) = -1.
 */
moe_status moe_permute(const moe_dims* dims, const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* perm_rows, int32_t* inv_perm, void* ws,
                       size_t ws_bytes, void* stream);

/* Expert gate/up projections with the SwiGLU product fused in the epilogue
 * ("Kimi K2 · Transformer blocks", g = x W1, u = x W3, a = g sigma(g), h = a (.) u).
 *   h [(T*k + Ts), H] bf16: rows 0..T*k-1 in grouped order (row p reads token
 *     perm_rows[p] / k of x through expert e with offsets[e] <= p < offsets[e+1]), then,
 *     if the shared expert is present (d_shared > 0, ws1/ws3 non-NULL), Ts = T rows of
 *     the shared expert for tokens 0..T-1.  Rows p >= offsets[E] of the routed block are
 *     left untouched.  g, u are fp32 accumulations of bf16 products.
 *   H = I: h rounded to bf16.  H = 2I when top_k <= MOE_HSPLIT_MAX_TOP_K or d_expert <=
 *     MOE_HSPLIT_MAX_D_EXPERT: h in two bf16 parts, columns [0, I) = bf16(h), [I, 2I) =
 *     bf16(h - bf16(h)) (16 significant bits; with so few slots per token, or so few terms
 *     per output of the down projection, a single rounding of h would take most of the
 *     output's error budget).  moe_expert_down reads h in the same form.  The FP8 entry
 *     points always use H = I. */
#define MOE_HSPLIT_MAX_TOP_K 2
#define MOE_HSPLIT_MAX_D_EXPERT 128
moe_status moe_expert_gate_up(const moe_dims* dims, const uint16_t* x, const int32_t* perm_rows,
                              const int32_t* offsets, const uint16_t* w1, const uint16_t* w3,
                              const uint16_t* ws1, const uint16_t* ws3, uint16_t* h, void* ws,
                              size_t ws_bytes, void* stream);

/* Expert down projections ("Kimi K2 · Transformer blocks", E_i = h W2; y_shared = h W2).
 *   h as produced by moe_expert_gate_up ([rows, H]; with H = 2I both parts are multiplied
 *   by W2 and summed in the fp32 accumulation);
 *   y_routed [T*k, d] fp32 grouped order (rows >= offsets[E] untouched);
 *   y_shared [T, d]   fp32 (NULL iff no shared expert).  fp32 accumulation; the expert
 *   outputs stay fp32 so that the layer output is rounded to bf16 only once. */
moe_status moe_expert_down(const moe_dims* dims, const uint16_t* h, const int32_t* offsets,
                           const uint16_t* w2, const uint16_t* ws2, float* y_routed,
                           float* y_shared, void* ws, size_t ws_bytes, void* stream);

/* moe_expert_gate_up followed by moe_expert_down, h kept in the workspace. */
moe_status moe_expert_ffn(const moe_dims* dims, const uint16_t* x, const int32_t* perm_rows,
                          const int32_t* offsets, const uint16_t* w1, const uint16_t* w3,
                          const uint16_t* w2, const uint16_t* ws1, const uint16_t* ws3,
                          const uint16_t* ws2, float* y_routed, float* y_shared,
                          void* ws, size_t ws_bytes, void* stream);

/* Weighted combine plus shared expert ("Kimi K2 · Transformer blocks", y_routed =
 * sum_i G_i E_i and Delta_ffn = y_routed + y_shared; the fp32 weighted sum over the k
 * slots of "Kimi K3 · Latent up-projection", moe_infer):
 *   out[t] = bf16( sum_{slot} topk_w[t, slot] * y_routed[inv_perm[t*k + slot]] + y_shared[t] )
 * with y_routed [T*k, d] and y_shared [T, d] fp32, summed in fp32 in slot order, one
 * rounding to bf16.  inv_perm = -1 slots add nothing;
 * y_shared may be NULL. */
moe_status moe_combine(const moe_dims* dims, const float* y_routed, const int32_t* inv_perm,
                       const float* topk_w, const float* y_shared, uint16_t* out,
                       void* stream);

/* The whole layer: route, permute, gate/up, down, combine; out [T, d] bf16.
 * Shared expert used iff d_shared > 0 (then ws1, ws3, ws2 must be non-NULL).
 * Inside the call the expert outputs (routed rows and the shared expert's) are kept in
 * the workspace as 24-bit floats: each fp32 result of the down projection with its 8
 * lowest mantissa bits cleared (16 significant bits, toward zero), 3 bytes per value
 * instead of 4.  That is 2^-15 of each value at most, against the 2^-9 of the output's
 * own bf16 rounding.  The output is bit-identical to moe_combine applied to
 * moe_expert_down's fp32 rows cut the same way. */
moe_status moe_forward(const moe_dims* dims, const uint16_t* x, const float* w_router,
                       const float* bias, const uint16_t* w1, const uint16_t* w3,
                       const uint16_t* w2, const uint16_t* ws1, const uint16_t* ws3,
                       const uint16_t* ws2, uint16_t* out, void* ws, size_t ws_bytes,
                       void* stream);

/* moe_forward for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments, kernels and
 * results as moe_forward, but no workspace argument: the intermediates live in a device
 * array of MOE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on (from
 * the module's load until the process ends).  The call itself allocates nothing.
 *   - Limit: moe_workspace_bytes(dims) <= MOE_NOALLOC_SCRATCH_BYTES, else MOE_ESCRATCH
 *     before anything is launched.  At the K2 shape (d 7168, 384 experts, top-8, I 2048,
 *     shared expert) that admits up to 512 tokens.
 *   - The array of the CURRENT device is used: `stream` must belong to it.
 *   - Every call on one GPU shares that GPU's array.  Calls that overlap on one GPU (on
 *     different streams, or from different host threads without ordering) race on it and
 *     give undefined results; calls ordered on one stream are safe.  Nothing in the array
 *     needs to start at zero: every call writes each intermediate before reading it. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
moe_status moe_forward_noalloc(const moe_dims* dims, const uint16_t* x, const float* w_router,
                               const float* bias, const uint16_t* w1, const uint16_t* w3,
                               const uint16_t* w2, const uint16_t* ws1, const uint16_t* ws3,
                               const uint16_t* ws2, uint16_t* out, void* stream);

/* For callers that go through many workspaces over a long run, such as a server that
 * captures graphs on freshly allocated workspaces: tells the library that the workspace
 * at `ws` (an address passed to earlier calls) will not be used again, so that its slot of
 * the router's arrival counts (see the conventions above) may go to another workspace,
 * including a slot held because a call on `ws` was captured into a graph.  Call it only
 * when no launch using `ws` is pending and no graph holding such launches will be
 * replayed.  Host-side bookkeeping only: nothing is launched.  An address the library has
 * not seen, or NULL, is ignored.  Always MOE_OK. */
moe_status moe_workspace_release(const void* ws);

/* The MoE half of a transformer block, with the steps either side of the layer fused in
 * ("Kimi K2 · Transformer blocks", MoE transformer block: x_ffn = RMSNorm(x'_n), the
 * mixture of experts on x_ffn, then x_{n+1} = x'_n + Delta_ffn; the block order of the
 * DeepseekV3DecoderLayer forward printed on the same page: post-attention RMSNorm, MLP,
 * residual add, with rms_norm_eps 1e-6 in the config):
 *   x_ffn[t] = bf16( x_res[t] / sqrt(mean(x_res[t]^2) + norm_eps) * norm_w )
 *   out[t]   = bf16( x_res[t] + Delta_ffn(x_ffn)[t] )
 * x_res [T, d] bf16 is the residual stream x'_n; norm_w [d] fp32 is the RMSNorm gain
 * (4-byte aligned; a bf16 checkpoint gain converts exactly); norm_eps >= 0, finite.
 * The norm is computed in fp64 and rounded to fp32, then to bf16 (round-to-nearest-even
 * both times); Delta_ffn is moe_forward's fp32 sum, the residual is added to it in fp32
 * and the total rounded to bf16 once.  out and x_res must not overlap (MOE_EINVAL).
 * Workspace: moe_block_workspace_bytes (moe_workspace_bytes plus the bf16 x_ffn, which
 * the call leaves at byte offset moe_workspace_bytes(dims) of ws). */
moe_status moe_block_workspace_bytes(const moe_dims* dims, size_t* bytes);
moe_status moe_forward_block(const moe_dims* dims, const uint16_t* x_res, const float* norm_w,
                             float norm_eps, const float* w_router, const float* bias,
                             const uint16_t* w1, const uint16_t* w3, const uint16_t* w2,
                             const uint16_t* ws1, const uint16_t* ws3, const uint16_t* ws2,
                             uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/* FP8 block-scaled expert weights, the form K2's checkpoints store them in ("nnterp
 * encyclopedia · kimi_k2", loading a K2 checkpoint: FP8 blocks with per-block scales;
 * the parameter table of "Kimi K2 · Transformer blocks" leaves the block scales out).
 * Codes are OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, S.1111.111 = NaN), one byte per weight in the bf16 layouts above; one fp32
 * scale per 128 x 128 block of each [out, in] matrix; weight = code value x scale.
 * The kernels dequantise exactly: codes become bf16 without rounding, and each 128-k
 * block's fp32 partial sum is multiplied by its scale.  Requires d and I (and Is) to be
 * multiples of 128 and at most 16384 (else MOE_EUNSUPPORTED).  All pointers are device
 * pointers; codes 16-byte aligned, scales 4-byte aligned; the shared expert's six
 * pointers are used iff d_shared > 0.  The router weights stay fp32 (moe_forward_fp8's
 * w_router). */
typedef struct moe_fp8_weights {
  const uint8_t* w1;       /* [E, I, d] */
  const uint8_t* w3;       /* [E, I, d] */
  const uint8_t* w2;       /* [E, d, I] */
  const float* w1_scale;   /* [E, I/128, d/128] */
  const float* w3_scale;   /* [E, I/128, d/128] */
  const float* w2_scale;   /* [E, d/128, I/128] */
  const uint8_t* ws1;      /* [Is, d] */
  const uint8_t* ws3;      /* [Is, d] */
  const uint8_t* ws2;      /* [d, Is] */
  const float* ws1_scale;  /* [Is/128, d/128] */
  const float* ws3_scale;  /* [Is/128, d/128] */
  const float* ws2_scale;  /* [d/128, Is/128] */
} moe_fp8_weights;

/* moe_expert_gate_up / moe_expert_down / moe_forward with FP8 expert weights (`w` is a
 * host pointer to the struct of device pointers); same workspace (moe_workspace_bytes),
 * outputs and semantics otherwise (moe_forward_fp8 keeps 24-bit expert rows inside the
 * call as moe_forward does). */
moe_status moe_expert_gate_up_fp8(const moe_dims* dims, const uint16_t* x,
                                  const int32_t* perm_rows, const int32_t* offsets,
                                  const moe_fp8_weights* w, uint16_t* h, void* ws,
                                  size_t ws_bytes, void* stream);
moe_status moe_expert_down_fp8(const moe_dims* dims, const uint16_t* h, const int32_t* offsets,
                               const moe_fp8_weights* w, float* y_routed, float* y_shared,
                               void* ws, size_t ws_bytes, void* stream);
moe_status moe_forward_fp8(const moe_dims* dims, const uint16_t* x, const float* w_router,
                           const float* bias, const moe_fp8_weights* w, uint16_t* out,
                           void* ws, size_t ws_bytes, void* stream);

/* Latent mixture of experts ("Kimi K3 · Latent up-projection", the module's forward and its
 * projection parameters):
 *   z, s, sel, G as in moe_route, computed on the full-width x;
 *   l = x W_down^T  [T, L] (bf16);
 *   u = sum_i G_i E_i(l)  (SwiGLU experts of input and output width L);
 *   u_hat = u / sqrt(mean(u^2) + 1e-6)  (unit gain; the norm precedes W_up; u_hat enters
 *   the up-projection rounded to bf16, or as two bf16 parts when L <= 1024);
 *   out = bf16(u_hat W_up^T + y_shared(x))  (shared expert on the full width).
 *   w_down [L, d] bf16; w1, w3 [E, I, L]; w2 [E, L, I]; w_up [d, L] bf16; shared expert
 *   [Is, d] / [d, Is] on the full width; out [T, d] bf16.  d_latent: multiple of 64,
 *   at most 8192.  Workspace from moe_latent_workspace_bytes. */
moe_status moe_latent_workspace_bytes(const moe_dims* dims, int32_t d_latent, size_t* bytes);
moe_status moe_forward_latent(const moe_dims* dims, int32_t d_latent, const uint16_t* x,
                              const float* w_router, const float* bias, const uint16_t* w_down,
                              const uint16_t* w1, const uint16_t* w3, const uint16_t* w2,
                              const uint16_t* w_up, const uint16_t* ws1, const uint16_t* ws3,
                              const uint16_t* ws2, uint16_t* out, void* ws, size_t ws_bytes,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
