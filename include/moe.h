/*
 * moe.h - C ABI of an MI355X (gfx950) library for the forward pass of a
 * top-k routed Mixture-of-Experts FFN layer.
 *
 * Page keys used in the citations below (web pages; sections as printed):
 *   [P1] "Naive-N0.5-Flash" open-source MoE blog, wzjinhao.cn/news/74695
 *   [P2] "The quietly activated expert group" MoE explainer, mqxn.cn/news/15586
 *   [P3] "Small MoE language model from scratch" tutorial, lshu.cn/news/325687
 *   [P4] "OpenMythos" re-implementation blog, lpnh.cn/news/1735864
 *   [P5] FLAME-MoE research-platform summary, lsdiaocha.cn/2025/0530/3166997.shtml
 *
 * Conventions shared by every call
 *   - All tensor arguments are device pointers owned by the caller; the
 *     library never allocates, frees or synchronises.  Work is enqueued on
 *     `stream` and results are valid once the caller has synchronised it.
 *   - Matrices are row-major.  Weights use the nn.Linear [out, in] layout, so
 *     both operands of every product are contiguous along the reduction.
 *   - "act-dtype" tensors (x, expert weights and biases, intermediate and
 *     output activations) are float32 when cfg->dtype == MOE_DTYPE_F32 and
 *     bfloat16 when cfg->dtype == MOE_DTYPE_BF16.  Router bias, routing
 *     weights and log-sum-exp values are always float32; indices int32.
 *     Expert weights may instead be INT8 codes with float32 row scales
 *     (cfg->weight_format, moe_weight_format).
 *   - Pointers to act-dtype and int32 data must be 16-byte aligned and
 *     d_model and d_ffn must be multiples of 8 (rows are read with 16-byte
 *     vector loads).
 *   - Workspace: calls that need scratch memory take (ws, ws_bytes).  With
 *     ws == NULL the call only writes the required size to *ws_bytes and
 *     returns MOE_OK (query mode, nothing is launched).  Otherwise *ws_bytes
 *     must hold the size of ws; if it is too small the required size is
 *     written back and MOE_ERR_WORKSPACE is returned.
 *   - Errors are reported before anything is enqueued; on error nothing is
 *     written.  A failed launch returns MOE_ERR_HIP.  No C++ exception
 *     crosses this interface.
 *   - Results are deterministic: there are no floating-point atomics, and
 *     every reduction runs in a fixed order.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null required pointer, bad size or option */
  MOE_ERR_UNSUPPORTED = 2, /* valid but not built (e.g. n_experts > 512) */
  MOE_ERR_WORKSPACE = 3,   /* workspace too small; *ws_bytes = required */
  MOE_ERR_HIP = 4          /* a HIP launch failed */
} moe_status;

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype;

/* Expert FFN form.  GELU: out = W2 gelu(W1 x + b1) + b2 with the exact erf
 * GELU ([P3 §3.1]).  SWIGLU: out = W2 (silu(W1g x) * (W1u x)) with W1 the
 * gate rows followed by the up rows ([P2 §3.1] names SwiGLU experts). */
typedef enum { MOE_ACT_GELU = 0, MOE_ACT_SWIGLU = 1 } moe_act;

/* Storage of the expert weights (W1, W2 of the routed and the shared
 * experts; router weights and biases always use the activation dtype).
 * ACT: the activation dtype.  INT8: 8-bit codes q with one float32 scale per
 * weight row, W[n, :] = scale[n] * q[n, :] ([P3 §6]: compress each expert's
 * weights to INT8 for deployment; the per-row symmetric scheme is this
 * library's reading).  INT8 needs BF16 activations and d_model, d_ffn
 * multiples of 128 (else MOE_ERR_UNSUPPORTED).  Accumulation is float32 as
 * for bf16 weights.  Where a product's reduction runs over one weight matrix
 * (every gate/up product, and the down product of routed experts or of a
 * single shared expert) the codes enter the matrix cores exactly and the
 * float32 sum of each output column is multiplied by its row scale.  The
 * down product that sums n_seg > 1 shared experts multiplies each code by
 * its scale and rounds the product to bfloat16 (to nearest even) first. */
typedef enum { MOE_WEIGHTS_ACT = 0, MOE_WEIGHTS_INT8 = 1 } moe_weight_format;

typedef struct {
  int64_t n_tokens;       /* T >= 1: tokens (batch * seq), [P3 §3.1] flattening */
  int32_t d_model;        /* d: hidden size */
  int32_t n_experts;      /* E: routed experts, 1 <= E <= 512 */
  int32_t top_k;          /* k: 1 <= k <= E ([P4 §2.1]: configurable k) */
  int32_t d_ffn;          /* f: expert intermediate size */
  int32_t n_shared;       /* S >= 0: always-active shared experts ([P4 §2.1]) */
  int32_t dtype;          /* moe_dtype */
  int32_t act;            /* moe_act */
  double capacity_factor; /* <= 0: no limit; else C = ceil(cf*T*k/E), exact on
                             the binary64 value of cf ([P4 §3.1]); NaN rejected */
  int32_t add_residual;   /* 1: y += x ([P2 §4.1] adds the input inside the layer) */
  int32_t weight_format;  /* moe_weight_format of the expert weights */
  float router_temperature; /* tau: the router's scores are logits / tau
                               ([P2 §5.1] temperature scaling to soften an
                               over-confident router); 0 means 1; otherwise
                               finite, > 0 and with 1/tau finite, else
                               INVALID_ARG */
} moe_config;

/* Device pointers to one layer's parameters (host struct, read during the call). */
typedef struct {
  const void* w_router;     /* [E, d] act-dtype, required */
  const float* router_bias; /* [E] float32 logit bias added before the softmax, or NULL */
  const void* w1;           /* [E, 2f, d] (SWIGLU: gate rows then up rows) or [E, f, d] (GELU) */
  const void* b1;           /* [E, 2f] / [E, f] act-dtype, or NULL */
  const void* w2;           /* [E, d, f] */
  const void* b2;           /* [E, d] act-dtype, or NULL */
  const void* shared_w1;    /* [S, 2f, d] / [S, f, d]; required iff S > 0 */
  const void* shared_b1;    /* [S, 2f] / [S, f] or NULL */
  const void* shared_w2;    /* [S, d, f]; required iff S > 0 */
  const void* shared_b2;    /* [S, d] or NULL */
  /* weight_format INT8: w1 / w2 / shared_w1 / shared_w2 hold int8 codes and
   * these hold one float32 scale per weight row (required with them);
   * ignored otherwise */
  const float* w1_scale;        /* [E, 2f] / [E, f] */
  const float* w2_scale;        /* [E, d] */
  const float* shared_w1_scale; /* [S, 2f] / [S, f] */
  const float* shared_w2_scale; /* [S, d] */
} moe_weights;

/* Auxiliary statistics, written to device memory.
 * f_e = counts_e / (T*k) with the counts taken before capacity, P_e = mean
 * over all tokens of the full softmax ([P4 §3.1] load-balance loss
 * E * sum f_e P_e); z = mean over tokens of logsumexp(scores)^2 (router
 * z-loss named in [P5 §2]); weighted = 0.01 lb + 0.001 z, the coefficients
 * [P5 §2] reports.  The other load-balance forms the pages give, unweighted:
 * lb_squares = E * sum_e P_e^2 ([P3 §3.1]); kl_uniform = sum_e (1/E)
 * (ln(1/E) - ln(P_e + 1e-8)), the KL divergence of the uniform distribution
 * from P with the page's 1e-8, and freq_penalty = sum_e (f_e - 1/E)^2
 * ([P2 §4.2]; its alpha of 0.001-0.01 is the caller's). */
typedef struct {
  double load_balance;
  double z_loss;
  double weighted;
  int64_t n_dropped; /* assignments over capacity */
  int64_t capacity;  /* C, or -1 when there is no limit */
  int64_t n_kept;    /* R = T*k - n_dropped */
  double lb_squares;
  double kl_uniform;
  double freq_penalty;
} moe_aux;

/* Static description of a status code. */
const char* moe_status_string(moe_status s);

/*
 * moe_route - router GEMM, softmax, top-k and renormalisation
 * ([P2 §3.2] a single linear layer; [P3 §3.1] steps 1-2; [P4 §3.1]
 * routing and top-k selection).
 *   logits[t,e] = sum_c x[t,c] W_r[e,c] + router_bias[e]   (float32 accumulate)
 *   s[t,e] = logits[t,e] / tau + router_noise[t,e]
 *   p = softmax_e(s), lse[t] = logsumexp_e(s[t,:])
 *   topk_idx[t,:] = the k experts of largest score (= largest p), sorted by
 *                   descending score, lower index first on exact ties; a
 *                   NaN score ranks below every number (the k indices stay
 *                   distinct; a NaN pick gets weight 0)
 *   topk_w[t,j]   = p[t,idx] / sum_j' p[t,idx']
 * tau = cfg->router_temperature ([P2 §5.1]); router_noise [T,E] float32 or
 * NULL: a perturbation the caller draws, added before the top-k ([P2 §2.2]
 * noisy top-k; [P3 §6] routing noise for exploration).
 * x [T,d], w_router [E,d] act-dtype; router_bias [E] float32 or NULL;
 * topk_idx [T,k] int32, topk_w [T,k] float32, token_lse [T] float32 (may be
 * NULL).  The call also leaves per-block routing statistics (expert counts,
 * probability sums, sum of lse^2) in ws; moe_aux_stats reads them from the
 * same ws, which must not be reused in between.  INVALID_ARG for a
 * misaligned (4-byte) router_noise.
 */
moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* router_bias, const float* router_noise, int32_t* topk_idx,
                     float* topk_w, float* token_lse, void* ws, size_t* ws_bytes,
                     hipStream_t stream);

/*
 * moe_permute - per-expert counts, capacity and a stable expert-contiguous
 * permutation ([P4 §3.1] capacity/overflow and its flatten-and-reorder
 * dispatch; [P1 §2.2] expert capacity).
 *   expert_counts[e] = #{(t,j): topk_idx[t,j] == e}          (before capacity)
 *   within expert e the assignments are ranked by ascending token index; the
 *   first C are kept (all without a limit); kept rows are ordered by
 *   (expert, token): expert_offsets[E+1] is the exclusive scan of the kept
 *   counts, perm_token[row] = t, perm_w[row] = topk_w[t,j],
 *   inv_row[t,j] = row or -1 if dropped, *n_dropped = dropped assignments.
 * topk_idx [T,k] int32 with values in [0,E) and the k indices of a token
 * distinct (checked on device: an index out of range, or a repeat of an
 * expert the token already lists, is counted as dropped and reported through
 * n_dropped = -1; the outputs are then those of the table without it);
 * topk_w [T,k] float32 (required iff perm_w != NULL); x [T,d] act-dtype
 * (required iff x_perm != NULL); outputs: expert_counts [E],
 * expert_offsets [E+1], perm_token [T*k] (first R entries valid),
 * perm_w [T*k] or NULL, inv_row [T*k], x_perm [T*k, d] or NULL (row r =
 * x[perm_token[r]]), n_dropped [1] int32.
 */
moe_status moe_permute(const moe_config* cfg, const int32_t* topk_idx, const float* topk_w,
                       const void* x, int32_t* expert_counts, int32_t* expert_offsets,
                       int32_t* perm_token, float* perm_w, int32_t* inv_row, void* x_perm,
                       int32_t* n_dropped, void* ws, size_t* ws_bytes, hipStream_t stream);

/*
 * moe_expert_ffn - grouped expert FFN over expert-contiguous rows
 * ([P4 §3.1] run every expert on its gathered rows; [P1 §4.2] group tokens
 * by expert and run one large product per expert).
 * Group g covers rows [group_offsets[g], group_offsets[g+1]) (device array,
 * non-decreasing, last entry <= rows_max); group_offsets may be NULL only
 * with n_groups == 1, meaning one dense group of rows_max rows.  Row r reads A row
 * a_rows ? a_rows[r] : r of `a` [*, d].  Each group is the sum of n_seg
 * FFNs of width f with weight 1 (n_seg = 1 for routed experts; the S shared
 * experts form one group with n_seg = S):
 *   out[r,:] = sum_{s<n_seg} FFN_{g*n_seg+s}(a[row(r),:])
 * w1 [n_groups*n_seg, 2f or f, d], b1 [.., 2f or f] or NULL,
 * w2 [n_groups*n_seg, d, f], b2 [.., d] or NULL, out [rows_max, d]; rows of
 * out outside every group are not written.  ws holds the intermediate
 * activations (rows_max x n_seg*f, act dtype).  Errors: INVALID_ARG for
 * n_groups < 1, n_seg outside [1, 64], rows_max < 0, NULL offsets with
 * n_groups > 1, NULL or misaligned a / w1 / w2 / out, weight_format other
 * than ACT (INT8 weights go through moe_expert_ffn_int8); UNSUPPORTED for
 * rows_max >= 2^31.  rows_max == 0 launches nothing.
 */
moe_status moe_expert_ffn(const moe_config* cfg, int32_t n_groups, int32_t n_seg,
                          int64_t rows_max, const void* a, const int32_t* a_rows,
                          const int32_t* group_offsets, const void* w1, const void* b1,
                          const void* w2, const void* b2, void* out, void* ws,
                          size_t* ws_bytes, hipStream_t stream);

/*
 * moe_expert_ffn_int8 - moe_expert_ffn with 8-bit expert weights ([P3 §6]:
 * experts compressed to INT8 for deployment).  cfg->weight_format must be
 * MOE_WEIGHTS_INT8.  w1 [n_groups*n_seg, 2f or f, d] and w2
 * [n_groups*n_seg, d, f] hold int8 codes; w1_scale [n_groups*n_seg, 2f or f]
 * and w2_scale [n_groups*n_seg, d] one float32 scale per weight row
 * (W[n, :] = scale[n] * q[n, :]); everything else as in moe_expert_ffn.
 * Errors as moe_expert_ffn, plus INVALID_ARG for NULL or misaligned
 * (4-byte) scales and UNSUPPORTED for shapes INT8 weights do not cover
 * (see moe_weight_format).
 */
moe_status moe_expert_ffn_int8(const moe_config* cfg, int32_t n_groups, int32_t n_seg,
                               int64_t rows_max, const void* a, const int32_t* a_rows,
                               const int32_t* group_offsets, const int8_t* w1,
                               const float* w1_scale, const void* b1, const int8_t* w2,
                               const float* w2_scale, const void* b2, void* out, void* ws,
                               size_t* ws_bytes, hipStream_t stream);

/*
 * moe_combine - weighted gather back to token order, atomic-free
 * ([P1 §2.1] weighted sum of the selected experts; [P5 §2] weights are the
 * normalised routing scores; [P2 §4.1] optional residual).
 *   y[t,:] = shared_y[t,:] + sum_{j: inv_row[t,j] >= 0} topk_w[t,j] * y_perm[inv_row[t,j],:]
 *            (+ residual[t,:])
 * summed in float32 in the order shared, j = 0..k-1, residual.
 * y_perm [R,d] (required, also when every slot is dropped), shared_y [T,d]
 * or NULL, residual [T,d] or NULL, y [T,d] act-dtype; inv_row [T,k] int32;
 * topk_w [T,k] float32.  INVALID_ARG for a NULL y_perm, inv_row, topk_w or
 * y, or a misaligned (16-byte) act-dtype pointer.
 */
moe_status moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* inv_row,
                       const float* topk_w, const void* shared_y, const void* residual,
                       void* y, hipStream_t stream);

/*
 * moe_aux_stats - load-balance and z-loss statistics ([P4 §3.1]
 * load-balance loss; [P5 §2] router z-loss and coefficients) from the
 * routing statistics moe_route left in route_ws, the pre-capacity
 * expert_counts [E] and n_dropped [1] of moe_permute.  Writes one moe_aux
 * to device memory `aux`.  route_ws / route_ws_bytes are the workspace
 * given to moe_route.
 */
moe_status moe_aux_stats(const moe_config* cfg, const int32_t* expert_counts,
                         const int32_t* n_dropped, const void* route_ws, size_t route_ws_bytes,
                         moe_aux* aux, hipStream_t stream);

/*
 * moe_forward - the whole layer: route, permute, routed and shared expert
 * FFNs, combine and aux statistics ([P3 §3.1] forward returns the output
 * and the auxiliary loss).  x, y [T,d] act-dtype.  router_noise [T,E]
 * float32 or NULL as in moe_route.  Optional outputs (NULL to skip):
 * topk_idx [T,k], topk_w [T,k], expert_counts [E], aux (device).
 * Expert weights per cfg->weight_format (INT8: the scale pointers of `w`
 * for the routed experts, and for the shared ones when S > 0, are
 * required).  ws: query with ws == NULL.
 */
moe_status moe_forward(const moe_config* cfg, const moe_weights* w, const void* x,
                       const float* router_noise, void* y, int32_t* topk_idx, float* topk_w,
                       int32_t* expert_counts, moe_aux* aux, void* ws, size_t* ws_bytes,
                       hipStream_t stream);

/*
 * moe_forward_static - moe_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The same layer and arguments as moe_forward, without
 * the workspace: the scratch memory is a static device array of
 * MOE_STATIC_SCRATCH_BYTES inside the library, one copy per GPU, held from
 * the first call on that GPU until the process ends (that first call looks
 * up the array's device address; no call allocates or frees anything).
 * Layers whose scratch need (moe_forward's workspace query) exceeds the
 * array are rejected with MOE_ERR_WORKSPACE before anything is launched;
 * 64 MiB covers, for example, 4096 tokens of a 512-wide, 16-expert top-2
 * layer with d_ffn 1024, or 128 decode tokens of a 7168-wide, 256-expert
 * top-8 layer.  Every call on one GPU uses the same array and leaves its
 * contents behind: calls that overlap in time on one GPU (other streams,
 * other threads) race, and the caller must order them.
 */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_static(const moe_config* cfg, const moe_weights* w, const void* x,
                              const float* router_noise, void* y, int32_t* topk_idx, float* topk_w,
                              int32_t* expert_counts, moe_aux* aux, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Training: the forward with the state the backward needs, and the backward
 * ([P3 §4.2] trains on loss = task loss + auxiliary loss and back-propagates
 * both; [P5 §2] weights load balance 0.01 and z-loss 0.001).
 */

/* Forward state kept for the backward: device buffers the caller owns, all
 * required (shared_preact only when S > 0).  scores [T,E] float32 (s of
 * moe_route), token_lse [T] float32, topk_idx [T,k] int32, topk_w [T,k]
 * float32, expert_counts [E] int32, expert_offsets [E+1] int32, perm_token
 * [T*k] int32, inv_row [T*k] int32, y_perm [T*k, d] act dtype (each kept
 * row's expert output), preact [T*k, 2f|f] act dtype (each kept row's
 * pre-activations x W1^T + b1, SwiGLU gate then up), shared_preact
 * [T, S*(2f|f)] act dtype (the shared experts' pre-activations, expert s at
 * columns s*(2f|f)). */
typedef struct {
  float* scores;
  float* token_lse;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* expert_counts;
  int32_t* expert_offsets;
  int32_t* perm_token;
  int32_t* inv_row;
  void* y_perm;
  void* preact;
  void* shared_preact;
} moe_saved;

/* Gradients written by moe_backward (device buffers the caller owns; each is
 * overwritten, not accumulated).  dx [T,d] act dtype and dw_router [E,d]
 * float32 are required; drouter_bias [E] may be NULL.  Expert weight
 * gradients are float32 in the weights' layouts: dw1 [E, 2f|f, d],
 * dw2 [E, d, f] required; db1 [E, 2f|f] and db2 [E, d] required iff the
 * layer has b1 / b2.  With S > 0: dws1 [S, 2f|f, d] and dws2 [S, d, f]
 * required, dsb1 / dsb2 iff the shared biases exist. */
typedef struct {
  void* dx;
  float* dw_router;
  float* drouter_bias;
  float* dw1;
  float* db1;
  float* dw2;
  float* db2;
  float* dws1;
  float* dsb1;
  float* dws2;
  float* dsb2;
} moe_grads;

/* Weights of the auxiliary terms in the training loss (moe_backward):
 * L_aux = load_balance * lb + z_loss * z + lb_squares * (E sum P^2)
 *       + kl_uniform * KL(uniform || P), the quantities of moe_aux.  The
 * pages train with 0.01 lb + 0.001 z ([P5 §2]); [P3 §3.1] uses
 * 0.01 E sum P^2 and [P2 §4.2] alpha (KL + frequency penalty), whose
 * frequency part depends on the selection only and has no gradient. */
typedef struct {
  double load_balance;
  double z_loss;
  double lb_squares;
  double kl_uniform;
} moe_loss_weights;

/*
 * moe_forward_train - moe_forward that also fills `saved` for moe_backward.
 * Arguments as moe_forward; saved (host struct of device pointers) is
 * required.  BF16 activations with activation-dtype expert weights only
 * (else MOE_ERR_UNSUPPORTED).
 */
moe_status moe_forward_train(const moe_config* cfg, const moe_weights* w, const void* x,
                             const float* router_noise, void* y, const moe_saved* saved,
                             moe_aux* aux, void* ws, size_t* ws_bytes, hipStream_t stream);

/*
 * moe_backward - gradients of  L = sum(dy * y) + L_aux  with respect to x
 * and every parameter, for the forward that filled `saved` (same cfg,
 * weights, x and router noise).  L_aux per `lw` (moe_loss_weights; NULL:
 * 0.01 lb + 0.001 z).  Top-k selection, capacity drops and the selection
 * shares f_e pass no gradient.
 *   combine: d o_tj = w_tj dy_t (kept slots), dw_tj = dy_t . o_tj;
 *   experts: a = x W1^T + b1 (saved); dW2 = d o^T act(a), dh = d o W2,
 *            da = dh * act'(a), dW1 = da^T x, dx += da W1 (rows added back
 *            to their tokens); shared experts with d o = dy; residual: dx += dy;
 *   router:  renormalisation, aux terms (d lb / d p_te = E f_e / T,
 *            d z / d s_te = 2 lse_t p_te / T, d (E sum P^2) / d p_te =
 *            2 E P_e / T, d KL / d p_te = -1 / (E (P_e + 1e-8) T)), softmax,
 *            then / tau:
 *            dW_r = dl^T x, d bias = sum_t dl, dx += dl W_r.
 * x, dy [T,d] act dtype.  Precision: bf16 operands with float32
 * accumulation; d o, a, dh, da and act(a) are stored as bf16 between the
 * steps.  BF16 activation-dtype weights only (else UNSUPPORTED); NULL
 * required buffers or a non-finite loss weight: INVALID_ARG.  ws: query
 * with ws == NULL.
 */
moe_status moe_backward(const moe_config* cfg, const moe_weights* w, const void* x,
                        const moe_saved* saved, const void* dy, const moe_loss_weights* lw,
                        const moe_grads* g, void* ws, size_t* ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
