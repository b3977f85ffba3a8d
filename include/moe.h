/*
 * libmoe_mi355x — forward and backward pass of one Mixture-of-Experts FFN
 * layer on one AMD MI355X (gfx950), as a C ABI.
 *
 * The layer (pages cited by title and section):
 *   router      logits = Wr x + br, one output per expert
 *               ("MoE混合专家模型：Transformer稀疏前馈网络原理与PyTorch实现", 2.1;
 *                "手撕一个极简 MoE-FFN", 三)
 *   gate        softmax over experts, or per-expert sigmoid normalized over all
 *               experts ("MoE架构解析", 四 技术飞跃③)
 *   top-k       the k highest-scoring experts per token, their scores
 *               renormalized to sum to 1 (0539edu page 2.1; kamacoder 三 and its
 *               worked example)
 *   dispatch    tokens grouped per expert, at most C per expert; the rest are
 *               dropped and contribute nothing ("MoE架构解析", 三 关键技术①)
 *   experts     Linear -> ReLU / GELU -> Linear with biases, or SwiGLU
 *               (kamacoder 四; 0539edu 4.1; learn-minimind guide 二), plus
 *               always-active shared experts ("MoE架构解析", 四 技术飞跃②)
 *   combine     y = sum over the kept slots of w * Expert(x) (+ shared)
 *               (0539edu 1.3; kamacoder 五)
 *   aux stats   f_e, P_e, L_aux = E * sum f_e P_e (0539edu 2.3; kamacoder 七)
 *
 * Conventions for every entry point
 *   - Array arguments are DEVICE pointers owned by the caller; moe_problem,
 *     moe_weights and moe_routing are HOST structs holding device pointers.
 *   - Work is enqueued on `stream` (NULL = the default stream) and nothing
 *     synchronizes with the host; buffers must stay alive until the stream
 *     has passed the work.  No entry point allocates or frees memory; scratch
 *     space is the caller's workspace of moe_workspace_size() bytes (256-byte
 *     aligned).  No pointer is kept after a call returns.
 *   - All validation happens before anything is launched: on an error return
 *     nothing was launched and no output was written.  MOE_ERR_HIP means a
 *     launch failed (moe_last_hip_error() gives the hipError_t of the calling
 *     thread); asynchronous faults surface at the caller's next sync.
 *   - Identical inputs give bit-identical outputs (no floating-point atomics,
 *     fixed reduction orders, stable dispatch).
 *   - Layouts are row-major.  Weights use the nn.Linear [out, in] layout.
 *     x and all weights and biases share `dtype`; y, topk_w, probs and the
 *     statistics are float32; indices are int32.
 *   - Shared experts are experts E .. E+S-1 of the weight arrays.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* a size, enum, flag or required pointer is invalid     */
  MOE_ERR_UNSUPPORTED = 2,   /* valid, but outside this library's limits (see below)  */
  MOE_ERR_WORKSPACE = 3,     /* workspace NULL or smaller than moe_workspace_size()   */
  MOE_ERR_HIP = 4            /* a HIP launch failed                                   */
};

enum { MOE_F32 = 0, MOE_BF16 = 1 };                      /* dtype of x, weights, biases */
enum { MOE_SOFTMAX = 0, MOE_SIGMOID_NORM = 1 };          /* gate                        */
enum { MOE_RELU = 0, MOE_GELU = 1, MOE_SWIGLU = 2 };     /* expert activation           */
enum { MOE_ROUTER_BIAS = 1, MOE_EXPERT_BIAS = 2,        /* flags                       */
       MOE_W_FP8 = 8,           /* expert weights as FP8 E4M3 codes with per-row scales (moe_weights) */
       MOE_EXPERT_CHOICE = 16 };/* expert-choice routing (see moe_expert_choice)                  */

/*
 * The problem.  T tokens (the pages' [B, L, d] input flattened to [B*L, d],
 * 0539edu page 4.1), E routed experts of which each token takes top_k, S
 * always-on shared experts, per-expert capacity (<= 0: unlimited).
 *
 * Limits (MOE_ERR_UNSUPPORTED beyond them): E <= 64, top_k <= 8,
 * E + S <= 128, T * (top_k + S) < 2^31, F1 * d_model < 2^30 (F1 = d_ff, or
 * 2 d_ff for SwiGLU: one expert's weights); for MOE_BF16, d_model and d_ff
 * are multiples of 8 and T * d_model, T * d_ff < 2^31 (the kernels address
 * token rows and one expert's rows with 32-bit byte offsets).  When both are
 * multiples of 64 the expert FFNs run on the tiled grouped GEMMs (and the
 * weight-streaming kernels for T <= 128); otherwise on an untiled grouped GEMM
 * that is correct for any multiple of 8 but slower.  GELU is the exact erf
 * form; SwiGLU has no biases.
 * MOE_W_FP8 (expert weights quantized to 8 bits, 0539edu page 5.2) needs
 * MOE_BF16, T <= 128 (the weight-streaming decode path) and d_model, d_ff
 * multiples of 128.
 * MOE_EXPERT_CHOICE ("MoE架构解析" 二 2.2: experts choose their tokens): every
 * expert takes exactly `capacity` tokens (1 <= capacity <= T, else
 * MOE_ERR_INVALID_ARG; T <= 16384); top_k is not used for routing.  The
 * routed rows are then E * capacity and, in every entry point below:
 * sorted_assign holds token ids (E * capacity of them, expert by expert, each
 * expert's tokens ascending), assign_row is the [T, E] row of each (token,
 * expert) pair (-1 where the expert did not take the token), the combine
 * weights are probs [T, E], and counts = kept = capacity.  moe_dispatch does
 * not apply (moe_expert_choice replaces it).
 */
typedef struct moe_problem {
  int32_t T, d_model, d_ff, num_experts, top_k, num_shared, capacity;
  int32_t dtype, gating, activation, flags;
} moe_problem;

/*
 * Weights (device pointers, `dtype`):
 *   w_router [E, d]         b_router [E]   (MOE_ROUTER_BIAS, else ignored)
 *   w_up     [E+S, F1, d]   b_up [E+S, F1] (MOE_EXPERT_BIAS, else ignored)
 *            F1 = d_ff, or 2*d_ff for SwiGLU: rows 0..d_ff-1 are the gate
 *            projection, rows d_ff..2*d_ff-1 the up projection
 *   w_down   [E+S, d, d_ff] b_down [E+S, d] (MOE_EXPERT_BIAS, else ignored)
 * For MOE_BF16 the down projection multiplies in fp16: each bf16 w_down value
 * is converted exactly when 2^-14 <= |w| < 65504 (smaller magnitudes are
 * truncated to fp16 subnormals, larger ones saturate).
 */
typedef struct moe_weights {
  const void *w_router, *b_router;
  const void *w_up, *b_up;
  const void *w_down, *b_down;
  /* MOE_W_FP8 only: w_up and w_down hold E4M3 codes (one byte each, same
   * shapes) and the dequantized weight of row r is code * scale[r]:
   *   s_up [E+S, F1] float32, s_down [E+S, d] float32 (see moe_quantize_fp8).
   * Ignored (may be NULL) otherwise. */
  const float *s_up, *s_down;
} moe_weights;

/*
 * Routing health indicators of one forward, written to device memory by
 * moe_routing_stats or moe_ffn_forward (0539edu 3.3: log the tokens each
 * expert actually processes, the routing entropy against the uniform
 * entropy ln N, and the variance of expert utilization; its troubleshooting
 * list judges balance by the coefficient of variation of utilization and
 * watches for experts at zero usage).
 *   entropy      -sum_e s_e ln s_e, s_e = counts[e] / (T*k): the share of
 *                routing decisions (before capacity drops); 0 ln 0 = 0
 *   entropy_p    -sum_e P[e] ln P[e] of the mean gate probabilities
 *   entropy_max  ln E (uniform routing)
 *   util_mean    mean over experts of kept[e] (tokens actually processed)
 *   util_var     population variance over experts of kept[e]
 *   util_cv      sqrt(util_var) / util_mean (0 when nothing is kept)
 *   dropped      sum_e (counts[e] - kept[e])
 *   idle         experts with kept[e] == 0
 */
typedef struct moe_route_stats {
  float entropy, entropy_p, entropy_max;
  float util_mean, util_var, util_cv;
  int32_t dropped, idle;
} moe_route_stats;

/*
 * Optional routing outputs of moe_ffn_forward (host struct; each device
 * pointer may be NULL, in which case the value lives only in the workspace).
 * Shapes and meaning as in moe_router_topk, moe_dispatch, moe_aux_stats and
 * moe_routing_stats.
 */
typedef struct moe_routing {
  int32_t *topk_idx;      /* [T, k]  */
  float *topk_w;          /* [T, k]  */
  float *probs;           /* [T, E]  */
  int32_t *counts;        /* [E]     */
  int32_t *kept;          /* [E]     */
  int32_t *offsets;       /* [E + 1] */
  int32_t *sorted_assign; /* [T * k] */
  int32_t *assign_row;    /* [T * k] */
  uint8_t *drop_mask;     /* [T * k] */
  float *f, *P, *l_aux;   /* [E], [E], [1] */
  moe_route_stats *stats; /* [1] (computed only when non-NULL) */
  int32_t *token_experts; /* [T] expert choice only: experts that took each token (0 = orphan) */
} moe_routing;

/* Host only.  Capacity ceil(capacity_factor * T * k / E): the page's
 * (tokens / experts) x CF ("MoE架构解析", 三 关键技术①) with the even share of
 * the T*k assignments as base (0539edu page 3.2: a multiple of the ideal even
 * share).  Returns 0 (= unlimited) when capacity_factor <= 0, -1 on invalid
 * T, k or E. */
int32_t moe_capacity(int32_t T, int32_t k, int32_t E, float capacity_factor);

/* Host only.  Workspace bytes needed by every entry point for this problem. */
moe_status moe_workspace_size(const moe_problem* p, size_t* bytes);

/*
 * Router, gate, top-k and renormalization (0539edu page 2.1; kamacoder 三;
 * "MoE架构解析" 四 技术飞跃③ for the normalized sigmoid).
 *   x           [T, d]  dtype
 *   topk_idx    [T, k]  out: experts in descending score, ties to the lower index
 *   topk_w      [T, k]  out: selected scores / their sum (softmax: probabilities,
 *                            sigmoid: sigma values; both give the same weights)
 *   probs       [T, E]  out, nullable: softmax p, or sigma / sum_e sigma
 *   prob_colsum [E]     out, nullable: sum over tokens of probs (fixed order)
 * With MOE_EXPERT_CHOICE probs is required and topk_idx, topk_w are ignored.
 */
moe_status moe_router_topk(const moe_problem* p, const void* x, const moe_weights* w,
                           int32_t* topk_idx, float* topk_w, float* probs,
                           float* prob_colsum, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Capacity-limited dispatch ("MoE架构解析", 三 关键技术①): assignments
 * a = t*k + s grouped by expert in ascending token order; each expert keeps
 * its first min(count, capacity) and drops the rest.
 *   topk_idx      [T, k] in   (each row: k distinct experts in [0, E))
 *   counts        [E]    out  assignments per expert before drops
 *   kept          [E]    out  min(counts, capacity)
 *   offsets       [E+1]  out  first row of each expert's kept rows; offsets[E]
 *                             = kept rows in total (shared expert q's rows then
 *                             start at offsets[E] + q*T)
 *   sorted_assign [T*k]  out  row r < offsets[E] holds assignment
 *                             sorted_assign[r]; the dropped assignments follow,
 *                             grouped by expert in token order
 *   assign_row    [T*k]  out  row of each assignment, -1 if dropped
 *   drop_mask     [T*k]  out  1 if dropped
 * Results are exact integers (bit-identical to any correct implementation).
 * Out-of-range ids are clamped into [0, E) (the result is then unspecified).
 * ws: moe_workspace_size() bytes; holds the per-16-token expert counts and
 * the per-512-token rank prefixes of the counting sort.
 */
moe_status moe_dispatch(const moe_problem* p, const int32_t* topk_idx, int32_t* counts,
                        int32_t* kept, int32_t* offsets, int32_t* sorted_assign,
                        int32_t* assign_row, uint8_t* drop_mask, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/*
 * Expert FFNs over the dispatched rows (kamacoder 四 and 六: one batch per
 * expert; shared experts on every token).  Row r < offsets[E] is token
 * sorted_assign[r] / k through expert e with offsets[e] <= r < offsets[e+1];
 * row offsets[E] + q*T + t is token t through shared expert q.
 *   y_exp [T*k + S*T, d] float32 out (only rows < offsets[E] + S*T written)
 * moe_expert_ffn = moe_expert_up followed by moe_expert_down with h in the
 * workspace.  h is [T*k + S*T, d_ff], float32 for MOE_F32 problems.  For
 * MOE_BF16 problems h holds fp16 bit patterns (uint16) of the activation
 * times 2^-8, and moe_expert_down multiplies its sums by 2^8 again: fp16
 * keeps 11 significant bits for |h| >= 2^-6 (an absolute step of 2^-16
 * below), and activations up to 65504 * 2^8 (about 1.68e7) in magnitude are
 * represented; larger ones saturate to that value (never inf; NaN stays NaN).
 * moe_expert_up uses no workspace (ws may be NULL); the others need
 * moe_workspace_size() bytes.
 */
moe_status moe_expert_ffn(const moe_problem* p, const void* x, const moe_weights* w,
                          const int32_t* offsets, const int32_t* sorted_assign, float* y_exp,
                          void* ws, size_t ws_bytes, hipStream_t stream);
moe_status moe_expert_up(const moe_problem* p, const void* x, const moe_weights* w,
                         const int32_t* offsets, const int32_t* sorted_assign, void* h,
                         void* ws, size_t ws_bytes, hipStream_t stream);
moe_status moe_expert_down(const moe_problem* p, const moe_weights* w, const int32_t* offsets,
                           const void* h, float* y_exp, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/*
 * Gate-weighted combine (0539edu 1.3 and 2.1; kamacoder 五):
 *   y[t] = sum over s with assign_row[t*k+s] >= 0 of topk_w[t,s] * y_exp[assign_row[t*k+s]]
 *          + sum over q < S of y_exp[offsets[E] + q*T + t]
 * A dropped slot adds nothing and the other weights are not renormalized.
 *   y [T, d] float32 out (every element written)
 */
moe_status moe_combine(const moe_problem* p, const float* topk_w, const int32_t* assign_row,
                       const int32_t* offsets, const float* y_exp, float* y,
                       hipStream_t stream);

/*
 * Load-balance statistics (0539edu 2.3; kamacoder 七):
 *   f[e] = counts[e] / (T * k)   (routing decisions before capacity drops)
 *   P[e] = prob_colsum[e] / T
 *   l_aux[0] = E * sum_e f[e] * P[e]   (without the weight alpha)
 */
moe_status moe_aux_stats(const moe_problem* p, const float* prob_colsum, const int32_t* counts,
                         float* f, float* P, float* l_aux, hipStream_t stream);

/*
 * Routing health indicators (see moe_route_stats) from the dispatch's
 * counts and kept [E] (int32) and the mean gate probabilities P [E]
 * (moe_aux_stats).  stats: one moe_route_stats in device memory.  Sums run
 * over experts in a fixed order: the result is deterministic.
 */
/*
 * Expert-choice routing ("MoE架构解析" 二 2.2: each expert picks the tokens it
 * scores highest, which balances the load exactly; a token may be picked by
 * several experts or by none).  Problem flag MOE_EXPERT_CHOICE.
 *   probs         [T, E] in   gate probabilities (moe_router_topk's probs)
 *   offsets       [E+1]  out  e * capacity
 *   sorted_assign [E * capacity] out  expert e's tokens in ascending order at
 *                              rows e*capacity .. (e+1)*capacity - 1: the
 *                              capacity tokens with the largest probs[t, e],
 *                              equal scores going to the lower token index
 *   row_of        [T, E] out  row of (t, e), or -1 if e did not take t
 *   token_experts [T]    out  number of experts that took t (may be NULL)
 * Integer results, exact given probs.  ws: moe_workspace_size() bytes.
 */
moe_status moe_expert_choice(const moe_problem* p, const float* probs, int32_t* offsets,
                             int32_t* sorted_assign, int32_t* row_of, int32_t* token_experts,
                             void* ws, size_t ws_bytes, hipStream_t stream);

moe_status moe_routing_stats(const moe_problem* p, const int32_t* counts, const int32_t* kept,
                             const float* P, moe_route_stats* stats, hipStream_t stream);

/*
 * The whole forward: router + top-k, dispatch, experts, combine, aux stats
 * (0539edu page 1.3 and 4.1; kamacoder 二).
 *   x [T, d] dtype in;  y [T, d] float32 out;  out: optional routing outputs.
 */
moe_status moe_ffn_forward(const moe_problem* p, const moe_weights* w, const void* x, float* y,
                           const moe_routing* out, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/*
 * moe_ffn_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same kernels and results, with the workspace taken from a file-scope
 * device array of MOE_STATIC_SCRATCH_BYTES that the library holds on every
 * device it runs on until the process ends (looked up, once per device, on
 * the first call with that device current; the stream must belong to the
 * current device).  Arguments as moe_ffn_forward without ws / ws_bytes.
 * Returns MOE_ERR_WORKSPACE, launching nothing, when the problem's
 * moe_workspace_size exceeds MOE_STATIC_SCRATCH_BYTES.  Allocates nothing.
 * Every call on a device shares that device's array, which keeps the last
 * call's contents (the forward needs none of it cleared): calls that overlap
 * on one device (other streams, other host threads) race.
 */
#define MOE_STATIC_SCRATCH_BYTES (128u << 20)
moe_status moe_ffn_forward_static(const moe_problem* p, const moe_weights* w, const void* x,
                                  float* y, const moe_routing* out, hipStream_t stream);

/*
 * Per-row FP8 E4M3 quantization (0539edu page 5.2: expert parameters in 8
 * bits), a one-time preparation of weights for MOE_W_FP8.  Row r of the
 * [rows, cols] bf16 matrix w gets scale[r] = max_j |w[r, j]| / 448 (1 for an
 * all-zero row) and q[r, j] = the E4M3 code nearest to w[r, j] / scale[r]
 * (float32 division; ties to the even code; magnitudes above 448 saturate).
 * E4M3: bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
 * exponent 0 is subnormal (m/8 * 2^-6); no infinities.  For w_up of shape
 * [E+S, F1, d] pass rows = (E+S)*F1, cols = d; for w_down rows = (E+S)*d,
 * cols = d_ff.  rows < 2^31, cols a multiple of 8.
 */
moe_status moe_quantize_fp8(const void* w, int64_t rows, int32_t cols, uint8_t* q, float* scale,
                            hipStream_t stream);

/*
 * Backward pass of the layer for training: the gradients of
 *     L = <dy, y> + alpha * L_aux
 * (the load-balancing loss added to the task loss before one backward:
 * 0539edu page 4.3; kamacoder 七, total loss), dy being the gradient of the
 * task loss with respect to y.  Top-k selection, capacity drops and the
 * counts f_e are piecewise constant and pass no gradient; a dropped slot
 * sends none to its expert or gate weight; the router receives gradient
 * through the renormalized top-k weights and through P_e.
 *
 * Limits: dtype MOE_BF16 with d_model and d_ff multiples of 64, token-choice
 * routing (no MOE_EXPERT_CHOICE), bf16 expert weights (no MOE_W_FP8);
 * otherwise MOE_ERR_UNSUPPORTED.  Also
 * unsupported when a transposed gradient operand would reach 4 GiB
 * (F1 or d_model times the padded row count, times 2 bytes).
 *
 * The expert activations are recomputed (not stored by the forward).
 *   x, w     the forward's input and weights
 *   dy       [T, d] float32 in
 *   alpha    weight of L_aux in the objective
 *   fwd      routing of the forward pass of the same x and weights (what
 *            moe_ffn_forward wrote into its moe_routing): topk_idx, topk_w,
 *            counts, offsets, sorted_assign, assign_row are required
 *   g        gradient outputs (host struct of device pointers, all float32,
 *            overwritten):
 *              dx        [T, d]               required
 *              dw_router [E, d]               required
 *              db_router [E]                  may be NULL
 *              dw_up     [E+S, F1, d]         required (F1 = 2 d_ff for SwiGLU)
 *              db_up     [E+S, d_ff]          required with MOE_EXPERT_BIAS (not SwiGLU), else ignored
 *              dw_down   [E+S, d, d_ff]       required
 *              db_down   [E+S, d]             as db_up
 *              d_topk_w  [T, k]               may be NULL: gradient of the slot weights (0 if dropped)
 *              d_logits  [T, E]               may be NULL: gradient of the router logits
 *   ws       moe_backward_workspace_size() bytes (256-byte aligned)
 * Deterministic: every sum runs in a fixed order.
 */
typedef struct moe_grads {
  float *dx, *dw_router, *db_router, *dw_up, *db_up, *dw_down, *db_down, *d_topk_w, *d_logits;
} moe_grads;

/* Host only.  Workspace bytes of moe_ffn_backward for this problem. */
moe_status moe_backward_workspace_size(const moe_problem* p, size_t* bytes);

moe_status moe_ffn_backward(const moe_problem* p, const moe_weights* w, const void* x,
                            const float* dy, float alpha, const moe_routing* fwd,
                            const moe_grads* g, void* ws, size_t ws_bytes, hipStream_t stream);

/* Host only.  Process-wide choice of the grouped GEMM's main loop, a tuning
 * and testing control that does not change results (both loops accumulate
 * every output in the same order, so their outputs are bit-identical):
 *   MOE_GEMM_AUTO (default): 16x16x32 MFMAs with 64-deep k-tiles for the
 *     up projection and for long down-style launches (at least 256 GFLOP),
 *     32x32x16 MFMAs with 32-deep k-tiles for shorter ones;
 *   MOE_GEMM_MF32: always the 32x32x16 loop;
 *   MOE_GEMM_MF16: the 16x16x32 loop wherever the reduction allows it (K
 *     slices of whole 64-deep k-tiles; otherwise the 32x32x16 loop).
 * Applies to launches issued after the call; MOE_ERR_INVALID_ARG for any
 * other value. */
#define MOE_GEMM_AUTO 0
#define MOE_GEMM_MF32 1
#define MOE_GEMM_MF16 2
moe_status moe_set_gemm_policy(int32_t policy);

/* Human-readable name of a status code (static string). */
const char* moe_status_string(moe_status s);
/* hipError_t of this thread's last MOE_ERR_HIP (0 if none). */
int32_t moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
