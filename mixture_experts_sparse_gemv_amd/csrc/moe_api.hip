// Host side of the C ABI: argument validation, workspace layout and the
// launch sequence of each entry point.  Nothing here synchronizes with the
// device, reads device memory or allocates.
#include <math.h>
#include <string.h>

#include "moe_internal.h"

namespace moe {

static thread_local int32_t g_last_hip_error = 0;

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

WsLayout ws_layout(const Shape& s) {
  WsLayout w{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  const size_t n = (size_t)s.T * s.k;
  const size_t rows = (size_t)s.max_rows();
  // expert choice: sorted_assign holds the E*cap token ids, assign_row the
  // [T, E] row of each (token, expert) pair, probs the gate probabilities
  const size_t na = s.ec() ? (size_t)s.routed_rows() : n;
  const size_t nr = s.ec() ? (size_t)s.T * s.E : n;
  w.topk_idx = take(n * 4);
  w.topk_w = take(n * 4);
  w.probs = s.ec() ? take((size_t)s.T * s.E * 4) : o;
  w.token_experts = s.ec() ? take((size_t)s.T * 4) : o;
  w.prob_part = take((size_t)router_blocks(s) * s.E * 4);
  w.chunk_counts = take((size_t)router_blocks(s) * s.E * 4);
  w.prob_colsum = take((size_t)s.E * 4);
  w.counts = take((size_t)s.E * 4);
  w.kept = take((size_t)s.E * 4);
  w.offsets = take((size_t)(s.E + 1) * 4);
  w.sorted_assign = take(na * 4);
  w.assign_row = take(nr * 4);
  w.drop_mask = take(n);
  w.f = take((size_t)s.E * 4);
  w.P = take((size_t)s.E * 4);
  w.l_aux = take(4);
  w.h = take(rows * s.f * (s.dtype == MOE_F32 ? 4 : 2));
  w.y_exp = take(rows * s.d * 4);
  const int nparts = down_parts(s);
  w.y_part = nparts > 0 ? take((size_t)nparts * rows * s.d * 4) : o;
  w.total = o;
  return w;
}

BwdLayout bwd_layout(const Shape& s) {
  BwdLayout b{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  const size_t rows = (size_t)s.max_rows();
  const size_t F1 = (size_t)s.up_rows(), nseg = (size_t)(s.E + s.S);
  const size_t ldk = (size_t)wgrad_ldk(s);
  const int ks = bwd_dx_ksplit(s);
  b.dyb = take((size_t)s.T * s.d * 2);
  b.w1t = take(nseg * F1 * s.d * 2);
  b.w2t = take(nseg * s.d * s.f * 2);
  b.Z = take(rows * F1 * 4);
  b.G = take(rows * s.f * 4);
  b.dZ = take(rows * F1 * 2);
  b.dxrows = take(rows * s.d * 4);
  b.dxparts = ks > 1 ? take((size_t)(ks - 1) * rows * s.d * 4) : o;
  b.A2 = take((size_t)s.d * ldk * 2);
  b.B2 = take((size_t)s.f * ldk * 2);
  b.A1 = take(F1 * ldk * 2);
  b.B1 = take((size_t)s.d * ldk * 2);
  b.dwpart = take((size_t)act_backward_parts(s) * (size_t)s.routed_rows() * 4);
  b.dwslot = take((size_t)s.T * s.k * 4);
  b.dlogits = take((size_t)s.T * s.E * 4);
  b.dxr = take((size_t)s.T * s.d * 4);
  b.rw_part = take((size_t)router_wgrad_slices(s) * s.E * s.d * 4);
  b.rb_part = take((size_t)router_wgrad_slices(s) * s.E * 4);
  b.poff = take((nseg + 1) * 4);
  b.logits = take((size_t)s.T * s.E * 4);
  b.prob_part = take((size_t)router_blocks(s) * s.E * 4);
  b.chunk_counts = take((size_t)router_blocks(s) * s.E * 4);
  b.total = o;
  return b;
}

static moe_status fail_hip(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = (int32_t)e;
  return MOE_ERR_HIP;
}

moe_status hip_failure(hipError_t e) { return fail_hip(e); }

// Validate the problem; on success fill `s`.
static moe_status check_problem(const moe_problem* p, Shape& s) {
  if (!p) return MOE_ERR_INVALID_ARG;
  if (p->T <= 0 || p->d_model <= 0 || p->d_ff <= 0 || p->num_experts <= 0 || p->top_k <= 0 ||
      p->top_k > p->num_experts || p->num_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if (p->dtype != MOE_F32 && p->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (p->gating != MOE_SOFTMAX && p->gating != MOE_SIGMOID_NORM) return MOE_ERR_INVALID_ARG;
  if (p->activation < MOE_RELU || p->activation > MOE_SWIGLU) return MOE_ERR_INVALID_ARG;
  if (p->flags & ~(MOE_ROUTER_BIAS | MOE_EXPERT_BIAS | MOE_W_FP8 | MOE_EXPERT_CHOICE))
    return MOE_ERR_INVALID_ARG;
  if (p->flags & MOE_EXPERT_CHOICE) {   // every expert takes exactly `capacity` tokens
    if (p->capacity < 1 || p->capacity > p->T) return MOE_ERR_INVALID_ARG;
    if (p->T > kEcMaxT || (long long)p->num_experts * p->capacity >= (1LL << 31))
      return MOE_ERR_UNSUPPORTED;
  }
  if (p->num_experts > kMaxExperts || p->top_k > kMaxTopK ||
      p->num_experts + p->num_shared > kMaxSegments)
    return MOE_ERR_UNSUPPORTED;
  const long long routed = (p->flags & MOE_EXPERT_CHOICE)
                               ? (long long)p->num_experts * p->capacity
                               : (long long)p->T * p->top_k;
  const long long rows = routed + (long long)p->T * p->num_shared;
  if (rows >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if ((long long)rows * p->d_ff >= (1LL << 40) || (long long)rows * p->d_model >= (1LL << 40))
    return MOE_ERR_UNSUPPORTED;
  if (p->dtype == MOE_BF16 && (p->d_model % 8 != 0 || p->d_ff % 8 != 0))
    return MOE_ERR_UNSUPPORTED;
  if (p->flags & MOE_W_FP8) {   // FP8 expert weights: the weight-streaming decode path only
    if (p->dtype != MOE_BF16 || p->T > kDecodeMaxT || p->d_model % 128 != 0 || p->d_ff % 128 != 0)
      return MOE_ERR_UNSUPPORTED;
  }
  // one expert's weight matrix must stay below 4 GiB (32-bit offsets in the kernels)
  const long long f1 = p->activation == MOE_SWIGLU ? 2LL * p->d_ff : p->d_ff;
  if (f1 * p->d_model * 4 >= (1LL << 32)) return MOE_ERR_UNSUPPORTED;
  // the grouped GEMM addresses token rows of x, and one segment's rows of h,
  // with 32-bit byte offsets
  if (p->dtype == MOE_BF16 && ((long long)p->T * p->d_model * 2 >= (1LL << 32) ||
                               (long long)p->T * p->d_ff * 2 >= (1LL << 32)))
    return MOE_ERR_UNSUPPORTED;
  s.T = p->T;
  s.d = p->d_model;
  s.f = p->d_ff;
  s.E = p->num_experts;
  s.k = p->top_k;
  s.S = p->num_shared;
  s.cap = p->capacity > 0 ? p->capacity : 0;
  s.dtype = p->dtype;
  s.gating = p->gating;
  s.act = p->activation;
  s.flags = p->flags;
  return MOE_OK;
}

static moe_status check_ws(const Shape& s, const void* ws, size_t ws_bytes, WsLayout& L) {
  L = ws_layout(s);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)ws & 255) != 0) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

static moe_status check_weights(const Shape& s, const moe_weights* w, bool router, bool experts) {
  if (!w) return MOE_ERR_INVALID_ARG;
  if (router && (!w->w_router || (s.router_bias() && !w->b_router))) return MOE_ERR_INVALID_ARG;
  if (experts && (!w->w_up || !w->w_down)) return MOE_ERR_INVALID_ARG;
  if (experts && s.expert_bias() && (!w->b_up || !w->b_down)) return MOE_ERR_INVALID_ARG;
  if (experts && s.w_fp8() && (!w->s_up || !w->s_down)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

template <class T>
static T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

}  // namespace moe

using namespace moe;

extern "C" {

int32_t moe_capacity(int32_t T, int32_t k, int32_t E, float capacity_factor) {
  if (T <= 0 || k <= 0 || E <= 0) return -1;
  if (!(capacity_factor > 0.0f)) return 0;
  const double c = ceil((double)capacity_factor * (double)T * (double)k / (double)E);
  return c >= 2147483647.0 ? 2147483647 : (int32_t)c;
}

moe_status moe_workspace_size(const moe_problem* p, size_t* bytes) {
  Shape s;
  moe_status st = check_problem(p, s);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = ws_layout(s).total;
  return MOE_OK;
}

moe_status moe_router_topk(const moe_problem* p, const void* x, const moe_weights* w,
                           int32_t* topk_idx, float* topk_w, float* probs, float* prob_colsum,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  WsLayout L;
  moe_status st = check_problem(p, s);
  if (st != MOE_OK) return st;
  if ((st = check_weights(s, w, true, false)) != MOE_OK) return st;
  if (!x) return MOE_ERR_INVALID_ARG;
  if (s.ec() ? !probs : (!topk_idx || !topk_w)) return MOE_ERR_INVALID_ARG;
  if (s.ec()) topk_idx = nullptr, topk_w = nullptr;   // expert choice uses the probabilities only
  if ((st = check_ws(s, ws, ws_bytes, L)) != MOE_OK) return st;
  float* part = at<float>(ws, L.prob_part);
  hipError_t e = launch_router(s, x, w->w_router, w->b_router, topk_idx, topk_w, probs, part,
                               at<int32_t>(ws, L.chunk_counts), stream);
  if (e == hipSuccess && prob_colsum) e = launch_colsum(s, part, prob_colsum, stream);
  return fail_hip(e);
}

moe_status moe_dispatch(const moe_problem* p, const int32_t* topk_idx, int32_t* counts,
                        int32_t* kept, int32_t* offsets, int32_t* sorted_assign,
                        int32_t* assign_row, uint8_t* drop_mask, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  Shape s;
  WsLayout L;
  moe_status st = check_problem(p, s);
  if (st != MOE_OK) return st;
  if (s.ec()) return MOE_ERR_INVALID_ARG;   // expert choice dispatches with moe_expert_choice
  if (!topk_idx || !counts || !kept || !offsets || !sorted_assign || !assign_row || !drop_mask)
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, ws, ws_bytes, L)) != MOE_OK) return st;
  return fail_hip(launch_dispatch(s, topk_idx, at<int32_t>(ws, L.chunk_counts), false, counts,
                                  kept, offsets,
                                  sorted_assign, assign_row, drop_mask, nullptr, nullptr, nullptr,
                                  nullptr, nullptr, nullptr, stream));
}

moe_status moe_expert_up(const moe_problem* p, const void* x, const moe_weights* w,
                         const int32_t* offsets, const int32_t* sorted_assign, void* h, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  Shape s;
  WsLayout L;
  moe_status st = check_problem(p, s);
  if (st != MOE_OK) return st;
  if ((st = check_weights(s, w, false, true)) != MOE_OK) return st;
  if (!x || !offsets || !sorted_assign || !h) return MOE_ERR_INVALID_ARG;
  (void)ws;  // the up projection needs no scratch
  (void)ws_bytes;
  (void)L;
  return fail_hip(launch_up(s, x, w->w_up, w->b_up, w->s_up, offsets, sorted_assign, h, stream));
}

moe_status moe_expert_down(const moe_problem* p, const moe_weights* w, const int32_t* offsets,
                           const void* h, float* y_exp, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  Shape s;
  WsLayout L;
  moe_status st = check_problem(p, s);
  if (st != MOE_OK) return st;
  if ((st = check_weights(s, w, false, true)) != MOE_OK) return st;
  if (!offsets || !h || !y_exp) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, ws, ws_bytes, L)) != MOE_OK) return st;
  return fail_hip(launch_down(s, h, w->w_down, w->b_down, w->s_down, offsets, y_exp,
                              at<float>(ws, L.y_part), true, stream));
}

moe_status moe_expert_ffn(const moe_problem* p, const void* x, const moe_weights* w,
                          const int32_t* offsets, const int32_t* sorted_assign, float* y_exp,
                          void* ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  WsLayout L;
  moe_status st = check_problem(p, s);
  if (st != MOE_OK) return st;
  if ((st = check_weights(s, w, false, true)) != MOE_OK) return st;
  if (!x || !offsets || !sorted_assign || !y_exp) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, ws, ws_bytes, L)) != MOE_OK) return st;
  void* h = at<void>(ws, L.h);
  hipError_t e = launch_up(s, x, w->w_up, w->b_up, w->s_up, offsets, sorted_assign, h, stream);
  if (e == hipSuccess)
    e = launch_down(s, h, w->w_down, w->b_down, w->s_down, offsets, y_exp, at<float>(ws, L.y_part), true,
                    stream);
  return fail_hip(e);
}

moe_status moe_combine(const moe_problem* p, const float* topk_w, const int32_t* assign_row,
                       const int32_t* offsets, const float* y_exp, float* y, hipStream_t stream) {
  Shape s;
  moe_status st = check_problem(p, s);
  if (st != MOE_OK) return st;
  if (!topk_w || !assign_row || !offsets || !y_exp || !y) return MOE_ERR_INVALID_ARG;
  if (s.ec())   // topk_w = probs [T, E], assign_row = row of each (token, expert) [T, E]
    return fail_hip(launch_combine_ec(s, topk_w, assign_row, offsets, y_exp, nullptr, 0, y, stream));
  return fail_hip(launch_combine(s, topk_w, assign_row, offsets, y_exp, nullptr, 0, y, stream));
}

moe_status moe_aux_stats(const moe_problem* p, const float* prob_colsum, const int32_t* counts,
                         float* f, float* P, float* l_aux, hipStream_t stream) {
  Shape s;
  moe_status st = check_problem(p, s);
  if (st != MOE_OK) return st;
  if (!prob_colsum || !counts || !f || !P || !l_aux) return MOE_ERR_INVALID_ARG;
  return fail_hip(launch_aux(s, prob_colsum, counts, f, P, l_aux, stream));
}

moe_status moe_expert_choice(const moe_problem* p, const float* probs, int32_t* offsets,
                             int32_t* sorted_assign, int32_t* row_of, int32_t* token_experts,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  WsLayout L;
  moe_status st = check_problem(p, s);
  if (st != MOE_OK) return st;
  if (!s.ec()) return MOE_ERR_INVALID_ARG;
  if (!probs || !offsets || !sorted_assign || !row_of) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, ws, ws_bytes, L)) != MOE_OK) return st;
  hipError_t e = launch_expert_choice(s, probs, sorted_assign, row_of, at<int32_t>(ws, L.counts),
                                      at<int32_t>(ws, L.kept), offsets, nullptr, stream);
  if (e == hipSuccess && token_experts) e = launch_token_experts(s, row_of, token_experts, stream);
  return fail_hip(e);
}

moe_status moe_routing_stats(const moe_problem* p, const int32_t* counts, const int32_t* kept,
                             const float* P, moe_route_stats* stats, hipStream_t stream) {
  Shape s;
  moe_status st = check_problem(p, s);
  if (st != MOE_OK) return st;
  if (!counts || !kept || !P || !stats) return MOE_ERR_INVALID_ARG;
  return fail_hip(launch_routing_stats(s, counts, kept, P, stats, stream));
}

moe_status moe_quantize_fp8(const void* w, int64_t rows, int32_t cols, uint8_t* q, float* scale,
                            hipStream_t stream) {
  if (!w || !q || !scale || rows <= 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
  if (rows >= (1LL << 31) || cols % 8 != 0) return MOE_ERR_UNSUPPORTED;
  return fail_hip(launch_quantize_fp8(w, rows, cols, q, scale, stream));
}

moe_status moe_ffn_forward(const moe_problem* p, const moe_weights* w, const void* x, float* y,
                           const moe_routing* out, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  Shape s;
  WsLayout L;
  moe_status st = check_problem(p, s);
  if (st != MOE_OK) return st;
  if ((st = check_weights(s, w, true, true)) != MOE_OK) return st;
  if (!x || !y) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, ws, ws_bytes, L)) != MOE_OK) return st;
  moe_routing r{};
  if (out) r = *out;
  int32_t* topk_idx = r.topk_idx ? r.topk_idx : at<int32_t>(ws, L.topk_idx);
  float* topk_w = r.topk_w ? r.topk_w : at<float>(ws, L.topk_w);
  int32_t* counts = r.counts ? r.counts : at<int32_t>(ws, L.counts);
  int32_t* kept = r.kept ? r.kept : at<int32_t>(ws, L.kept);
  int32_t* offsets = r.offsets ? r.offsets : at<int32_t>(ws, L.offsets);
  int32_t* sorted_assign = r.sorted_assign ? r.sorted_assign : at<int32_t>(ws, L.sorted_assign);
  int32_t* assign_row = r.assign_row ? r.assign_row : at<int32_t>(ws, L.assign_row);
  uint8_t* drop_mask = r.drop_mask ? r.drop_mask : at<uint8_t>(ws, L.drop_mask);
  float* f = r.f ? r.f : at<float>(ws, L.f);
  float* P = r.P ? r.P : at<float>(ws, L.P);
  float* l_aux = r.l_aux ? r.l_aux : at<float>(ws, L.l_aux);
  float* part = at<float>(ws, L.prob_part);
  void* h = at<void>(ws, L.h);
  float* y_exp = at<float>(ws, L.y_exp);

  int32_t* chunk_counts = at<int32_t>(ws, L.chunk_counts);
  hipError_t e;
  if (s.ec()) {
    // expert choice: probabilities -> each expert's top-cap tokens -> f, P, L_aux
    float* probs = r.probs ? r.probs : at<float>(ws, L.probs);
    float* colsum = at<float>(ws, L.prob_colsum);
    e = launch_router(s, x, w->w_router, w->b_router, nullptr, nullptr, probs, part, chunk_counts,
                      stream);
    if (e == hipSuccess)
      e = launch_expert_choice(s, probs, sorted_assign, assign_row, counts, kept, offsets, colsum,
                               stream);
    if (e == hipSuccess) e = launch_aux(s, colsum, counts, f, P, l_aux, stream);
    if (e == hipSuccess && r.token_experts)
      e = launch_token_experts(s, assign_row, r.token_experts, stream);
    if (e == hipSuccess && r.stats) e = launch_routing_stats(s, counts, kept, P, r.stats, stream);
    topk_w = probs;   // the combine weights
  } else {
    e = launch_router(s, x, w->w_router, w->b_router, topk_idx, topk_w, r.probs, part,
                      chunk_counts, stream);
    if (e == hipSuccess)
      e = launch_dispatch(s, topk_idx, chunk_counts, true, counts,
                          kept, offsets, sorted_assign, assign_row, drop_mask, part,
                          at<float>(ws, L.prob_colsum), f, P, l_aux, r.stats, stream);
  }
  if (e == hipSuccess)
    e = launch_up(s, x, w->w_up, w->b_up, w->s_up, offsets, sorted_assign, h, stream);
  // The down projection's K slices (if any) are summed by the combine.
  float* y_part = at<float>(ws, L.y_part);
  const int nparts = down_parts(s);
  if (e == hipSuccess)
    e = launch_down(s, h, w->w_down, w->b_down, w->s_down, offsets, y_exp, y_part, nparts == 0, stream);
  if (e == hipSuccess)
    e = s.ec() ? launch_combine_ec(s, topk_w, assign_row, offsets, y_exp, y_part, nparts, y, stream)
               : launch_combine(s, topk_w, assign_row, offsets, y_exp, y_part, nparts, y, stream);
  return fail_hip(e);
}

// Backward limits beyond check_problem's.
static moe_status check_backward(const Shape& s) {
  if (s.dtype != MOE_BF16 || s.ec() || s.w_fp8()) return MOE_ERR_UNSUPPORTED;
  if (s.d % 64 != 0 || s.f % 64 != 0) return MOE_ERR_UNSUPPORTED;   // tiled kernels only
  const long long ldk = wgrad_ldk(s);
  // transposed operands [F1 or d, ldk] bf16 are addressed with 32-bit offsets
  if ((long long)s.up_rows() * ldk * 2 >= (1LL << 32) || (long long)s.d * ldk * 2 >= (1LL << 32) ||
      (long long)s.f * ldk * 2 >= (1LL << 32))
    return MOE_ERR_UNSUPPORTED;
  // token rows (x, dy) and the largest row segment are addressed likewise
  if ((long long)s.T * s.d * 4 >= (1LL << 32) || s.max_rows() * (long long)s.up_rows() * 2 >= (1LL << 32))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status moe_backward_workspace_size(const moe_problem* p, size_t* bytes) {
  Shape s;
  moe_status st = check_problem(p, s);
  if (st != MOE_OK) return st;
  if ((st = check_backward(s)) != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  *bytes = bwd_layout(s).total;
  return MOE_OK;
}

moe_status moe_ffn_backward(const moe_problem* p, const moe_weights* w, const void* x,
                            const float* dy, float alpha, const moe_routing* fwd,
                            const moe_grads* g, void* ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  moe_status st = check_problem(p, s);
  if (st != MOE_OK) return st;
  if ((st = check_backward(s)) != MOE_OK) return st;
  if ((st = check_weights(s, w, true, true)) != MOE_OK) return st;
  if (!x || !dy || !fwd || !g || !isfinite(alpha)) return MOE_ERR_INVALID_ARG;
  if (!fwd->topk_idx || !fwd->topk_w || !fwd->counts || !fwd->offsets || !fwd->sorted_assign ||
      !fwd->assign_row)
    return MOE_ERR_INVALID_ARG;
  if (!g->dx || !g->dw_router || !g->dw_up || !g->dw_down) return MOE_ERR_INVALID_ARG;
  if (s.expert_bias() && (!g->db_up || !g->db_down)) return MOE_ERR_INVALID_ARG;
  const BwdLayout B = bwd_layout(s);
  if (!ws || ws_bytes < B.total) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)ws & 255) != 0) return MOE_ERR_INVALID_ARG;

  const int F1 = s.up_rows(), nseg = s.E + s.S, ldk = wgrad_ldk(s);
  const int ks = bwd_dx_ksplit(s);
  const long long part_elems = s.max_rows() * s.d;
  const int32_t* offsets = fwd->offsets;
  const int32_t* sa = fwd->sorted_assign;
  const float* topk_w = fwd->topk_w;
  uint16_t* dyb = at<uint16_t>(ws, B.dyb);
  uint16_t* w1t = at<uint16_t>(ws, B.w1t);
  uint16_t* w2t = at<uint16_t>(ws, B.w2t);
  float* Z = at<float>(ws, B.Z);
  float* G = at<float>(ws, B.G);
  uint16_t* dZ = at<uint16_t>(ws, B.dZ);
  float* dxrows = at<float>(ws, B.dxrows);
  float* dxparts = at<float>(ws, B.dxparts);
  uint16_t* A2 = at<uint16_t>(ws, B.A2);
  uint16_t* B2 = at<uint16_t>(ws, B.B2);
  uint16_t* A1 = at<uint16_t>(ws, B.A1);
  uint16_t* B1 = at<uint16_t>(ws, B.B1);
  float* dwpart = at<float>(ws, B.dwpart);
  float* dwslot = at<float>(ws, B.dwslot);
  float* dlogits = g->d_logits ? g->d_logits : at<float>(ws, B.dlogits);
  float* dxr = at<float>(ws, B.dxr);
  int32_t* poff = at<int32_t>(ws, B.poff);
  const void* b_up = s.expert_bias() ? w->b_up : nullptr;
  const void* b_down = s.expert_bias() ? w->b_down : nullptr;

  // operands in the layouts the grouped GEMM reads: bf16 dy, W1^T and W2^T
  hipError_t e = launch_cast_bf16(dy, dyb, (long long)s.T * s.d, stream);
  if (e == hipSuccess) e = launch_transpose(w->w_up, w1t, nseg, F1, s.d, stream);
  if (e == hipSuccess) e = launch_transpose(w->w_down, w2t, nseg, s.d, s.f, stream);
  // recomputed pre-activations, and G = dy_rows W2
  if (e == hipSuccess)
    e = launch_bwd_lin(s, x, w->w_up, b_up, F1, s.d, Z, offsets, sa, stream);
  if (e == hipSuccess) e = launch_bwd_lin(s, dyb, w2t, nullptr, s.f, s.d, G, offsets, sa, stream);
  // the weight gradients' transposed operands are zero-padded per segment
  if (e == hipSuccess) e = launch_wgrad_offsets(s, offsets, poff, stream);
  // h, dZ (row-major, and transposed into A1), h^T into B2, and the column
  // partials of the gate weights' gradient
  if (e == hipSuccess)
    e = launch_act_backward(s, Z, G, dy, b_down, offsets, sa, topk_w, poff, fwd->assign_row,
                            fwd->topk_idx, ldk, dZ, A1, B2, dwpart, dwslot, stream);
  // dX rows = dZ W1
  if (e == hipSuccess)
    e = launch_bwd_dx(s, dZ, w1t, F1, s.d, dxrows, dxparts, part_elems, ks, offsets, stream);
  if (e == hipSuccess)
    e = launch_seg_transpose(s, 0, dy, s.d, offsets, sa, topk_w, poff, A2, ldk, stream);
  if (e == hipSuccess)
    e = launch_seg_transpose(s, 1, x, s.d, offsets, sa, topk_w, poff, B1, ldk, stream);
  if (e == hipSuccess) e = launch_bwd_wgrad(s, A2, B2, s.d, s.f, ldk, g->dw_down, offsets, stream);
  if (e == hipSuccess) e = launch_bwd_wgrad(s, A1, B1, F1, s.d, ldk, g->dw_up, offsets, stream);
  if (e == hipSuccess && s.expert_bias()) e = launch_seg_rowsum(s, A2, s.d, ldk, poff, g->db_down, stream);
  if (e == hipSuccess && s.expert_bias()) e = launch_seg_rowsum(s, A1, F1, ldk, poff, g->db_up, stream);
  // router: the logits again (router kernel, no top-k output), then its backward
  float* logits = at<float>(ws, B.logits);
  if (e == hipSuccess)
    e = launch_router(s, x, w->w_router, w->b_router, nullptr, nullptr, nullptr,
                      at<float>(ws, B.prob_part), at<int32_t>(ws, B.chunk_counts), stream, logits);
  if (e == hipSuccess)
    e = launch_router_backward(s, logits, w->w_router, fwd->topk_idx, fwd->assign_row, dwslot,
                               fwd->counts, alpha, dlogits, g->d_topk_w, dxr, stream);
  if (e == hipSuccess)
    e = launch_router_wgrad(s, dlogits, x, at<float>(ws, B.rw_part), at<float>(ws, B.rb_part),
                            g->dw_router, g->db_router, stream);
  // dx = router part + the rows of every kept slot and shared expert
  if (e == hipSuccess)
    e = launch_dx_gather(s, dxr, dxrows, dxparts, ks - 1, part_elems, fwd->assign_row, offsets,
                         g->dx, stream);
  return fail_hip(e);
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

int32_t moe_last_hip_error(void) { return g_last_hip_error; }

moe_status moe_set_gemm_policy(int32_t policy) {
  if (policy != MOE_GEMM_AUTO && policy != MOE_GEMM_MF32 && policy != MOE_GEMM_MF16)
    return MOE_ERR_INVALID_ARG;
  moe::set_gemm_policy(policy);
  return MOE_OK;
}

}  // extern "C"
