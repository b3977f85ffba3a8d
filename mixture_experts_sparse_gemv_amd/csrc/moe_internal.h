// Internal declarations of libmoe_mi355x: problem shape, workspace layout,
// device helpers and the host-side launchers each kernel file provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------- limits
constexpr int kMaxExperts = 64;       // routed experts: one wave lane per expert
constexpr int kMaxTopK = 8;
constexpr int kMaxSegments = 128;     // routed + shared experts
// T at or below which the streaming decode path runs.  Its kernels carry up
// to 4 groups of 16 token rows per weight stage; a segment with more rows
// (above T = 64) streams its weights once per 64 rows.  Measured on the
// large-expert shape (d_model 4096, SwiGLU 14336, 8 experts, top-2), ms per
// forward, decode path vs 256-row grouped GEMM tiles: T = 24: 0.47 vs 0.66,
// 32: 0.47 vs 0.67, 48: 0.54 vs 0.67, 64: 0.56 vs 0.68, 128 by the GEMM 0.69.
#ifndef MOE_DECODE_MAX_T
#define MOE_DECODE_MAX_T 128
#endif
constexpr int kDecodeMaxT = MOE_DECODE_MAX_T;
static_assert(kDecodeMaxT >= 1 && kDecodeMaxT <= 128, "streaming path bound");
constexpr int kEcMaxT = 16384;        // expert-choice selection keeps a column of T scores in LDS
constexpr int kNumCUs = 256;          // MI355X compute units (sizes the K split of small GEMMs)

// ---------------------------------------------------------------- shape
struct Shape {
  int T, d, f, E, k, S, cap;   // cap <= 0: unlimited
  int dtype, gating, act, flags;
  int up_rows() const { return act == MOE_SWIGLU ? 2 * f : f; }
  // expert-choice routing: every expert takes exactly cap tokens
  bool ec() const { return flags & MOE_EXPERT_CHOICE; }
  // rows of the routed experts' segments, and what a sorted_assign entry is
  // divided by to give its token (assignment ids t*k+s; token ids for ec)
  long long routed_rows() const { return ec() ? (long long)E * cap : (long long)T * k; }
  int tok_div() const { return ec() ? 1 : k; }
  long long max_rows() const { return routed_rows() + (long long)S * T; }
  bool router_bias() const { return flags & MOE_ROUTER_BIAS; }
  bool expert_bias() const { return (flags & MOE_EXPERT_BIAS) && act != MOE_SWIGLU; }
  // bf16 widths that are multiples of 8 but not of 64: the untiled grouped
  // GEMM (csrc/gemm_generic.hip) instead of the tiled and streaming kernels
  bool generic() const { return dtype == MOE_BF16 && (d % 64 != 0 || f % 64 != 0); }
  bool decode() const { return dtype == MOE_BF16 && T <= kDecodeMaxT && !generic(); }
  bool w_fp8() const { return flags & MOE_W_FP8; }
};

// Router blocks each handle this many tokens (their per-expert probability
// sums are the partial sums later reduced in block order).
constexpr int kRouterTokens = 16;
inline int router_blocks(const Shape& s) { return (s.T + kRouterTokens - 1) / kRouterTokens; }
// Dispatch scatter blocks each rank the assignments of this many tokens
// (a multiple of kRouterTokens: the per-chunk expert counts are summed per
// scatter block).
constexpr int kScatterTokens = 512;
inline int scatter_blocks(const Shape& s) { return (s.T + kScatterTokens - 1) / kScatterTokens; }

// Split of the reduction dimension in the decode down-projection (bf16 and
// FP8 weights: FP8 stages hold twice the K elements, and 8 slices measured
// 2% faster than 4 on the 8-expert d = 4096, f = 14336 layer; 16 slower).
constexpr int kDecodeSplitK = 4, kDecodeSplitK8 = 8;

// K slices of the (non-decode) down projection: 1, 2 or 4.  More than one
// when its expected tile count would leave most compute units idle; slice 0
// is written to y_exp, slice i > 0 to y_part + (i - 1) * max_rows * d, and
// the slices are summed in slice order (by the combine, or by a fold pass).
int down_ksplit(const Shape& s);
// The grouped GEMM's main-loop choice (MOE_GEMM_AUTO / _MF32 / _MF16).
void set_gemm_policy(int policy);
// K slices of the decode down projection (slice 0 into y_exp with the bias,
// slice i > 0 into y_part + (i - 1) * max_rows * d_model).
int decode_nsplit(const Shape& s);
// Partial slices of the down projection that y_part holds for the combine
// when launch_down runs with complete = false.
int down_parts(const Shape& s);

// ---------------------------------------------------------------- workspace
struct WsLayout {
  size_t topk_idx, topk_w, probs, token_experts, prob_part, chunk_counts, prob_colsum, counts, kept, offsets, sorted_assign,
      assign_row, drop_mask, f, P, l_aux, h, y_exp, y_part, total;
};
WsLayout ws_layout(const Shape& s);
// MOE_OK for hipSuccess; otherwise records e as the thread's last HIP error
// (moe_last_hip_error) and returns MOE_ERR_HIP.
moe_status hip_failure(hipError_t e);

// ---------------------------------------------------------------- vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(((uint32_t)u) << 16);
}

// The intermediate h of bf16 problems is stored in fp16 scaled by 2^-8 (the
// down projection multiplies its fp32 sums by 2^8, exactly).  fp16 keeps 11
// significant bits for |h| >= 2^-6 and an absolute step of 2^-16 below, and
// the scale moves its overflow from 65504 to 65504 * 2^8 ~ 1.68e7.  Larger
// magnitudes saturate to +-65504 * 2^8 (never inf); NaN stays NaN.
constexpr float kHStoreScale = 0.00390625f;   // 2^-8
constexpr float kHLoadScale = 256.0f;         // 2^8
__device__ __forceinline__ _Float16 h_to_f16(float v) {
  v *= kHStoreScale;
  v = fabsf(v) > 65504.0f ? copysignf(65504.0f, v) : v;
  return (_Float16)v;
}

// Eight bf16 values (16 bytes) -> eight fp16 values.  bf16 -> fp32 is exact
// (a shift); fp32 -> fp16 is exact for magnitudes in [2^-14, 65504], which is
// where bf16 weights of a trained or N(0, 0.02^2) layer lie; smaller values
// become fp16 subnormals (truncated), larger ones saturate.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo = __uint_as_float(v[i] << 16);
    float hi = __uint_as_float(v[i] & 0xffff0000u);
    fp16x2_t p = __builtin_amdgcn_cvt_pkrtz(lo, hi);
    r[i] = __builtin_bit_cast(uint32_t, p);
  }
  return r;
}

// Wave-wide reductions without the LDS crossbar: four DPP steps inside each
// row of 16 lanes (quad swaps across 1 and 2 lanes, then the half-row and
// row mirrors, after which every lane of a row holds the row's result), then
// the four row results read as scalars and combined in a fixed order.  Every
// lane returns the result.  Call with the whole wave active.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f(float v, int l) {   // l uniform
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

// exp(x) through the hardware base-2 exponential.
__device__ __forceinline__ float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// silu(z) = z / (1 + exp(-z)).
__device__ __forceinline__ float silu_f(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + fast_exp(-z));
}

// GELU in the exact erf form, 0.5 z (1 + erf(z / sqrt 2)), with erf from
// Abramowitz & Stegun, Handbook of Mathematical Functions, 7.1.28: for u >= 0,
// erf(u) = 1 - (1 + a1 u + a2 u^2 + ... + a6 u^6)^-16, absolute error at most
// 3e-7 (no exponential: six fma, four squarings, one reciprocal; the power
// overflows to inf for large u, where the reciprocal gives erf = 1).  With
// r = 1 - erf(|z|/sqrt 2): GELU(z) = z - z r / 2 for z >= 0, z r / 2 below.
__device__ __forceinline__ float gelu_f(float z) {
  const float u = fabsf(z) * 0.70710678118654752f;
  float p = fmaf(4.30638e-5f, u, 2.765672e-4f);
  p = fmaf(p, u, 1.520143e-4f);
  p = fmaf(p, u, 9.2705272e-3f);
  p = fmaf(p, u, 4.22820123e-2f);
  p = fmaf(p, u, 7.05230784e-2f);
  p = fmaf(p, u, 1.0f);
  p *= p;
  p *= p;
  p *= p;
  p *= p;
  const float r = __builtin_amdgcn_rcpf(p);
  const float hz = 0.5f * z;
  return z >= 0.0f ? fmaf(-hz, r, z) : hz * r;
}

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; all are asynchronous on `st`.
// Also writes each 16-token chunk's per-expert sum of probabilities
// (prob_part) and count of selections (chunk_counts), both [chunks, E], and,
// when `logits` is non-null, the logits (with bias) [T, E].  topk_idx null:
// no top-k output.
hipError_t launch_router(const Shape& s, const void* x, const void* wr, const void* br,
                         int32_t* topk_idx, float* topk_w, float* probs, float* prob_part,
                         int32_t* chunk_counts, hipStream_t st, float* logits = nullptr);
hipError_t launch_colsum(const Shape& s, const float* prob_part, float* colsum, hipStream_t st);
// Dispatch.  counted: chunk_counts already hold the router's per-chunk
// counts (else they are computed from topk_idx first).  When prob_part is
// non-null it also reduces the probability sums into colsum and writes f, P,
// l_aux (and the routing health indicators when stats is non-null).
hipError_t launch_dispatch(const Shape& s, const int32_t* topk_idx, int32_t* chunk_counts,
                           bool counted, int32_t* counts, int32_t* kept, int32_t* offsets,
                           int32_t* sorted_assign, int32_t* assign_row, uint8_t* drop_mask,
                           const float* prob_part, float* colsum, float* f, float* P,
                           float* l_aux, moe_route_stats* stats, hipStream_t st);
hipError_t launch_routing_stats(const Shape& s, const int32_t* counts, const int32_t* kept,
                                const float* P, moe_route_stats* stats, hipStream_t st);
hipError_t launch_aux(const Shape& s, const float* colsum, const int32_t* counts, float* f,
                      float* P, float* l_aux, hipStream_t st);
// Expert choice: each expert's top-cap tokens by probs[:, e] (ties to the lower
// token), in ascending token order: sorted_assign[e*cap + i] = token,
// row_of[t*E + e] = row or -1; counts = kept = cap, offsets[e] = e*cap; colsum
// = column sums of probs (fixed order).  token_experts[t] = experts that took t.
hipError_t launch_expert_choice(const Shape& s, const float* probs, int32_t* sorted_assign,
                                int32_t* row_of, int32_t* counts, int32_t* kept,
                                int32_t* offsets, float* colsum, hipStream_t st);
hipError_t launch_token_experts(const Shape& s, const int32_t* row_of, int32_t* token_experts,
                                hipStream_t st);
// y[t] = sum over experts e with row_of[t*E+e] >= 0 of probs[t*E+e] * y_exp row + shared rows.
hipError_t launch_combine_ec(const Shape& s, const float* probs, const int32_t* row_of,
                             const int32_t* offsets, const float* y_exp, const float* y_part,
                             int nparts, float* y, hipStream_t st);
// s_up / s_down: FP8 row scales (MOE_W_FP8), else ignored.
hipError_t launch_up(const Shape& s, const void* x, const void* w_up, const void* b_up,
                     const float* s_up, const int32_t* offsets, const int32_t* sorted_assign,
                     void* h, hipStream_t st);
// complete = true: y_exp holds the whole result on return (K slices folded);
// false: slices 1.. stay in y_part for the combine to add (down_parts(s) of
// them).
hipError_t launch_down(const Shape& s, const void* h, const void* w_down, const void* b_down,
                       const float* s_down, const int32_t* offsets, float* y_exp, float* y_part,
                       bool complete, hipStream_t st);
hipError_t launch_up_generic(const Shape& s, const void* x, const void* w_up, const void* b_up,
                             const int32_t* offsets, const int32_t* sorted_assign, void* h,
                             hipStream_t st);
hipError_t launch_down_generic(const Shape& s, const void* h, const void* w_down,
                               const void* b_down, const int32_t* offsets, float* y_exp,
                               hipStream_t st);
// y_part/nparts: K-slice partials of y_exp still to be added (nparts = 0: none).
hipError_t launch_quantize_fp8(const void* w, long long rows, int cols, uint8_t* q, float* scales,
                               hipStream_t st);
hipError_t launch_combine(const Shape& s, const float* topk_w, const int32_t* assign_row,
                          const int32_t* offsets, const float* y_exp, const float* y_part,
                          int nparts, float* y, hipStream_t st);

// ---------------------------------------------------------------- backward
// K slices of the dX GEMM (reduction over F1, d outputs), as down_ksplit.
int bwd_dx_ksplit(const Shape& s);
// Weight-gradient layout: segment seg's rows occupy columns poff .. poff+pad
// of the transposed operands, pad = rows rounded up to a multiple of 64 (at
// least 64; the padding is zero), so every segment has a whole, non-empty
// number of 64-deep (and 32-deep) k-tiles.
__host__ __device__ __forceinline__ int wgrad_pad(int rows) {
  return rows <= 0 ? 64 : (rows + 63) / 64 * 64;
}
// Row stride of the transposed weight-gradient operands: every segment's
// padded rows fit.
inline int wgrad_ldk(const Shape& s) {
  return (int)(((s.max_rows() + 63) / 64) * 64 + 64LL * (s.E + s.S));
}
int router_wgrad_slices(const Shape& s);
struct BwdLayout {
  size_t dyb, w1t, w2t, Z, G, dZ, dxrows, dxparts, A2, B2, A1, B1, dwpart, dwslot, dlogits, dxr,
      rw_part, rb_part, poff, logits, prob_part, chunk_counts, total;
};
BwdLayout bwd_layout(const Shape& s);

hipError_t launch_cast_bf16(const float* src, uint16_t* dst, long long n, hipStream_t st);
// dst[m] = src[m]^T for nmat bf16 matrices of R x C (multiples of 64).
hipError_t launch_transpose(const void* src, void* dst, int nmat, int R, int C, hipStream_t st);
hipError_t launch_bwd_lin(const Shape& s, const void* X, const void* W, const void* bias,
                          int Wrows, int K, float* out, const int32_t* offsets,
                          const int32_t* sorted_assign, hipStream_t st);
hipError_t launch_bwd_dx(const Shape& s, const void* X, const void* W, int K, int N, float* out,
                         float* out2, long long part_elems, int ksplit, const int32_t* offsets,
                         hipStream_t st);
hipError_t launch_bwd_wgrad(const Shape& s, const void* A, const void* B, int M, int N, int ldk,
                            float* out, const int32_t* offsets, hipStream_t st);
// h, dZ and the transposed weight-gradient operands (A1 = dZ^T, B2 = h^T,
// [F1 or f][ldk], zero-padded per segment as poff says), and the slot
// weights' gradient dwslot[a] = <h, G> + <b2_e, dy_t> (0 if dropped), summed
// from per-row column partials dwpart [T*k][act_backward_parts(s)].
hipError_t launch_act_backward(const Shape& s, const float* Z, const float* G, const float* dy,
                               const void* b_down, const int32_t* offsets,
                               const int32_t* sorted_assign, const float* topk_w,
                               const int32_t* poff, const int32_t* assign_row,
                               const int32_t* topk_idx, int ldk, uint16_t* dZ, uint16_t* A1,
                               uint16_t* B2, float* dwpart, float* dwslot, hipStream_t st);
int act_backward_parts(const Shape& s);
hipError_t launch_wgrad_offsets(const Shape& s, const int32_t* offsets, int32_t* poff,
                                hipStream_t st);
hipError_t launch_seg_transpose(const Shape& s, int kind, const void* src, int C,
                                const int32_t* offsets, const int32_t* sorted_assign,
                                const float* topk_w, const int32_t* poff, uint16_t* out, int ldk,
                                hipStream_t st);
hipError_t launch_seg_rowsum(const Shape& s, const uint16_t* M, int C, int ldk,
                             const int32_t* poff, float* db, hipStream_t st);
// logits: [T, E] as launch_router writes them; dwslot as launch_act_backward
// writes it.
hipError_t launch_router_backward(const Shape& s, const float* logits, const void* wr,
                                  const int32_t* topk_idx, const int32_t* assign_row,
                                  const float* dwslot, const int32_t* counts, float alpha,
                                  float* dlogits, float* d_topk_w, float* dxr, hipStream_t st);
hipError_t launch_router_wgrad(const Shape& s, const float* dlogits, const void* x, float* part,
                               float* bpart, float* dwr, float* dbr, hipStream_t st);
hipError_t launch_dx_gather(const Shape& s, const float* dxr, const float* dxrows,
                            const float* parts, int nparts, long long part_elems,
                            const int32_t* assign_row, const int32_t* offsets, float* dx,
                            hipStream_t st);

}  // namespace moe
