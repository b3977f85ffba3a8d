// Backward pass of the MoE-FFN layer (bf16 problems, token-choice routing).
//
// Objective: L = <dy, y> + alpha * L_aux — the task loss and the load-balancing
// loss merged before one backward ("MoE混合专家模型…" 4.3; "手撕一个极简
// MoE-FFN" 七).  Top-k selection, capacity drops and the counts f_e are
// piecewise constant and pass no gradient; a dropped slot sends none to its
// expert or gate weight; shared experts have weight 1.
//
// The expert activations are recomputed from the routing the forward pass
// returns, instead of being stored by it:
//   Z  = x_rows W1^T + b1                 grouped GEMM, fp32 [rows, F1]
//   G  = dy_rows W2                        grouped GEMM against W2 transposed
//   per tile of 64 rows x 64 columns of h: h = act(Z), dZ = act'(Z) * (w G)
//            (SwiGLU: [w G u silu'(g); w G silu(g)]), written row-major and
//            transposed, and the partial sums of <h, G>; the gate weight's
//            gradient dw = (sum of the partials) + <b2, dy>
//   dX_rows = dZ W1                        grouped GEMM against W1 transposed
//   dW2_e = (w dy)_e^T H_e, dW1_e = dZ_e^T x_e   per-expert GEMMs reducing
//            over the expert's rows (operands transposed, rows zero-padded)
//   db2_e, db1_e = sums over the expert's rows
//   router: dw -> renormalized top-k -> softmax / normalized sigmoid (+ the
//            aux term alpha E f_e / T on every p[t, e]) -> dlogits;
//            dx += dlogits Wr, dWr = dlogits^T x, dbr = column sums
//   dx[t] = router part + sum over kept slots and shared experts of dX rows.
// Every sum runs in a fixed order: results are deterministic.
#include "moe_internal.h"

namespace moe {

namespace {

// Row segments: routed rows [0, offsets[E]) by expert, then the S shared
// experts' T rows each.  Token and gate weight of a row.
__device__ __forceinline__ void row_info(int r, const int32_t* offsets, const int32_t* sorted_assign,
                                         const float* topk_w, int T, int k, int E, int& seg,
                                         int& tok, float& wgt, int& assign) {
  const int off_E = offsets[E];
  if (r < off_E) {
    int lo = 0, hi = E;   // last e with offsets[e] <= r
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (offsets[mid] <= r) lo = mid; else hi = mid;
    }
    seg = lo;
    assign = sorted_assign[r];
    tok = assign / k;
    wgt = topk_w[assign];
  } else {
    const int q = (r - off_E) / T;
    seg = E + q;
    tok = (r - off_E) - q * T;
    wgt = 1.0f;
    assign = -1;
  }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// ---------------------------------------------------------------- elementwise
__global__ __launch_bounds__(256) void cast_bf16_kernel(const float* __restrict__ src,
                                                        uint16_t* __restrict__ dst, long long n4) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4 v = *(const f32x4*)(src + 4 * i);
  u32x2 o;
  o[0] = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
  o[1] = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
  *(u32x2*)(dst + 4 * i) = o;
}

// dst[m][c][r] = src[m][r][c] for nmat matrices of R x C bf16 (R, C multiples of 64).
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ src,
                                                        uint16_t* __restrict__ dst, int R, int C) {
  __shared__ uint16_t tile[64][64 + 2];
  const long long mat = (long long)blockIdx.z * R * C;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tid = threadIdx.x;
  // read 64 rows x 64 columns: 8 threads per row, 8 columns each
  for (int rr = tid / 8; rr < 64; rr += 32) {
    const u32x4 v = *(const u32x4*)(src + mat + (long long)(r0 + rr) * C + c0 + (tid % 8) * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      tile[rr][(tid % 8) * 8 + 2 * i] = (uint16_t)(v[i] & 0xffffu);
      tile[rr][(tid % 8) * 8 + 2 * i + 1] = (uint16_t)(v[i] >> 16);
    }
  }
  __syncthreads();
  for (int cc = tid / 8; cc < 64; cc += 32) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = (tid % 8) * 8 + 2 * i;
      v[i] = (uint32_t)tile[rr][cc] | ((uint32_t)tile[rr + 1][cc] << 16);
    }
    *(u32x4*)(dst + mat + (long long)(c0 + cc) * R + r0 + (tid % 8) * 8) = v;
  }
}

// Padded column start of every segment for the weight-gradient operands:
// poff[seg] = sum of wgrad_pad(rows) of the segments before it.
__global__ __launch_bounds__(64) void wgrad_offsets_kernel(const int32_t* __restrict__ offsets,
                                                           int T, int E, int S,
                                                           int32_t* __restrict__ poff) {
  if (threadIdx.x != 0) return;
  int acc = 0;
  for (int seg = 0; seg < E + S; ++seg) {
    poff[seg] = acc;
    const int rows = seg < E ? offsets[seg + 1] - offsets[seg] : T;
    acc += wgrad_pad(rows);
  }
  poff[E + S] = acc;
}

// out[c][poff[seg] + i] = scale(row) * src[token(row)][c] for the segment's
// rows i (bf16), 0 in the padding.  SRC32: fp32 source (else bf16); SCALE:
// times the row's gate weight.  Block = 64 padded rows (two 32-row halves,
// each inside one segment) x 64 columns; thread = a pair of adjacent rows x 8
// columns, staged in LDS as [column][row pair] bf16 pairs so each output row
// leaves as 128 contiguous bytes written by 8 lanes.
constexpr int ST_R = 64;   // padded rows per block
template <bool SRC32, bool SCALE>
__global__ __launch_bounds__(256) void seg_transpose_kernel(
    const void* __restrict__ src, int C, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_assign, const float* __restrict__ topk_w,
    const int32_t* __restrict__ poff, int T, int k, int E, int S, uint16_t* __restrict__ out,
    int ldk) {
  constexpr int PW = ST_R / 2 + 4;   // words per staged column: 32 row pairs + 16 bytes
  __shared__ uint32_t tile[64][PW];
  __shared__ int sh_seg[2];
  const int p0 = blockIdx.x * ST_R, c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  const int nseg = E + S;
  const int pend = poff[nseg];   // end of the used columns (a multiple of 64)
  if (p0 >= pend) return;        // uniform
  if (tid < nseg) {
    const int lo = poff[tid], hi = poff[tid + 1];
    if (lo <= p0 && p0 < hi) sh_seg[0] = tid;
    if (lo <= p0 + 32 && p0 + 32 < hi) sh_seg[1] = tid;
  }
  __syncthreads();
  const int pr = tid / 8, cq = (tid % 8) * 8;   // row pair, first of 8 columns
  const int hf = pr >> 4;                       // the 32-row half (uniform per wave)
  const bool used = p0 + 32 * hf < pend;
  const int seg = used ? sh_seg[hf] : 0;
  const int rows = seg < E ? offsets[seg + 1] - offsets[seg] : T;
  const int base = seg < E ? offsets[seg] : offsets[E] + (seg - E) * T;
  float v[2][8];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int i = p0 + 2 * pr + rr - poff[seg];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[rr][j] = 0.0f;
    if (!used || i >= rows) continue;
    const int r = base + i;
    int srow = i;   // shared expert: row i is token i
    float sc = 1.0f;
    if (seg < E) {
      const int a = sorted_assign[r];
      srow = a / k;
      if (SCALE) sc = topk_w[a];
    }
    if (SRC32) {
      const float* sp = (const float*)src + (long long)srow * C + c0 + cq;
      const f32x4 a0 = *(const f32x4*)sp, a1 = *(const f32x4*)(sp + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[rr][j] = a0[j] * sc, v[rr][4 + j] = a1[j] * sc;
    } else {
      const u32x4 a = *(const u32x4*)((const uint16_t*)src + (long long)srow * C + c0 + cq);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[rr][2 * j] = __uint_as_float(a[j] << 16) * sc;
        v[rr][2 * j + 1] = __uint_as_float(a[j] & 0xffff0000u) * sc;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    tile[cq + j][pr] = (uint32_t)f32_to_bf16_rne(v[0][j]) | ((uint32_t)f32_to_bf16_rne(v[1][j]) << 16);
  __syncthreads();
  // output row cc, rows p0 + 8 ch .. + 7 (16 bytes); chunks past the used
  // columns (whole 32-row halves) are not written
  const int ch = tid & 7;
  if (p0 + 8 * ch < pend) {
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int cc = (tid >> 3) + 32 * pass;
      *(u32x4*)(out + (long long)(c0 + cc) * ldk + p0 + 8 * ch) = *(const u32x4*)&tile[cc][4 * ch];
    }
  }
}

// db[seg][c] = sum over the segment's padded columns of M[c][.] (bf16), in
// column order per lane, then a fixed butterfly.  One wave per (seg, c).
__global__ __launch_bounds__(256) void seg_rowsum_kernel(const uint16_t* __restrict__ M, int C,
                                                         int ldk, const int32_t* __restrict__ poff,
                                                         int nseg, float* __restrict__ db) {
  const long long wid = ((long long)blockIdx.x * 256 + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (wid >= (long long)nseg * C) return;
  const int seg = (int)(wid / C), c = (int)(wid % C);
  const int lo = poff[seg], hi = poff[seg + 1];
  const uint16_t* row = M + (long long)c * ldk;
  float s = 0.0f;
  for (int i = lo + lane * 8; i < hi; i += 512) {
    const u32x4 v = *(const u32x4*)(row + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) s += __uint_as_float(v[j] << 16) + __uint_as_float(v[j] & 0xffff0000u);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) db[(long long)seg * C + c] = s;
}

// ---------------------------------------------------------------- activation backward
// GELU'(z) = Phi(z) + z phi(z), Phi from the erf approximation of the
// forward (Abramowitz & Stegun 7.1.28), phi(z) = exp(-z^2/2) / sqrt(2 pi).
__device__ __forceinline__ float gelu_grad_f(float z) {
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
  const float r = __builtin_amdgcn_rcpf(p);   // 1 - erf(|z| / sqrt 2)
  const float cdf = z >= 0.0f ? 1.0f - 0.5f * r : 0.5f * r;
  const float pdf = 0.3989422804014327f * fast_exp(-0.5f * z * z);
  return fmaf(z, pdf, cdf);
}

// One block per 64 padded rows (the weight-gradient layout of
// wgrad_offsets_kernel: segments start at multiples of 64, so each 32-row
// half of the block lies in one segment) and 64 columns c of h.  For each row
// it forms h = act(Z), dZ = act'(Z) w G (SwiGLU: the gate and the up column)
// and the partial sum <h, G> over its 64 columns; it writes dZ row-major (the
// dX product's operand) and both transposed weight-gradient operands, dZ^T
// into A1 [F1][ldk] and h^T into B2 [f][ldk] (zero in the padding rows), so
// no separate transposes are needed.  Thread = a pair of adjacent rows x 8
// columns; the pairs are staged in LDS as [column][row pair] bf16 pairs, so
// each transposed row leaves as 128 contiguous bytes written by 8 lanes.
// dwpart[row][c / 64] holds the partial sums of routed rows;
// slot_grad_kernel adds them in column order.
constexpr int AB_C = 64;   // columns of h per block
constexpr int AB_R = 64;   // padded rows per block
template <int ACT>
__global__ __launch_bounds__(256) void act_backward_kernel(
    const float* __restrict__ Z, const float* __restrict__ G, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_assign, const float* __restrict__ topk_w,
    const int32_t* __restrict__ poff, int T, int E, int S, int f, int ldk,
    uint16_t* __restrict__ dZ, uint16_t* __restrict__ A1, uint16_t* __restrict__ B2,
    float* __restrict__ dwpart, int nparts) {
  constexpr bool SWIGLU = ACT == MOE_SWIGLU;
  constexpr int PW = AB_R / 2 + 4;   // words per staged column: 32 row pairs + 16 bytes
  __shared__ uint32_t th[AB_C][PW], tz[AB_C][PW], tu[SWIGLU ? AB_C : 1][PW];
  __shared__ int sh_seg[2];
  const int p0 = blockIdx.x * AB_R, c0 = blockIdx.y * AB_C;
  const int tid = threadIdx.x;
  const int nseg = E + S;
  const int pend = poff[nseg];   // end of the used columns (a multiple of 64)
  if (p0 >= pend) return;        // uniform
  if (tid < nseg) {
    const int lo = poff[tid], hi = poff[tid + 1];
    if (lo <= p0 && p0 < hi) sh_seg[0] = tid;
    if (lo <= p0 + 32 && p0 + 32 < hi) sh_seg[1] = tid;
  }
  __syncthreads();
  const int pr = tid >> 3, cq = (tid & 7) * 8;   // row pair, first of 8 columns
  const int hf = pr >> 4;                        // the 32-row half (uniform per wave)
  const bool used = p0 + 32 * hf < pend;
  const int seg = used ? sh_seg[hf] : 0;
  const int rows = seg < E ? offsets[seg + 1] - offsets[seg] : T;
  const int base = seg < E ? offsets[seg] : offsets[E] + (seg - E) * T;
  const int F1 = SWIGLU ? 2 * f : f;
  float h[2][8], dz[2][8], du[2][8], dot[2];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
#pragma unroll
    for (int q = 0; q < 8; ++q) h[rr][q] = dz[rr][q] = du[rr][q] = 0.0f;
    dot[rr] = 0.0f;
    const int i = p0 + 2 * pr + rr - poff[seg];
    if (!used || i >= rows) continue;
    const long long r = base + i;
    const float wgt = seg < E ? topk_w[sorted_assign[r]] : 1.0f;
    const float* zr = Z + r * F1 + c0 + cq;
    const float* gr = G + r * f + c0 + cq;
    const f32x4 z0 = *(const f32x4*)zr, z1 = *(const f32x4*)(zr + 4);
    const f32x4 g0 = *(const f32x4*)gr, g1 = *(const f32x4*)(gr + 4);
    f32x4 u0 = {}, u1 = {};
    if (SWIGLU) u0 = *(const f32x4*)(zr + f), u1 = *(const f32x4*)(zr + f + 4);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float z = q < 4 ? z0[q] : z1[q - 4];
      const float g = q < 4 ? g0[q] : g1[q - 4];
      const float wg = wgt * g;
      if (ACT == MOE_RELU) {
        h[rr][q] = fmaxf(z, 0.0f);
        dz[rr][q] = z > 0.0f ? wg : 0.0f;
      } else if (ACT == MOE_GELU) {
        h[rr][q] = gelu_f(z);
        dz[rr][q] = wg * gelu_grad_f(z);
      } else {
        const float u = q < 4 ? u0[q] : u1[q - 4];
        const float sg = __builtin_amdgcn_rcpf(1.0f + fast_exp(-z));
        const float si = z * sg;
        h[rr][q] = si * u;
        dz[rr][q] = wg * u * sg * fmaf(z, 1.0f - sg, 1.0f);
        du[rr][q] = wg * si;
      }
      dot[rr] = fmaf(h[rr][q], g, dot[rr]);
    }
    u32x4 zo, uo;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      zo[q] = (uint32_t)f32_to_bf16_rne(dz[rr][2 * q]) |
              ((uint32_t)f32_to_bf16_rne(dz[rr][2 * q + 1]) << 16);
      uo[q] = (uint32_t)f32_to_bf16_rne(du[rr][2 * q]) |
              ((uint32_t)f32_to_bf16_rne(du[rr][2 * q + 1]) << 16);
    }
    *(u32x4*)(dZ + r * F1 + c0 + cq) = zo;
    if (SWIGLU) *(u32x4*)(dZ + r * F1 + f + c0 + cq) = uo;
  }
  // each row's partial <h, G>: its 8 threads are consecutive lanes
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    float v = dot[rr];
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    const int i = p0 + 2 * pr + rr - poff[seg];
    if (used && i < rows && seg < E && (tid & 7) == 0)
      dwpart[(base + i) * (long long)nparts + blockIdx.y] = v;
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    th[cq + q][pr] = (uint32_t)f32_to_bf16_rne(h[0][q]) | ((uint32_t)f32_to_bf16_rne(h[1][q]) << 16);
    tz[cq + q][pr] =
        (uint32_t)f32_to_bf16_rne(dz[0][q]) | ((uint32_t)f32_to_bf16_rne(dz[1][q]) << 16);
    if (SWIGLU)
      tu[cq + q][pr] =
          (uint32_t)f32_to_bf16_rne(du[0][q]) | ((uint32_t)f32_to_bf16_rne(du[1][q]) << 16);
  }
  __syncthreads();
  // transposed: column cc, rows p0 + 8 ch .. + 7 (16 bytes); a column's 8
  // chunks are 8 consecutive lanes.  Chunks past the used columns (whole
  // 32-row halves) are not written.
  const int ch = tid & 7;
  if (p0 + 8 * ch < pend) {
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int cc = (tid >> 3) + 32 * pass;
      const long long o = (long long)(c0 + cc) * ldk + p0 + 8 * ch;
      *(u32x4*)(B2 + o) = *(const u32x4*)&th[cc][4 * ch];
      *(u32x4*)(A1 + o) = *(const u32x4*)&tz[cc][4 * ch];
      if (SWIGLU) *(u32x4*)(A1 + (long long)f * ldk + o) = *(const u32x4*)&tu[cc][4 * ch];
    }
  }
}

// dwslot[t*k + s] = <h, G> + <b2_e, dy_t> for a kept slot (0 if dropped):
// one wave per token; for each slot the lanes split the column partials of
// its row (dwpart[row][.]) and the d products of the bias term, then a fixed
// sum over the wave (DPP row steps, then the row results) adds them.
__global__ __launch_bounds__(256) void slot_grad_kernel(
    const int32_t* __restrict__ assign_row, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ dwpart, int nparts, const uint16_t* __restrict__ b_down,
    const float* __restrict__ dy, int T, int k, int d, float* __restrict__ dwslot) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;   // per wave
  for (int s = 0; s < k; ++s) {
    const int row = assign_row[(long long)t * k + s];
    float v = 0.0f;
    if (row >= 0) {   // uniform over the wave
      for (int c = lane; c < nparts; c += 64) v += dwpart[(long long)row * nparts + c];
      if (b_down) {
        const uint16_t* br = b_down + (long long)topk_idx[(long long)t * k + s] * d;
        const float* dyr = dy + (long long)t * d;
        for (int j = lane; j < d; j += 64) v = fmaf(bf16_to_f32(br[j]), dyr[j], v);
      }
    }
    v = wave_sum_dpp(v);
    if (lane == 0) dwslot[(long long)t * k + s] = v;
  }
}

// ---------------------------------------------------------------- router backward
// One wave per RBT tokens; for each token, lane e holds the logit of expert e
// (from the router kernel) and computes the keys (softmax p, or sigma for the
// normalized sigmoid), then
//   dkey[e_s] += (dw_s - sum_s' w_s' dw_s') / S   (renormalized top-k)
//   dp[e]      = alpha E f_e / T                    (aux loss through P)
//   softmax:  dl = p (dkey + dp - sum p (dkey + dp))
//   sigmoid:  dl = (dkey + (dp - sum p dp) / sum sigma) sigma (1 - sigma)
// written to dlogits [T, E]; router_dx_kernel then forms dx_router = dl Wr.
constexpr int RBT = 4;   // tokens per wave
__global__ __launch_bounds__(256) void router_backward_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ assign_row, const float* __restrict__ dwslot,
    const int32_t* __restrict__ counts, float alpha, int T, int E, int k, int gating,
    float* __restrict__ dlogits, float* __restrict__ d_topk_w) {
  const int lane = threadIdx.x & 63;
  const int tb = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RBT;
  if (tb >= T) return;   // per wave
  const bool act = lane < E;
  const float dp = act ? alpha * (float)E * ((float)counts[act ? lane : 0] / ((float)T * k)) / T
                       : 0.0f;
#pragma unroll
  for (int i = 0; i < RBT; ++i) {
    const int t = tb + i;
    if (t >= T) continue;   // uniform over the wave
    const float l = act ? logits[(long long)t * E + lane] : 0.0f;
    float key, p, sig = 0.0f, tot = 1.0f;
    if (gating == MOE_SOFTMAX) {
      const float m = wave_max_dpp(act ? l : -INFINITY);
      const float ex = act ? fast_exp(l - m) : 0.0f;
      const float sum = wave_sum_dpp(ex);
      p = ex / sum;
      key = p;
    } else {
      sig = act ? 1.0f / (1.0f + fast_exp(-l)) : 0.0f;
      tot = wave_sum_dpp(sig);
      p = sig / tot;
      key = sig;
    }
    // renormalized top-k
    float S = 0.0f, inner = 0.0f, dws[kMaxTopK], ks_[kMaxTopK];
    int es[kMaxTopK];
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
      es[s] = 0;
      dws[s] = 0.0f;
      if (s < k) {
        es[s] = topk_idx[(long long)t * k + s];
        dws[s] = assign_row[(long long)t * k + s] >= 0 ? dwslot[(long long)t * k + s] : 0.0f;
      }
      es[s] = __builtin_amdgcn_readfirstlane(es[s]);   // the same entry in every lane
      ks_[s] = lane_f(key, es[s]);
      if (s < k) S += ks_[s];
    }
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s)
      if (s < k) inner = fmaf(ks_[s] / S, dws[s], inner);
    float dkey = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s)
      if (s < k && es[s] == lane) dkey += (dws[s] - inner) / S;
    float dl;
    if (gating == MOE_SOFTMAX) {
      const float g = dkey + dp;
      const float pg = wave_sum_dpp(act ? p * g : 0.0f);
      dl = act ? p * (g - pg) : 0.0f;
    } else {
      const float pd = wave_sum_dpp(act ? p * dp : 0.0f);
      const float ds = dkey + (dp - pd) / tot;
      dl = act ? ds * sig * (1.0f - sig) : 0.0f;
    }
    if (act) dlogits[(long long)t * E + lane] = dl;
    if (d_topk_w && lane < k) {
      float v = 0.0f;
#pragma unroll
      for (int s = 0; s < kMaxTopK; ++s) v = s == lane ? dws[s] : v;
      d_topk_w[(long long)t * k + lane] = v;
    }
  }
}

// dx_router[t, j] = sum_e dl[t, e] Wr[e, j] on the fp32 matrix cores
// (MFMA 16x16x4: A = 16 tokens x 4 experts of dl, B = 4 experts x 16 columns
// of Wr widened from bf16; the experts are padded to a multiple of 4 with
// zeros).  One wave per 16 tokens x 64 columns, K = E in steps of 4.
__global__ __launch_bounds__(256) void router_dx_kernel(const float* __restrict__ dl,
                                                        const uint16_t* __restrict__ wr, int T,
                                                        int d, int E, float* __restrict__ dxr) {
  const int lane = threadIdx.x & 63;
  const int ntj = (d + 63) / 64;
  const long long wid = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long t0 = wid / ntj * 16;
  const int j0 = (int)(wid % ntj) * 64;
  if (t0 >= T) return;   // per wave
  const int i = lane & 15, kq = lane >> 4;
  const long long t = t0 + i < T ? t0 + i : T - 1;
  f32x4 acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = f32x4{};
  for (int e0 = 0; e0 < E; e0 += 4) {
    const int e = e0 + kq;
    const float av = e < E ? dl[t * E + e] : 0.0f;
    float bv[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int j = j0 + n * 16 + i;
      bv[n] = (e < E && j < d) ? bf16_to_f32(wr[(long long)e * d + j]) : 0.0f;
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv[n], acc[n], 0, 0, 0);
  }
  // lane holds tokens t0 + 4 kq + r (r = 0..3) of column i of each 16-column tile
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int j = j0 + n * 16 + i;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const long long tr = t0 + 4 * kq + r;
      if (tr < T && j < d) dxr[tr * d + j] = acc[n][r];
    }
  }
}

// Partial router weight gradient over a slice of `tpb` tokens (a multiple of
// 64): part[slice][e][j] = sum over the slice's tokens (in order) of
// dl[t, e] x[t, j]; bpart[slice][e] likewise of dl[t, e] (blocks of column
// chunk 0).  Block = 256 columns; the slice moves through LDS 64 tokens at a
// time (x by 16-byte loads, dl as [64][EB]).  Thread = CPT adjacent columns
// x EB / CPT experts (a wave shares its experts, so their dl values are LDS
// broadcasts): with many experts each LDS read of dl feeds CPT products.
template <int EB>
__global__ __launch_bounds__(256) void router_wgrad_part_kernel(
    const float* __restrict__ dl, const uint16_t* __restrict__ x, int T, int d, int E, int tpb,
    float* __restrict__ part, float* __restrict__ bpart) {
  constexpr int CPT = EB >= 32 ? EB / 16 : 1;   // columns per thread = expert groups
  constexpr int EPT = EB / CPT;                 // experts per thread
  __shared__ __attribute__((aligned(16))) uint16_t xs[64][256 + 8];
  __shared__ __attribute__((aligned(16))) float sdl[64][EB];
  const int tid = threadIdx.x;
  const int eg = tid / (256 / CPT), cg = tid % (256 / CPT);   // expert group, column group
  const int c0 = blockIdx.x * 256, jc = cg * CPT;             // first column of the thread
  const int ts = blockIdx.y * tpb, te = min(T, ts + tpb);
  float acc[EPT][CPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e)
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[e][c] = 0.0f;
  float bsum = 0.0f;
  for (int t0 = ts; t0 < te; t0 += 64) {
    __syncthreads();   // the previous tile's reads are done
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = tid + 256 * i;          // 16-byte chunk: row q / 32, columns (q % 32) * 8
      const int rr = q >> 5, cc = (q & 31) * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (t0 + rr < te && c0 + cc < d) v = *(const u32x4*)(x + (long long)(t0 + rr) * d + c0 + cc);
      *(u32x4*)&xs[rr][cc] = v;
    }
    for (int i = tid; i < 64 * EB; i += 256) {
      const int rr = i / EB, e = i % EB;
      sdl[rr][e] = (e < E && t0 + rr < te) ? dl[(long long)(t0 + rr) * E + e] : 0.0f;
    }
    __syncthreads();
#pragma unroll 4
    for (int rr = 0; rr < 64; ++rr) {
      float xv[CPT];
      if (CPT == 4) {
        const u32x2 p = *(const u32x2*)&xs[rr][jc];
        xv[0] = __uint_as_float(p[0] << 16);
        xv[1 % CPT] = __uint_as_float(p[0] & 0xffff0000u);
        xv[2 % CPT] = __uint_as_float(p[1] << 16);
        xv[3 % CPT] = __uint_as_float(p[1] & 0xffff0000u);
      } else {
#pragma unroll
        for (int c = 0; c < CPT; ++c) xv[c] = bf16_to_f32(xs[rr][jc + c]);
      }
#pragma unroll
      for (int e = 0; e < EPT; e += 4) {
        const f32x4 dv = *(const f32x4*)&sdl[rr][eg * EPT + e];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          acc[e][c] = fmaf(dv[0], xv[c], acc[e][c]);
          acc[e + 1][c] = fmaf(dv[1], xv[c], acc[e + 1][c]);
          acc[e + 2][c] = fmaf(dv[2], xv[c], acc[e + 2][c]);
          acc[e + 3][c] = fmaf(dv[3], xv[c], acc[e + 3][c]);
        }
      }
      if (blockIdx.x == 0 && tid < E) bsum += sdl[rr][tid];
    }
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int ee = eg * EPT + e;
    if (ee >= E) continue;
    float* o = part + ((long long)blockIdx.y * E + ee) * d + c0 + jc;
#pragma unroll
    for (int c = 0; c < CPT; ++c)
      if (c0 + jc + c < d) o[c] = acc[e][c];
  }
  if (blockIdx.x == 0 && tid < E) bpart[(long long)blockIdx.y * E + tid] = bsum;
}

// out[i] = sum over the nslices slices of part[slice * n + i], i < n: thread
// (o, q) of a block sums slices q, q + 16, ... of output o (in order), then
// the 16 group sums are added in group order.  16 outputs per block.
__global__ __launch_bounds__(256) void slice_sum_kernel(const float* __restrict__ part,
                                                        int nslices, long long n,
                                                        float* __restrict__ out) {
  __shared__ float acc[16][17];
  const int o = threadIdx.x & 15, q = threadIdx.x >> 4;
  const long long i = (long long)blockIdx.x * 16 + o;
  float v = 0.0f;
  if (i < n)
    for (int sl = q; sl < nslices; sl += 16) v += part[(long long)sl * n + i];
  acc[q][o] = v;
  __syncthreads();
  if (q == 0 && i < n) {
    float t = 0.0f;
#pragma unroll
    for (int g = 0; g < 16; ++g) t += acc[g][o];
    out[i] = t;
  }
}

// dx[t] = dx_router[t] + sum over kept slots (slot order) of the dX row (+ its
// K-slice parts) + sum over shared experts of their rows.  One thread per 4
// columns.
__global__ __launch_bounds__(256) void dx_gather_kernel(
    const float* __restrict__ dxr, const float* __restrict__ dxrows,
    const float* __restrict__ parts, int nparts, long long part_elems,
    const int32_t* __restrict__ assign_row, const int32_t* __restrict__ offsets, int T, int d,
    int k, int E, int S, float* __restrict__ dx) {
  const int dv = d / 4;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (long long)T * dv) return;
  const int t = (int)(gid / dv);
  const int c = (int)(gid % dv) * 4;
  auto row = [&](long long r) {
    f32x4 v = *(const f32x4*)(dxrows + r * d + c);
    for (int p = 0; p < nparts; ++p) v += *(const f32x4*)(parts + p * part_elems + r * d + c);
    return v;
  };
  f32x4 acc = *(const f32x4*)(dxr + (long long)t * d + c);
  for (int s = 0; s < k; ++s) {
    const int r = assign_row[(long long)t * k + s];
    if (r >= 0) acc += row(r);
  }
  const long long base = offsets[E];
  for (int q = 0; q < S; ++q) acc += row(base + (long long)q * T + t);
  *(f32x4*)(dx + (long long)t * d + c) = acc;
}

}  // namespace

// ---------------------------------------------------------------- launchers
hipError_t launch_cast_bf16(const float* src, uint16_t* dst, long long n, hipStream_t st) {
  const long long n4 = n / 4;
  cast_bf16_kernel<<<(int)((n4 + 255) / 256), 256, 0, st>>>(src, dst, n4);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* src, void* dst, int nmat, int R, int C, hipStream_t st) {
  transpose_kernel<<<dim3(C / 64, R / 64, nmat), 256, 0, st>>>((const uint16_t*)src,
                                                               (uint16_t*)dst, R, C);
  return hipGetLastError();
}

hipError_t launch_wgrad_offsets(const Shape& s, const int32_t* offsets, int32_t* poff,
                                hipStream_t st) {
  wgrad_offsets_kernel<<<1, 64, 0, st>>>(offsets, s.T, s.E, s.S, poff);
  return hipGetLastError();
}

// kind 0: fp32 rows gathered by token and scaled by the gate weight (dy);
// kind 1: bf16 rows gathered by token (x).
hipError_t launch_seg_transpose(const Shape& s, int kind, const void* src, int C,
                                const int32_t* offsets, const int32_t* sorted_assign,
                                const float* topk_w, const int32_t* poff, uint16_t* out, int ldk,
                                hipStream_t st) {
  const dim3 grid((ldk + ST_R - 1) / ST_R, C / 64);
  if (kind == 0)
    seg_transpose_kernel<true, true><<<grid, 256, 0, st>>>(
        src, C, offsets, sorted_assign, topk_w, poff, s.T, s.k, s.E, s.S, out, ldk);
  else
    seg_transpose_kernel<false, false><<<grid, 256, 0, st>>>(
        src, C, offsets, sorted_assign, topk_w, poff, s.T, s.k, s.E, s.S, out, ldk);
  return hipGetLastError();
}

hipError_t launch_seg_rowsum(const Shape& s, const uint16_t* M, int C, int ldk,
                             const int32_t* poff, float* db, hipStream_t st) {
  const long long waves = (long long)(s.E + s.S) * C;
  seg_rowsum_kernel<<<(int)((waves * 64 + 255) / 256), 256, 0, st>>>(M, C, ldk, poff, s.E + s.S,
                                                                      db);
  return hipGetLastError();
}

hipError_t launch_act_backward(const Shape& s, const float* Z, const float* G, const float* dy,
                               const void* b_down, const int32_t* offsets,
                               const int32_t* sorted_assign, const float* topk_w,
                               const int32_t* poff, const int32_t* assign_row,
                               const int32_t* topk_idx, int ldk, uint16_t* dZ, uint16_t* A1,
                               uint16_t* B2, float* dwpart, float* dwslot, hipStream_t st) {
  const dim3 grid((ldk + AB_R - 1) / AB_R, s.f / AB_C);
  const int nparts = s.f / AB_C;
  const uint16_t* b2 = (const uint16_t*)b_down;
#define MOE_ACT_BWD(A)                                                                          \
  act_backward_kernel<A><<<grid, 256, 0, st>>>(Z, G, offsets, sorted_assign, topk_w, poff,    \
                                               s.T, s.E, s.S, s.f, ldk, dZ, A1, B2, dwpart,    \
                                               nparts)
  if (s.act == MOE_RELU) MOE_ACT_BWD(MOE_RELU);
  else if (s.act == MOE_GELU) MOE_ACT_BWD(MOE_GELU);
  else MOE_ACT_BWD(MOE_SWIGLU);
#undef MOE_ACT_BWD
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  slot_grad_kernel<<<(s.T + 3) / 4, 256, 0, st>>>(assign_row, topk_idx, dwpart, nparts, b2, dy,
                                                  s.T, s.k, s.d, dwslot);
  return hipGetLastError();
}

int act_backward_parts(const Shape& s) { return s.f / AB_C; }

hipError_t launch_router_backward(const Shape& s, const float* logits, const void* wr,
                                  const int32_t* topk_idx, const int32_t* assign_row,
                                  const float* dwslot, const int32_t* counts, float alpha,
                                  float* dlogits, float* d_topk_w, float* dxr, hipStream_t st) {
  router_backward_kernel<<<(s.T + 4 * RBT - 1) / (4 * RBT), 256, 0, st>>>(
      logits, topk_idx, assign_row, dwslot, counts, alpha, s.T, s.E, s.k, s.gating, dlogits,
      d_topk_w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long waves = (long long)(s.T + 15) / 16 * ((s.d + 63) / 64);
  router_dx_kernel<<<(int)((waves + 3) / 4), 256, 0, st>>>(dlogits, (const uint16_t*)wr, s.T, s.d,
                                                          s.E, dxr);
  return hipGetLastError();
}

// Token slice per block of the router weight gradient: a multiple of 64,
// about 512 blocks in all.
static int router_wgrad_tpb(const Shape& s) {
  const int cchunks = (s.d + 255) / 256;
  const int want = 512 / cchunks > 1 ? 512 / cchunks : 1;     // slices wanted
  int tpb = (s.T + want - 1) / want;
  tpb = (tpb + 63) / 64 * 64;
  return tpb < 64 ? 64 : tpb;
}

int router_wgrad_slices(const Shape& s) {
  const int tpb = router_wgrad_tpb(s);
  return (s.T + tpb - 1) / tpb;
}

hipError_t launch_router_wgrad(const Shape& s, const float* dlogits, const void* x, float* part,
                               float* bpart, float* dwr, float* dbr, hipStream_t st) {
  const int tpb = router_wgrad_tpb(s), ns = router_wgrad_slices(s);
  const dim3 grid((s.d + 255) / 256, ns);
  const uint16_t* xb = (const uint16_t*)x;
  if (s.E <= 8)
    router_wgrad_part_kernel<8><<<grid, 256, 0, st>>>(dlogits, xb, s.T, s.d, s.E, tpb, part, bpart);
  else if (s.E <= 16)
    router_wgrad_part_kernel<16><<<grid, 256, 0, st>>>(dlogits, xb, s.T, s.d, s.E, tpb, part, bpart);
  else if (s.E <= 32)
    router_wgrad_part_kernel<32><<<grid, 256, 0, st>>>(dlogits, xb, s.T, s.d, s.E, tpb, part, bpart);
  else
    router_wgrad_part_kernel<64><<<grid, 256, 0, st>>>(dlogits, xb, s.T, s.d, s.E, tpb, part, bpart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n = (long long)s.E * s.d;
  slice_sum_kernel<<<(int)((n + 15) / 16), 256, 0, st>>>(part, ns, n, dwr);
  e = hipGetLastError();
  if (e != hipSuccess || !dbr) return e;
  slice_sum_kernel<<<(s.E + 15) / 16, 256, 0, st>>>(bpart, ns, s.E, dbr);
  return hipGetLastError();
}

hipError_t launch_dx_gather(const Shape& s, const float* dxr, const float* dxrows,
                            const float* parts, int nparts, long long part_elems,
                            const int32_t* assign_row, const int32_t* offsets, float* dx,
                            hipStream_t st) {
  const long long n = (long long)s.T * (s.d / 4);
  dx_gather_kernel<<<(int)((n + 255) / 256), 256, 0, st>>>(dxr, dxrows, parts, nparts, part_elems,
                                                           assign_row, offsets, s.T, s.d, s.k, s.E,
                                                           s.S, dx);
  return hipGetLastError();
}

}  // namespace moe
