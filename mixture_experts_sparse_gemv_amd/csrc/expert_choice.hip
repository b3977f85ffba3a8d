// Expert-choice routing ("MoE架构解析", 二 2.2): every expert picks the C
// tokens it scores highest, so all experts carry exactly C rows; a token can
// be picked by several experts or by none.
//
// Selection, one block per expert: the column probs[:, e] (non-negative, so
// its float bits order like the values) is staged in LDS; a 4-pass radix
// select (8 bits per pass, LDS histogram) finds the C-th largest value v*;
// the tokens above v*, then the lowest-index tokens equal to v*, are kept —
// ties go to the lower token.  An order-preserving compaction (block scans
// over contiguous token chunks) writes each expert's tokens in ascending
// order: sorted_assign[e*C + i] = token, row_of[t*E + e] = e*C + i or -1.
//
// Combine: y[t] = sum over experts e (in order) with row_of[t, e] >= 0 of
// probs[t, e] * y_exp[row] (no renormalization), plus the shared experts.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int EW = 16;          // waves of a selection block
constexpr int ET = EW * 64;     // threads

// Exclusive scan over the block of one int per thread (in thread order);
// returns the thread's exclusive prefix and the block total in *total.
__device__ int block_exclusive_scan(int v, int* wtot, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int base = 0, all = 0;
  for (int w = 0; w < EW; ++w) {
    const int t = wtot[w];
    if (w < wave) base += t;
    all += t;
  }
  __syncthreads();   // wtot is reused by the next scan
  *total = all;
  return base + incl - v;
}

__global__ __launch_bounds__(ET) void ec_select_kernel(const float* __restrict__ probs, int T,
                                                       int E, int C,
                                                       int32_t* __restrict__ sorted_assign,
                                                       int32_t* __restrict__ row_of,
                                                       int32_t* counts, int32_t* kept,
                                                       int32_t* offsets, float* colsum) {
  __shared__ uint32_t key[kEcMaxT];
  __shared__ int hist[256];
  __shared__ int wtot[EW];
  __shared__ float wsum[EW];
  __shared__ uint32_t pick[2];   // chosen digit, remaining rank
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = blockIdx.x;

  // stage the column; its sum in a fixed order (per thread in token order,
  // then a wave butterfly, then the waves in order)
  float part = 0.f;
  for (int t = tid; t < T; t += ET) {
    const float p = probs[(long long)t * E + e];
    key[t] = __float_as_uint(p);
    part += p;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o);
  if (lane == 0) wsum[wave] = part;

  // radix select of the C-th largest key, most significant byte first
  uint32_t prefix = 0, mask = 0;
  int remaining = C;   // rank still to find among the keys matching prefix
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += ET) hist[i] = 0;
    __syncthreads();
    for (int t = tid; t < T; t += ET) {
      const uint32_t k = key[t];
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds digits 4l .. 4l+3; suffix sums over lanes from the top
      const int h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
                h3 = hist[4 * lane + 3];
      const int mine = h0 + h1 + h2 + h3;
      int suf = mine;   // sum over lanes >= this lane
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_down(suf, o);
        if (lane + o < 64) suf += u;
      }
      const uint64_t reach = __ballot(suf >= remaining);   // a prefix of lanes from 0
      const int top = 63 - __builtin_clzll(reach);         // highest lane reaching the rank
      if (lane == top) {
        int above = suf - mine;   // keys in higher digits
        const int h[4] = {h0, h1, h2, h3};
        int d = 3;
        for (; d > 0; --d) {
          if (above + h[d] >= remaining) break;
          above += h[d];
        }
        pick[0] = (uint32_t)(4 * lane + d);
        pick[1] = (uint32_t)(remaining - above);
      }
    }
    __syncthreads();
    prefix |= pick[0] << shift;
    mask |= 255u << shift;
    remaining = (int)pick[1];
    __syncthreads();
  }
  const uint32_t vstar = prefix;   // the C-th largest key; take `remaining` of its ties

  // compaction in token order over contiguous chunks per thread
  const int CH = (T + ET - 1) / ET;
  const int t0 = min(T, tid * CH), t1 = min(T, t0 + CH);
  int neq = 0;
  for (int t = t0; t < t1; ++t) neq += key[t] == vstar;
  int dummy;
  int eq_before = block_exclusive_scan(neq, wtot, &dummy);
  int nsel = 0;
  for (int t = t0, eq = eq_before; t < t1; ++t) {
    const uint32_t k = key[t];
    if (k > vstar || (k == vstar && eq++ < remaining)) ++nsel;
  }
  int total_sel;
  const int sel_before = block_exclusive_scan(nsel, wtot, &total_sel);
  for (int t = t0, eq = eq_before, pos = sel_before; t < t1; ++t) {
    const uint32_t k = key[t];
    const bool take = k > vstar || (k == vstar && eq++ < remaining);
    if (take) {
      sorted_assign[(long long)e * C + pos] = t;
      row_of[(long long)t * E + e] = e * C + pos;
      ++pos;
    } else {
      row_of[(long long)t * E + e] = -1;
    }
  }
  if (tid == 0) {
    counts[e] = C;
    kept[e] = C;
    offsets[e] = e * C;
    if (e == E - 1) offsets[E] = E * C;
    float cs = 0.f;
    for (int w = 0; w < EW; ++w) cs += wsum[w];
    if (colsum) colsum[e] = cs;
  }
}

// token_experts[t] = number of experts that picked t (0 = orphan token)
__global__ __launch_bounds__(256) void token_experts_kernel(const int32_t* __restrict__ row_of,
                                                            int T, int E,
                                                            int32_t* __restrict__ token_experts) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  int n = 0;
  for (int e = 0; e < E; ++e) n += row_of[(long long)t * E + e] >= 0;
  token_experts[t] = n;
}

// One thread per NV groups of 4 outputs of a token, group j at column
// 4 (i + j d / (4 NV)) (as in the top-k combine).
template <int NV>
__global__ __launch_bounds__(256) void combine_ec_kernel(const float* __restrict__ probs,
                                                         const int32_t* __restrict__ row_of,
                                                         const int32_t* __restrict__ offsets,
                                                         const float* __restrict__ y_exp,
                                                         const float* __restrict__ y_part,
                                                         int nparts, long long part_elems,
                                                         float* __restrict__ y, int T, int d, int E,
                                                         int S) {
  const int dv = d / (4 * NV);   // threads per token
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)T * dv) return;
  const int t = (int)(gid / dv);
  const int c0 = (int)(gid % dv) * 4;
  auto row = [&](long long r, f32x4 (&v)[NV]) {
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] = *(const f32x4*)(y_exp + r * d + c0 + j * dv * 4);
    for (int p = 0; p < nparts; ++p) {
#pragma unroll
      for (int j = 0; j < NV; ++j)
        v[j] += *(const f32x4*)(y_part + p * part_elems + r * d + c0 + j * dv * 4);
    }
  };
  f32x4 acc[NV] = {};
  f32x4 v[NV];
  for (int e = 0; e < E; ++e) {
    const int r = row_of[(long long)t * E + e];
    if (r >= 0) {
      const float w = probs[(long long)t * E + e];
      row(r, v);
#pragma unroll
      for (int j = 0; j < NV; ++j) acc[j] += w * v[j];
    }
  }
  if (S > 0) {
    const long long base = offsets[E];
    for (int q = 0; q < S; ++q) {
      row(base + (long long)q * T + t, v);
#pragma unroll
      for (int j = 0; j < NV; ++j) acc[j] += v[j];
    }
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) *(f32x4*)(y + (long long)t * d + c0 + j * dv * 4) = acc[j];
}

}  // namespace

hipError_t launch_expert_choice(const Shape& s, const float* probs, int32_t* sorted_assign,
                                int32_t* row_of, int32_t* counts, int32_t* kept,
                                int32_t* offsets, float* colsum, hipStream_t st) {
  ec_select_kernel<<<s.E, ET, 0, st>>>(probs, s.T, s.E, s.cap, sorted_assign, row_of, counts, kept,
                                       offsets, colsum);
  return hipGetLastError();
}

hipError_t launch_token_experts(const Shape& s, const int32_t* row_of, int32_t* token_experts,
                                hipStream_t st) {
  token_experts_kernel<<<(s.T + 255) / 256, 256, 0, st>>>(row_of, s.T, s.E, token_experts);
  return hipGetLastError();
}

hipError_t launch_combine_ec(const Shape& s, const float* probs, const int32_t* row_of,
                             const int32_t* offsets, const float* y_exp, const float* y_part,
                             int nparts, float* y, hipStream_t st) {
  if (s.d % 16 == 0 && s.d >= 256) {
    const long long n = (long long)s.T * (s.d / 16);
    combine_ec_kernel<4><<<(int)((n + 255) / 256), 256, 0, st>>>(
        probs, row_of, offsets, y_exp, y_part, nparts, s.max_rows() * s.d, y, s.T, s.d, s.E, s.S);
  } else {
    const long long n = (long long)s.T * (s.d / 4);
    combine_ec_kernel<1><<<(int)((n + 255) / 256), 256, 0, st>>>(
        probs, row_of, offsets, y_exp, y_part, nparts, s.max_rows() * s.d, y, s.T, s.d, s.E, s.S);
  }
  return hipGetLastError();
}

}  // namespace moe
