// Gate-weighted combine (0539edu 1.3 and 2.1; kamacoder 五; shared experts:
// "MoE架构解析" 四 技术飞跃②):
//   y[t] = sum over kept slots s of w[t, s] * y_exp[assign_row[t*k+s]]
//          + sum over shared experts q of y_exp[offsets[E] + q*T + t]
// One thread per NV groups of 4 consecutive outputs of a token (16-byte
// loads and stores; group j of thread i starts at column 4 (i + j d / (4 NV)),
// so each load instruction of a wave reads contiguous bytes, and a thread has
// NV loads per row in flight behind one read of the token's slots); the sum
// runs in slot order, then shared-expert order, so the result does not
// depend on scheduling.  Every element of y is written.
// When the down projection ran in K slices, a row of y_exp is its slice-0
// value plus the other slices' partials, added here in slice order.
#include "moe_internal.h"

namespace moe {
namespace {

template <int VEC, int NV>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ topk_w,
                                                      const int32_t* __restrict__ assign_row,
                                                      const int32_t* __restrict__ offsets,
                                                      const float* __restrict__ y_exp,
                                                      const float* __restrict__ y_part,
                                                      int nparts, long long part_elems,
                                                      float* __restrict__ y, int T, int d, int k,
                                                      int E, int S) {
  const int dv = d / (VEC * NV);   // threads per token
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)T * dv) return;
  const int t = (int)(gid / dv);
  const int c0 = (int)(gid % dv) * VEC;
  typedef float vec_t __attribute__((ext_vector_type(VEC)));
  // row value of group j: y_exp plus the K-slice partials, in slice order
  auto row = [&](long long r, vec_t (&v)[NV]) {
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] = *(const vec_t*)(y_exp + r * d + c0 + j * dv * VEC);
    for (int p = 0; p < nparts; ++p) {
#pragma unroll
      for (int j = 0; j < NV; ++j)
        v[j] += *(const vec_t*)(y_part + p * part_elems + r * d + c0 + j * dv * VEC);
    }
  };
  vec_t acc[NV] = {};
  vec_t v[NV];
  for (int s = 0; s < k; ++s) {
    const int r = assign_row[(long long)t * k + s];
    if (r >= 0) {
      const float w = topk_w[(long long)t * k + s];
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
  for (int j = 0; j < NV; ++j) *(vec_t*)(y + (long long)t * d + c0 + j * dv * VEC) = acc[j];
}

}  // namespace

hipError_t launch_combine(const Shape& s, const float* topk_w, const int32_t* assign_row,
                          const int32_t* offsets, const float* y_exp, const float* y_part,
                          int nparts, float* y, hipStream_t st) {
  const long long part_elems = s.max_rows() * s.d;
  if (s.d % 16 == 0 && s.d >= 256) {
    const long long n = (long long)s.T * (s.d / 16);
    combine_kernel<4, 4><<<(int)((n + 255) / 256), 256, 0, st>>>(
        topk_w, assign_row, offsets, y_exp, y_part, nparts, part_elems, y, s.T, s.d, s.k, s.E, s.S);
  } else if (s.d % 4 == 0) {
    const long long n = (long long)s.T * (s.d / 4);
    combine_kernel<4, 1><<<(int)((n + 255) / 256), 256, 0, st>>>(
        topk_w, assign_row, offsets, y_exp, y_part, nparts, part_elems, y, s.T, s.d, s.k, s.E, s.S);
  } else {
    const long long n = (long long)s.T * s.d;
    combine_kernel<1, 1><<<(int)((n + 255) / 256), 256, 0, st>>>(
        topk_w, assign_row, offsets, y_exp, y_part, nparts, part_elems, y, s.T, s.d, s.k, s.E, s.S);
  }
  return hipGetLastError();
}

}  // namespace moe
