// Expert FFNs for decode-sized batches (T <= 16): the sparse GEMV regime.
//
// Each expert sees at most T <= 16 rows, so the work is a stream of the
// touched experts' weights through the matrix cores with the (few) token
// rows as the 16-wide MFMA operand: bf16 MFMA 16x16x32 for the up
// projection, fp16 MFMA 16x16x32 for the down projection (W2 converted to
// fp16 in registers).  The weights are read from HBM exactly once; experts
// with no rows are skipped without reading their weights.  One wave is one
// work item; its loads of consecutive K steps are independent, so many are
// in flight per wave.
//
// Up:   wave = (segment, 16 output columns of h); for SwiGLU its two MFMA
//       "A" fragments are the gate rows and the matching up rows, otherwise
//       two groups of 16 rows of W1 (32 output columns).
// Down: wave = (segment, 32 output columns, one of nsplit slices of K); the
//       slice partials are summed in a fixed order by a reduction kernel.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int WAVES = 4;   // waves per block
constexpr int UNROLL = 8;  // K steps whose loads are issued together

__device__ __forceinline__ void seg_info(const int32_t* offsets, int seg, int E, int T, int& rows,
                                         int& start) {
  if (seg < E) {
    start = offsets[seg];
    rows = offsets[seg + 1] - start;
  } else {
    start = offsets[E] + (seg - E) * T;
    rows = T;
  }
}

template <int ACT>  // MOE_RELU / MOE_GELU / MOE_SWIGLU
__global__ __launch_bounds__(64 * WAVES) void decode_up_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w_up,
    const uint16_t* __restrict__ b_up, _Float16* __restrict__ h, const int32_t* offsets,
    const int32_t* sorted_assign, int T, int k, int E, int S, int d, int f, int items_per_seg) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * WAVES + (threadIdx.x >> 6);
  const int seg = item / items_per_seg;
  const int it = item % items_per_seg;
  if (seg >= E + S) return;
  int rows, start;
  seg_info(offsets, seg, E, T, rows, start);
  if (rows <= 0) return;

  const int F1 = ACT == MOE_SWIGLU ? 2 * f : f;
  const int r0 = ACT == MOE_SWIGLU ? 16 * it : 32 * it;
  const int r1 = ACT == MOE_SWIGLU ? f + 16 * it : 32 * it + 16;
  const int kg = lane >> 4;  // k group of 8
  const uint16_t* a0 = w_up + ((long long)seg * F1 + r0 + (lane & 15)) * d + kg * 8;
  const uint16_t* a1 = w_up + ((long long)seg * F1 + r1 + (lane & 15)) * d + kg * 8;
  const int tl = lane & 15;  // token of this lane's B fragment
  const bool tvalid = tl < rows;
  long long tok = 0;
  if (tvalid) tok = seg < E ? sorted_assign[start + tl] / k : tl;
  const uint16_t* bp = x + tok * d + kg * 8;

  f32x4 acc0 = {}, acc1 = {};
  const int nsteps = d / 32;
  auto step = [&](const u32x4& va0, const u32x4& va1, u32x4 vb) {
    if (!tvalid) vb = u32x4{0u, 0u, 0u, 0u};
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va0),
                                                   __builtin_bit_cast(bf16x8, vb), acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va1),
                                                   __builtin_bit_cast(bf16x8, vb), acc1, 0, 0, 0);
  };
  int s = 0;
  for (; s + UNROLL <= nsteps; s += UNROLL) {   // UNROLL steps of loads in flight
    u32x4 va0[UNROLL], va1[UNROLL], vb[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      va0[u] = *(const u32x4*)(a0 + (s + u) * 32);
      va1[u] = *(const u32x4*)(a1 + (s + u) * 32);
      vb[u] = *(const u32x4*)(bp + (s + u) * 32);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) step(va0[u], va1[u], vb[u]);
  }
  for (; s < nsteps; ++s)
    step(*(const u32x4*)(a0 + s * 32), *(const u32x4*)(a1 + s * 32), *(const u32x4*)(bp + s * 32));
  if (!tvalid) return;
  // D[n][token]: lane holds token lane & 15 and rows 4*(lane>>4) + 0..3.
  const int nb = 4 * (lane >> 4);
  _Float16* hrow = h + (long long)(start + tl) * f;
  if (ACT == MOE_SWIGLU) {
    f16x4 v;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = (_Float16)(silu_f(acc0[r]) * acc1[r]);
    *(f16x4*)(hrow + 16 * it + nb) = v;
  } else {
    f16x4 v0, v1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float z0 = acc0[r], z1 = acc1[r];
      if (b_up) {
        z0 += bf16_to_f32(b_up[(long long)seg * F1 + r0 + nb + r]);
        z1 += bf16_to_f32(b_up[(long long)seg * F1 + r1 + nb + r]);
      }
      v0[r] = (_Float16)(ACT == MOE_RELU ? fmaxf(z0, 0.f) : gelu_f(z0));
      v1[r] = (_Float16)(ACT == MOE_RELU ? fmaxf(z1, 0.f) : gelu_f(z1));
    }
    *(f16x4*)(hrow + r0 + nb) = v0;
    *(f16x4*)(hrow + r1 + nb) = v1;
  }
}

__global__ __launch_bounds__(64 * WAVES) void decode_down_kernel(
    const _Float16* __restrict__ h, const uint16_t* __restrict__ w_down, float* __restrict__ y_part,
    const int32_t* offsets, int T, int E, int S, int d, int f, int nsplit, long long part_stride,
    int items_per_seg) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * WAVES + (threadIdx.x >> 6);
  const int seg = item / items_per_seg;
  const int rem = item % items_per_seg;
  const int nt = rem / nsplit, ks = rem % nsplit;
  if (seg >= E + S) return;
  int rows, start;
  seg_info(offsets, seg, E, T, rows, start);
  if (rows <= 0) return;

  const int kg = lane >> 4;
  const int klen = f / nsplit;  // a multiple of 32
  const int k0 = ks * klen;
  const uint16_t* a0 = w_down + ((long long)seg * d + 32 * nt + (lane & 15)) * f + k0 + kg * 8;
  const uint16_t* a1 = a0 + 16LL * f;
  const int tl = lane & 15;
  const bool tvalid = tl < rows;
  const _Float16* bp = h + (long long)(start + (tvalid ? tl : 0)) * f + k0 + kg * 8;

  f32x4 acc0 = {}, acc1 = {};
  const int nsteps = klen / 32;
  auto step = [&](const u32x4& wa0, const u32x4& wa1, u32x4 vb) {
    const u32x4 va0 = bf16x8_to_f16x8(wa0);
    const u32x4 va1 = bf16x8_to_f16x8(wa1);
    if (!tvalid) vb = u32x4{0u, 0u, 0u, 0u};
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, va0),
                                                  __builtin_bit_cast(f16x8, vb), acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, va1),
                                                  __builtin_bit_cast(f16x8, vb), acc1, 0, 0, 0);
  };
  int s = 0;
  for (; s + UNROLL <= nsteps; s += UNROLL) {
    u32x4 va0[UNROLL], va1[UNROLL], vb[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      va0[u] = *(const u32x4*)(a0 + (s + u) * 32);
      va1[u] = *(const u32x4*)(a1 + (s + u) * 32);
      vb[u] = *(const u32x4*)(bp + (s + u) * 32);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) step(va0[u], va1[u], vb[u]);
  }
  for (; s < nsteps; ++s)
    step(*(const u32x4*)(a0 + s * 32), *(const u32x4*)(a1 + s * 32), *(const u32x4*)(bp + s * 32));
  if (!tvalid) return;
  const int nb = 4 * (lane >> 4);
  float* out = y_part + ks * part_stride + (long long)(start + tl) * d + 32 * nt + nb;
  *(f32x4*)out = acc0;
  *(f32x4*)(out + 16) = acc1;
}

// y_exp[r, :] = sum over the K slices (in order) of y_part + b2.
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ y_part,
                                                           const uint16_t* __restrict__ b_down,
                                                           float* __restrict__ y_exp,
                                                           const int32_t* offsets, int T, int E,
                                                           int S, int d, int nsplit,
                                                           long long part_stride) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int d4 = d / 4;
  const long long r = gid / d4;
  const int c = (int)(gid % d4) * 4;
  const int off_E = offsets[E];
  if (r >= (long long)off_E + (long long)S * T) return;
  f32x4 acc = *(const f32x4*)(y_part + r * d + c);
  for (int ks = 1; ks < nsplit; ++ks) acc += *(const f32x4*)(y_part + ks * part_stride + r * d + c);
  if (b_down) {
    int seg;
    if (r < off_E) {
      int lo = 0, hi = E;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offsets[mid] <= r) lo = mid; else hi = mid;
      }
      seg = lo;
    } else {
      seg = E + (int)((r - off_E) / T);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += bf16_to_f32(b_down[(long long)seg * d + c + i]);
  }
  *(f32x4*)(y_exp + r * d + c) = acc;
}

}  // namespace

hipError_t launch_decode_up(const Shape& s, const void* x, const void* w_up, const void* b_up,
                            const int32_t* offsets, const int32_t* sorted_assign, void* h,
                            hipStream_t st) {
  const int nseg = s.E + s.S;
  const int items_per_seg = s.act == MOE_SWIGLU ? s.f / 16 : s.f / 32;
  const long long items = (long long)nseg * items_per_seg;
  const int blocks = (int)((items + WAVES - 1) / WAVES);
  const uint16_t* b = s.expert_bias() ? (const uint16_t*)b_up : nullptr;
#define MOE_DECODE_UP(A)                                                                        \
  decode_up_kernel<A><<<blocks, 64 * WAVES, 0, st>>>((const uint16_t*)x, (const uint16_t*)w_up, \
                                                      b, (_Float16*)h, offsets, sorted_assign,  \
                                                      s.T, s.k, s.E, s.S, s.d, s.f,             \
                                                      items_per_seg)
  if (s.act == MOE_SWIGLU) MOE_DECODE_UP(MOE_SWIGLU);
  else if (s.act == MOE_GELU) MOE_DECODE_UP(MOE_GELU);
  else MOE_DECODE_UP(MOE_RELU);
#undef MOE_DECODE_UP
  return hipGetLastError();
}

hipError_t launch_decode_down(const Shape& s, const void* h, const void* w_down,
                              const void* b_down, const int32_t* offsets, float* y_exp,
                              float* y_part, hipStream_t st) {
  const int nseg = s.E + s.S;
  // K slices of a multiple of 32 (f is a multiple of 64)
  const int nsplit = (s.f % (32 * kDecodeSplitK) == 0) ? kDecodeSplitK : 2;
  const int items_per_seg = (s.d / 32) * nsplit;
  const long long items = (long long)nseg * items_per_seg;
  const int blocks = (int)((items + WAVES - 1) / WAVES);
  const long long part_stride = s.max_rows() * s.d;
  decode_down_kernel<<<blocks, 64 * WAVES, 0, st>>>((const _Float16*)h, (const uint16_t*)w_down,
                                                    y_part, offsets, s.T, s.E, s.S, s.d, s.f,
                                                    nsplit, part_stride, items_per_seg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n = s.max_rows() * (s.d / 4);
  const uint16_t* b = s.expert_bias() ? (const uint16_t*)b_down : nullptr;
  split_reduce_kernel<<<(int)((n + 255) / 256), 256, 0, st>>>(y_part, b, y_exp, offsets, s.T, s.E,
                                                             s.S, s.d, nsplit, part_stride);
  return hipGetLastError();
}

}  // namespace moe
