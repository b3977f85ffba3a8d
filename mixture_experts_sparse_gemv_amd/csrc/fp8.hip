// Per-row FP8 E4M3 quantization of expert weights ("MoE混合专家模型" 5.2:
// quantizing the expert parameters to 8 bits halves their memory and the
// bytes a decode step streams).
//
// Row r of a [rows, cols] bf16 matrix gets the scale s = max_j |w| / 448
// (1 for an all-zero row); each value w / s (float32, correctly rounded) is
// rounded to the nearest OCP E4M3 value, ties to the even code, magnitudes
// above 448 saturating to 448.  The dequantized weight is code_value * s.
// A one-time preparation step, not part of the forward.
#include "moe_internal.h"

namespace moe {
namespace {

// Nearest E4M3 code of v (sign in bit 7).  Below 2^-6 the values are the
// multiples of 2^-9; above, 3 mantissa bits: round the float32 mantissa to 3
// bits (ties to even), which can carry into the exponent.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = v < 0.0f ? 0x80u : 0u;
  const float a = fminf(fabsf(v), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.0f);   // 0 .. 8 (8 is 2^-6, the first normal)
  } else {
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    code = ((((b >> 23) & 0xFFu) - 120u) << 3) | ((b >> 20) & 7u);
  }
  return sign | code;
}

__global__ __launch_bounds__(256) void quantize_fp8_kernel(const uint16_t* __restrict__ w,
                                                           int cols, uint8_t* __restrict__ q,
                                                           float* __restrict__ scales) {
  __shared__ float wmax[4];
  const long long r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint16_t* wr = w + r * cols;
  float amax = 0.0f;
  for (int j = tid; j < cols; j += 256) amax = fmaxf(amax, fabsf(bf16_to_f32(wr[j])));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if (lane == 0) wmax[wave] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  if (tid == 0) scales[r] = s;
  uint8_t* qr = q + r * cols;
  for (int j = tid; j < cols; j += 256) qr[j] = (uint8_t)e4m3_code(__fdiv_rn(bf16_to_f32(wr[j]), s));
}

}  // namespace

hipError_t launch_quantize_fp8(const void* w, long long rows, int cols, uint8_t* q, float* scales,
                               hipStream_t st) {
  quantize_fp8_kernel<<<(unsigned)rows, 256, 0, st>>>((const uint16_t*)w, cols, q, scales);
  return hipGetLastError();
}

}  // namespace moe
