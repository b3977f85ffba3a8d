// Grouped expert GEMMs for bf16 layers whose d_model or d_ff is a multiple of
// 8 but not of 64 (the tiled kernels stream whole 64-element rows).
//
// The same products as the tiled grouped GEMM (kamacoder 四; 0539edu 4.1;
// learn-minimind 二):
//   up:   h[r, n] = act(sum_j x[tok(r), j] W1_e[n, j] + b1_e[n]), or for SwiGLU
//         silu(sum_j x Wg_e[n, j]) * (sum_j x Wu_e[n, j]); h stored in fp16
//         scaled by 2^-8
//   down: y_exp[r, n] = 2^8 sum_j h[r, j] W2_e[n, j] + b2_e[n]
// over the routed segments (token rows gathered through sorted_assign) and
// the shared segments (every token).
//
// A block computes 64 rows x 64 output columns of one segment with 4 waves
// of 32 x 32 (MFMA 32x32x16: bf16 for the up projection, fp16 with W2
// converted for the down projection).  Each lane loads its fragments straight
// from global memory, 16 bytes of one row per 16-deep k-step: the reduction
// length is a multiple of 8, so a lane's 8 elements lie wholly inside the row
// or wholly past its end, and those past it are zero.  Rows past a segment's
// end and columns past the output width read a valid row and are not stored.
// This is the path for uncommon widths, kept simple: no LDS staging.
#include "moe_internal.h"

namespace moe {
namespace {

enum { GEN_RELU = 0, GEN_GELU = 1, GEN_SWIGLU = 2, GEN_DOWN = 3 };

struct GenArgs {
  const uint16_t* X;       // up: x [T, K] bf16; down: h [rows, K] fp16 (scaled 2^-8)
  const uint16_t* W;       // [segments][Wrows][K] bf16
  const uint16_t* bias;    // [segments][Wrows] bf16, or null
  void* out;               // up: h [rows, Nout] fp16; down: y_exp [rows, Nout] fp32
  const int32_t* offsets;  // [E + 1]
  const int32_t* sorted_assign;
  int T, k, E, S, K, Nout, Wrows, f;
};

template <int MODE>
__global__ __launch_bounds__(256) void gemm_generic_kernel(GenArgs a) {
  constexpr int BM = 64, BN = 64;
  constexpr bool SWIGLU = MODE == GEN_SWIGLU, DOWN = MODE == GEN_DOWN;
  constexpr int NACC = SWIGLU ? 2 : 1;   // SwiGLU: gate and up rows of the same columns
  __shared__ int seg_tile[kMaxSegments + 1], seg_rows[kMaxSegments], seg_row0[kMaxSegments];
  __shared__ int sh_tile[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nseg = a.E + a.S;

  // segments' rows, first rows and 64-row tiles, prefix summed by wave 0
  if (wave == 0) {
    const int off_E = a.offsets[a.E];
    int c[2] = {0, 0};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int sg = 2 * lane + u;
      if (sg < nseg) {
        int r0, r;
        if (sg < a.E) {
          r0 = a.offsets[sg];
          r = a.offsets[sg + 1] - r0;
        } else {
          r0 = off_E + (sg - a.E) * a.T;
          r = a.T;
        }
        seg_rows[sg] = r;
        seg_row0[sg] = r0;
        c[u] = (r + BM - 1) / BM;
      }
    }
    const int v = c[0] + c[1];
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    const int excl = incl - v;
    if (2 * lane < nseg) seg_tile[2 * lane] = excl;
    if (2 * lane + 1 < nseg) seg_tile[2 * lane + 1] = excl + c[0];
    if (lane == 63) seg_tile[nseg] = incl;
  }
  __syncthreads();
  const int L = blockIdx.x;
  if (L >= seg_tile[nseg]) return;   // uniform: the grid covers an upper bound of the tiles
  if (tid < nseg && seg_tile[tid] <= L && L < seg_tile[tid + 1]) {
    sh_tile[0] = tid;
    sh_tile[1] = L - seg_tile[tid];
  }
  __syncthreads();
  const int seg = sh_tile[0], mt = sh_tile[1];
  const int rows = seg_rows[seg], row0 = seg_row0[seg];
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.y * BN + wn * 32;     // first output column of the wave
  const int m0 = mt * BM + wm * 32;             // first row (within the segment) of the wave

  // this lane's token row (B operand column) and weight rows (A operand rows)
  const int ml = m0 + (lane & 31);
  const int mc = ml < rows ? ml : rows - 1;
  long long xrow;
  if (DOWN) xrow = (long long)(row0 + mc);
  else xrow = (seg < a.E) ? (long long)(a.sorted_assign[row0 + mc] / a.k) : (long long)mc;
  const uint16_t* xp = a.X + xrow * a.K;
  const int nl = n0 + (lane & 31);
  const int nc = nl < a.Nout ? nl : a.Nout - 1;
  const uint16_t* wp[NACC];
  wp[0] = a.W + ((long long)seg * a.Wrows + nc) * a.K;
  if (SWIGLU) wp[NACC - 1] = a.W + ((long long)seg * a.Wrows + a.f + nc) * a.K;

  f32x16 acc[NACC];
#pragma unroll
  for (int q = 0; q < NACC; ++q) acc[q] = f32x16{};
  const int kl = 8 * (lane >> 5);   // this lane's 8 elements of a 16-deep k-step
  for (int k0 = 0; k0 < a.K; k0 += 16) {
    const bool in = k0 + kl < a.K;
    const u32x4 xv = in ? *(const u32x4*)(xp + k0 + kl) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int q = 0; q < NACC; ++q) {
      const u32x4 wv = in ? *(const u32x4*)(wp[q] + k0 + kl) : u32x4{0, 0, 0, 0};
      if (DOWN)
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
            __builtin_bit_cast(f16x8, bf16x8_to_f16x8(wv)), __builtin_bit_cast(f16x8, xv), acc[q],
            0, 0, 0);
      else
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, wv), __builtin_bit_cast(bf16x8, xv), acc[q], 0, 0, 0);
    }
  }

  // D[weight row][token]: lane holds token row m0 + (lane & 31) and, in
  // register group g, the 4 consecutive columns n0 + 8g + 4 (lane >> 5) + 0..3
  if (ml >= rows) return;
  const long long orow = row0 + ml;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int col = n0 + 8 * g + 4 * (lane >> 5);
    if (col >= a.Nout) continue;   // Nout is a multiple of 8: 4 columns in or out together
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = acc[0][4 * g + r];
    if (SWIGLU) {
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = silu_f(v[r]) * acc[NACC - 1][4 * g + r];
    } else {
      if (DOWN) {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] *= kHLoadScale;   // h was stored scaled by 2^-8
      }
      if (a.bias) {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] += bf16_to_f32(a.bias[(long long)seg * a.Wrows + col + r]);
      }
    }
    if (DOWN) {
      *(f32x4*)((float*)a.out + orow * a.Nout + col) = f32x4{v[0], v[1], v[2], v[3]};
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (MODE == GEN_RELU) v[r] = fmaxf(v[r], 0.0f);
        if (MODE == GEN_GELU) v[r] = gelu_f(v[r]);
      }
      *(f16x4*)((_Float16*)a.out + orow * a.Nout + col) =
          f16x4{h_to_f16(v[0]), h_to_f16(v[1]), h_to_f16(v[2]), h_to_f16(v[3])};
    }
  }
}

// An upper bound of the 64-row tiles of all segments: every routed segment
// adds at most one partial tile.
int generic_tiles(const Shape& s) {
  return (int)((s.routed_rows() + 63) / 64 + s.E + (long long)s.S * ((s.T + 63) / 64));
}

}  // namespace

hipError_t launch_up_generic(const Shape& s, const void* x, const void* w_up, const void* b_up,
                             const int32_t* offsets, const int32_t* sorted_assign, void* h,
                             hipStream_t st) {
  GenArgs a{(const uint16_t*)x, (const uint16_t*)w_up,
            s.expert_bias() ? (const uint16_t*)b_up : nullptr, h, offsets, sorted_assign, s.T,
            s.tok_div(), s.E, s.S, s.d, s.f, s.up_rows(), s.f};
  const dim3 grid(generic_tiles(s), (s.f + 63) / 64);
  if (s.act == MOE_SWIGLU) gemm_generic_kernel<GEN_SWIGLU><<<grid, 256, 0, st>>>(a);
  else if (s.act == MOE_GELU) gemm_generic_kernel<GEN_GELU><<<grid, 256, 0, st>>>(a);
  else gemm_generic_kernel<GEN_RELU><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_down_generic(const Shape& s, const void* h, const void* w_down,
                               const void* b_down, const int32_t* offsets, float* y_exp,
                               hipStream_t st) {
  GenArgs a{(const uint16_t*)h, (const uint16_t*)w_down,
            s.expert_bias() ? (const uint16_t*)b_down : nullptr, y_exp, offsets, nullptr, s.T,
            s.tok_div(), s.E, s.S, s.f, s.d, s.d, s.f};
  const dim3 grid(generic_tiles(s), (s.d + 63) / 64);
  gemm_generic_kernel<GEN_DOWN><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace moe
