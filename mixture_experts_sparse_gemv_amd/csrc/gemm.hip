// Grouped expert GEMMs over the variable-length expert segments.
//
// Up projection  (kamacoder 四; 0539edu 4.1; learn-minimind 二):
//   h[r, n] = act(sum_j x[tok(r), j] * W1_e[n, j] + b1_e[n])        ReLU / GELU
//   h[r, n] = silu(sum_j x Wg_e[n, j]) * (sum_j x Wu_e[n, j])       SwiGLU
// Down projection:
//   y_exp[r, n] = sum_j h[r, j] * W2_e[n, j] + b2_e[n]
// where row r belongs to expert e (offsets[e] <= r < offsets[e+1], token
// sorted_assign[r] / k) or to a shared expert (token r - segment start).
//
// Dense contractions, so they run on the matrix cores: bf16 MFMA 32x32x16
// for the up projection, fp16 MFMA 32x32x16 for the down projection (h is
// fp16; each bf16 W2 tile is converted to fp16 while it is staged into LDS).
// Accumulation is fp32.  Block = 4 waves in a 2x2 grid; block tile BM token
// rows x BN weight rows x BK=64; tiles are double-buffered in LDS with an XOR
// swizzle of the 16-byte chunks (chunk ^ row%8) so that the fragment reads of
// 32 consecutive rows spread over all banks.  The MFMA "A" operand is the
// weight tile and "B" the token tile, so each lane's accumulator holds four
// consecutive output columns of one token row: the epilogue stores 8-byte
// (fp16 x4) or 16-byte (fp32 x4) vectors.
//
// The tile schedule is computed on the device from offsets[] (no host sync):
// every block derives the per-segment m-tile counts, their prefix sum, and its
// own (segment, n-tile, m-tile).  Block ids are remapped so that each of the 8
// XCDs (block b runs on XCD b % 8) gets a contiguous range of tiles: the tiles
// of one expert weight stay within one XCD's L2.
#include "moe_internal.h"

namespace moe {
namespace {

enum { MODE_RELU = 0, MODE_GELU = 1, MODE_SWIGLU = 2, MODE_DOWN = 3 };

struct GemmArgs {
  const uint16_t* X;       // up: x [T, K] bf16; down: h [rows, K] fp16
  const uint16_t* W;       // [segments][Wrows][K] bf16
  const uint16_t* bias;    // [segments][Wrows] bf16, or null
  void* out;               // up: h [rows, Nout] fp16; down: y_exp [rows, Nout] fp32
  const int32_t* offsets;  // [E + 1]
  const int32_t* sorted_assign;
  int T, k, E, S, K, Nout, Wrows, f;
};

// Per-segment row count and first row.
__device__ __forceinline__ void segment_rows(const GemmArgs& a, int seg, int off_E, int& rows,
                                             int& start) {
  if (seg < a.E) {
    start = a.offsets[seg];
    rows = a.offsets[seg + 1] - start;
  } else {
    start = off_E + (seg - a.E) * a.T;
    rows = a.T;
  }
}

template <int BM, int BN, int MODE>
__global__ __launch_bounds__(256, 1) void grouped_gemm_kernel(GemmArgs a) {
  constexpr int BK = 64;
  constexpr bool SWIGLU = MODE == MODE_SWIGLU;
  constexpr bool DOWN = MODE == MODE_DOWN;
  constexpr int WM = BM / 2, WN = BN / 2;  // wave tile: token rows x weight rows
  constexpr int MI = WM / 32, NI = WN / 32;
  constexpr int NOUT_TILE = SWIGLU ? BN / 2 : BN;
  constexpr int XCH = BM / 32, WCH = BN / 32;  // 16-byte chunks per thread per k-tile
  static_assert(!SWIGLU || (NI % 2 == 0), "SwiGLU pairs gate and up sub-tiles");

  __shared__ u32x4 smem[2][(BM + BN) * 8];
  __shared__ int seg_tile[kMaxSegments + 1];
  __shared__ int sh_seg;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int nseg = a.E + a.S;
  const int NT = (a.Nout + NOUT_TILE - 1) / NOUT_TILE;
  const int off_E = a.offsets[a.E];

  // ---- tile schedule: prefix sum of m-tiles per segment (wave 0, 2 segments per lane)
  if (wave == 0) {
    int c0 = 0, c1 = 0, r, st;
    const int s0 = 2 * lane, s1 = 2 * lane + 1;
    if (s0 < nseg) { segment_rows(a, s0, off_E, r, st); c0 = (r + BM - 1) / BM; }
    if (s1 < nseg) { segment_rows(a, s1, off_E, r, st); c1 = (r + BM - 1) / BM; }
    int v = c0 + c1, incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      int u = __shfl_up(incl, o);
      if (lane >= o) incl += u;
    }
    const int excl = incl - v;
    if (s0 < nseg) seg_tile[s0] = excl;
    if (s1 < nseg) seg_tile[s1] = excl + c0;
    if (lane == 63) seg_tile[nseg] = incl;
  }
  __syncthreads();
  const int total = seg_tile[nseg] * NT;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per = (total + 7) >> 3;
  const int L = xcd * per + slot;
  if (slot >= per || L >= total) return;  // uniform over the block
  if (tid < nseg && seg_tile[tid] * NT <= L && L < seg_tile[tid + 1] * NT) sh_seg = tid;
  __syncthreads();
  const int seg = sh_seg;
  const int mtiles = seg_tile[seg + 1] - seg_tile[seg];
  const int local = L - seg_tile[seg] * NT;
  const int nt = local / mtiles, mt = local % mtiles;
  int seg_rows, row_start;
  segment_rows(a, seg, off_E, seg_rows, row_start);

  // ---- global source rows of this thread's chunks
  const int kc_ld = tid & 7;
  const uint16_t* xsrc[XCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int m = mt * BM + (tid >> 3) + 32 * i;
    const int mm = m < seg_rows ? m : seg_rows - 1;
    long long row;
    if (DOWN) {
      row = row_start + mm;
    } else {
      row = seg < a.E ? a.sorted_assign[row_start + mm] / a.k : mm;
    }
    xsrc[i] = a.X + row * a.K + kc_ld * 8;
  }
  const uint16_t* wsrc[WCH];
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    const int rho = (tid >> 3) + 32 * i;
    int wr;
    if (SWIGLU) {
      const int half = BN / 2;
      const int nn = nt * half + (rho < half ? rho : rho - half);
      const int nc = nn < a.f ? nn : a.f - 1;
      wr = rho < half ? nc : a.f + nc;
    } else {
      const int nn = nt * BN + rho;
      wr = nn < a.Wrows ? nn : a.Wrows - 1;
    }
    wsrc[i] = a.W + ((long long)seg * a.Wrows + wr) * a.K + kc_ld * 8;
  }

  u32x4 xr[XCH], wreg[WCH];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) wreg[i] = *(const u32x4*)(wsrc[i] + kt * BK);
#pragma unroll
    for (int i = 0; i < XCH; ++i) xr[i] = *(const u32x4*)(xsrc[i] + kt * BK);
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int rho = (tid >> 3) + 32 * i;
      smem[buf][rho * 8 + (kc_ld ^ (rho & 7))] = DOWN ? bf16x8_to_f16x8(wreg[i]) : wreg[i];
    }
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int rho = (tid >> 3) + 32 * i;
      smem[buf][BN * 8 + rho * 8 + (kc_ld ^ (rho & 7))] = xr[i];
    }
  };

  // LDS rows of this wave's fragments
  int wrow[NI], xrow[MI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    if (SWIGLU) {
      const int jj = j < NI / 2 ? j : j - NI / 2;
      wrow[j] = (j < NI / 2 ? 0 : BN / 2) + wn * (BN / 4) + jj * 32 + (lane & 31);
    } else {
      wrow[j] = wn * WN + j * 32 + (lane & 31);
    }
  }
#pragma unroll
  for (int i = 0; i < MI; ++i) xrow[i] = wm * WM + i * 32 + (lane & 31);

  f32x16 acc[NI][MI];
#pragma unroll
  for (int j = 0; j < NI; ++j)
#pragma unroll
    for (int i = 0; i < MI; ++i) acc[j][i] = f32x16{};

  const int nk = a.K / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tile(kt + 1);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int kc = 2 * s + (lane >> 5);
      u32x4 wf[NI], xf[MI];
#pragma unroll
      for (int j = 0; j < NI; ++j) wf[j] = smem[cur][wrow[j] * 8 + (kc ^ (wrow[j] & 7))];
#pragma unroll
      for (int i = 0; i < MI; ++i) xf[i] = smem[cur][BN * 8 + xrow[i] * 8 + (kc ^ (xrow[i] & 7))];
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          if (DOWN)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8, wf[j]), __builtin_bit_cast(f16x8, xf[i]), acc[j][i], 0, 0, 0);
          else
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, wf[j]), __builtin_bit_cast(bf16x8, xf[i]), acc[j][i], 0, 0, 0);
        }
    }
    if (kt + 1 < nk) store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds token row (lane & 31) of each 32x32 tile and, in
  // register group g, the four consecutive weight rows 8g + 4*(lane>>5) + 0..3.
  constexpr int NJ = SWIGLU ? NI / 2 : NI;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int m = mt * BM + wm * WM + i * 32 + (lane & 31);
      const bool valid = m < seg_rows;
      const long long orow = (long long)row_start + m;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nloc = j * 32 + 8 * g + 4 * (lane >> 5);
        const int col = SWIGLU ? nt * (BN / 2) + wn * (BN / 4) + nloc : nt * BN + wn * WN + nloc;
        if (!valid || col >= a.Nout) continue;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[j][i][4 * g + r];
        if (SWIGLU) {
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = silu_f(v[r]) * acc[j + NI / 2][i][4 * g + r];
        } else if (a.bias) {
          const u32x2 b = *(const u32x2*)(a.bias + (long long)seg * a.Wrows + col);
          v[0] += __uint_as_float(b[0] << 16);
          v[1] += __uint_as_float(b[0] & 0xffff0000u);
          v[2] += __uint_as_float(b[1] << 16);
          v[3] += __uint_as_float(b[1] & 0xffff0000u);
        }
        if (DOWN) {
          *(f32x4*)((float*)a.out + orow * a.Nout + col) = f32x4{v[0], v[1], v[2], v[3]};
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (MODE == MODE_RELU) v[r] = fmaxf(v[r], 0.0f);
            if (MODE == MODE_GELU) v[r] = gelu_f(v[r]);
          }
          f16x4 hv = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
          *(f16x4*)((_Float16*)a.out + orow * a.Nout + col) = hv;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- fp32 path
// One thread per output element; used for float32 problems (small layers).
template <int MODE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* X, const float* W,
                                                       const float* bias, float* out,
                                                       const int32_t* offsets,
                                                       const int32_t* sorted_assign, int T, int k,
                                                       int E, int S, int K, int Nout, int Wrows,
                                                       int f) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long r = gid / Nout;
  const int n = (int)(gid % Nout);
  const int off_E = offsets[E];
  if (r >= (long long)off_E + (long long)S * T) return;
  int seg;
  long long src_row;
  if (r < off_E) {
    int lo = 0, hi = E;  // last e with offsets[e] <= r
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (offsets[mid] <= r) lo = mid; else hi = mid;
    }
    seg = lo;
    src_row = (MODE == MODE_DOWN) ? r : sorted_assign[r] / k;
  } else {
    seg = E + (int)((r - off_E) / T);
    src_row = (MODE == MODE_DOWN) ? r : (r - off_E) % T;
  }
  const float* xrow = X + src_row * K;
  const float* wrow = W + ((long long)seg * Wrows + n) * K;
  float z = 0.f;
  for (int j = 0; j < K; ++j) z = fmaf(xrow[j], wrow[j], z);
  float v;
  if (MODE == MODE_SWIGLU) {
    const float* urow = W + ((long long)seg * Wrows + f + n) * K;
    float u = 0.f;
    for (int j = 0; j < K; ++j) u = fmaf(xrow[j], urow[j], u);
    v = silu_f(z) * u;
  } else {
    if (bias) z += bias[(long long)seg * Wrows + n];
    v = MODE == MODE_RELU ? fmaxf(z, 0.f) : MODE == MODE_GELU ? gelu_f(z) : z;
  }
  out[r * Nout + n] = v;
}

// Block tiles per projection.
constexpr int UP_BM = 256, UP_BN = 256;
constexpr int DN_BM = 128, DN_BN = 128;

int grid_blocks(const Shape& s, int BM, int NT) {
  const long long mt = ((long long)s.T * s.k + BM - 1) / BM + s.E +
                       (long long)s.S * ((s.T + BM - 1) / BM);
  const long long g = NT * mt;
  return (int)((g + 7) / 8 * 8);
}

}  // namespace

hipError_t launch_decode_up(const Shape& s, const void* x, const void* w_up, const void* b_up,
                            const int32_t* offsets, const int32_t* sorted_assign, void* h,
                            hipStream_t st);
hipError_t launch_decode_down(const Shape& s, const void* h, const void* w_down,
                              const void* b_down, const int32_t* offsets, float* y_exp,
                              float* y_part, hipStream_t st);

hipError_t launch_up(const Shape& s, const void* x, const void* w_up, const void* b_up,
                     const int32_t* offsets, const int32_t* sorted_assign, void* h,
                     hipStream_t st) {
  const void* bias = s.expert_bias() ? b_up : nullptr;
  if (s.dtype == MOE_F32) {
    const long long n = s.max_rows() * s.f;
    const int blocks = (int)((n + 255) / 256);
    const float* X = (const float*)x;
    const float* W = (const float*)w_up;
    const float* B = (const float*)bias;
    float* O = (float*)h;
    if (s.act == MOE_RELU)
      gemm_f32_kernel<MODE_RELU><<<blocks, 256, 0, st>>>(X, W, B, O, offsets, sorted_assign, s.T,
                                                        s.k, s.E, s.S, s.d, s.f, s.up_rows(), s.f);
    else if (s.act == MOE_GELU)
      gemm_f32_kernel<MODE_GELU><<<blocks, 256, 0, st>>>(X, W, B, O, offsets, sorted_assign, s.T,
                                                        s.k, s.E, s.S, s.d, s.f, s.up_rows(), s.f);
    else
      gemm_f32_kernel<MODE_SWIGLU><<<blocks, 256, 0, st>>>(X, W, B, O, offsets, sorted_assign,
                                                          s.T, s.k, s.E, s.S, s.d, s.f,
                                                          s.up_rows(), s.f);
    return hipGetLastError();
  }
  if (s.decode()) return launch_decode_up(s, x, w_up, b_up, offsets, sorted_assign, h, st);
  GemmArgs a{(const uint16_t*)x, (const uint16_t*)w_up, (const uint16_t*)bias, h, offsets,
             sorted_assign, s.T, s.k, s.E, s.S, s.d, s.f, s.up_rows(), s.f};
  if (s.act == MOE_SWIGLU) {
    const int NT = (s.f + UP_BN / 2 - 1) / (UP_BN / 2);
    grouped_gemm_kernel<UP_BM, UP_BN, MODE_SWIGLU><<<grid_blocks(s, UP_BM, NT), 256, 0, st>>>(a);
  } else {
    const int NT = (s.f + UP_BN - 1) / UP_BN;
    if (s.act == MOE_RELU)
      grouped_gemm_kernel<UP_BM, UP_BN, MODE_RELU><<<grid_blocks(s, UP_BM, NT), 256, 0, st>>>(a);
    else
      grouped_gemm_kernel<UP_BM, UP_BN, MODE_GELU><<<grid_blocks(s, UP_BM, NT), 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_down(const Shape& s, const void* h, const void* w_down, const void* b_down,
                       const int32_t* offsets, float* y_exp, float* y_part, hipStream_t st) {
  const void* bias = s.expert_bias() ? b_down : nullptr;
  if (s.dtype == MOE_F32) {
    const long long n = s.max_rows() * s.d;
    const int blocks = (int)((n + 255) / 256);
    gemm_f32_kernel<MODE_DOWN><<<blocks, 256, 0, st>>>(
        (const float*)h, (const float*)w_down, (const float*)bias, y_exp, offsets, nullptr, s.T,
        s.k, s.E, s.S, s.f, s.d, s.d, s.f);
    return hipGetLastError();
  }
  if (s.decode()) return launch_decode_down(s, h, w_down, b_down, offsets, y_exp, y_part, st);
  GemmArgs a{(const uint16_t*)h, (const uint16_t*)w_down, (const uint16_t*)bias, y_exp, offsets,
             nullptr, s.T, s.k, s.E, s.S, s.f, s.d, s.d, s.f};
  const int NT = (s.d + DN_BN - 1) / DN_BN;
  grouped_gemm_kernel<DN_BM, DN_BN, MODE_DOWN><<<grid_blocks(s, DN_BM, NT), 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace moe
