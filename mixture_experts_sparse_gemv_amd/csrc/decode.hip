// Expert FFNs for decode-sized batches (T <= 16): the sparse-GEMV regime
// ("MoE混合专家模型" 5.2: with few tokens the layer is a stream of the
// touched experts' weights).
//
// Each expert sees at most T <= 16 rows, so the work is a stream of the
// touched experts' weights through the matrix cores with the (few) token
// rows as the 16-wide MFMA operand: bf16 MFMA 16x16x32 for the up
// projection, fp16 MFMA 16x16x32 for the down projection (W2 converted to
// fp16 in registers).  Every weight byte of a touched expert is read from
// HBM exactly once; experts with no rows are skipped without reading their
// weights.
//
// One 64-lane wave (its own block) is one work item: DR consecutive rows of
// one weight matrix (for SwiGLU DR/2 gate rows and the DR/2 matching up
// rows) over a range of K.  The weights move from HBM straight into LDS by
// buffer_load ... lds (one 128-byte line of one row per 8 lanes, so every
// instruction consumes whole lines; non-temporal, since nothing re-reads
// them), through a ring of NST stages of 64 K-elements, NST-1 stages in
// flight.  Each stage also carries the 64 K-elements of the 16 token rows
// (x gathered through sorted_assign, or h), the MFMA "B" operand.
// LDS rows are XOR-swizzled in 16-byte chunks ((row/2) % 8) so the fragment
// reads are free of bank conflicts.
//
// Up:   item = (segment, DR rows of W1) -> h columns, bias + activation.
// Down: item = (segment, DR rows of W2 = DR columns of y, one of nsplit
//       slices of K); the slice partials are summed in a fixed order (and the
//       bias added) by split_reduce_kernel.
#include "moe_internal.h"

namespace moe {
namespace {

enum { DEC_DOWN = 3 };   // modes: MOE_RELU, MOE_GELU, MOE_SWIGLU (up) or DEC_DOWN

#ifndef MOE_DECODE_ROWS
#define MOE_DECODE_ROWS 32
#endif
#ifndef MOE_DECODE_STAGES
#define MOE_DECODE_STAGES 4
#endif
constexpr int DR = MOE_DECODE_ROWS;     // weight rows per work item
constexpr int NST = MOE_DECODE_STAGES;  // LDS ring stages
constexpr int DK = 64;                  // K elements per stage: one 128-byte line per row
constexpr int RG = DR / 16;             // MFMA row groups
constexpr int NDMA = DR / 8;            // DMA instructions per stage (8 rows each)
static_assert(DR % 16 == 0 && DR <= 64 && NST >= 2 && NST <= 4, "decode tiling");

struct DecodeArgs {
  const uint16_t* X;       // up: x [T, d] bf16; down: h [rows, f] fp16
  const uint16_t* W;       // [segments][Wrows][K] bf16
  const uint16_t* bias;    // up: [segments][Wrows] bf16, or null
  void* out;               // up: h [rows, f] fp16; down: y_part [nsplit][rows][d] fp32
  const int32_t* offsets;
  const int32_t* sorted_assign;
  int T, k, E, S, K, Wrows, f, nsplit, items_per_seg;
  long long part_stride;
  long long xbytes;        // bytes of X (bounds of its buffer resource)
};

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

// s_waitcnt with vmcnt = n (n <= 63), expcnt and lgkmcnt not waited for.
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int MODE>
__global__ __launch_bounds__(64) void decode_kernel(DecodeArgs a) {
  constexpr bool DOWN = MODE == DEC_DOWN, SWIGLU = MODE == MOE_SWIGLU;
  static_assert(!SWIGLU || RG % 2 == 0, "SwiGLU pairs MFMA row groups of gate and up rows");
  constexpr int LR = DR + 16;   // LDS rows per stage: DR weight rows, then 16 token rows
  // The ring as distinct arrays ([row][8 chunks of 16 bytes] each): the
  // compiler then sees that a DMA into one stage never aliases the fragment
  // reads of another and keeps its own waits per stage.
  __shared__ u32x4 ring0[LR * 8], ring1[LR * 8], ring2[NST > 2 ? LR * 8 : 1],
      ring3[NST > 3 ? LR * 8 : 1];
  const int lane = threadIdx.x;
  const int seg = blockIdx.x / a.items_per_seg, it = blockIdx.x % a.items_per_seg;
  if (seg >= a.E + a.S) return;
  int rows, start;
  seg_info(a.offsets, seg, a.E, a.T, rows, start);
  if (rows <= 0) return;   // untouched expert: its weights are never read

  const int nt = DOWN ? it / a.nsplit : it;       // row block of the weight matrix
  const int ks = DOWN ? it % a.nsplit : 0;        // K slice
  const int klen = DOWN ? a.K / a.nsplit : a.K;
  const int k0 = ks * klen;
  const int nk = klen / DK;

  // Buffer-resource DMA: uniform bases (the expert's matrix and the token
  // rows, from column k0), per-lane 32-bit byte offsets that stay fixed over
  // the loop (one expert's matrix is below 4 GiB), and the stage's K offset
  // as the scalar offset.  Instruction q of a stage fills LDS rows 8q ..
  // 8q+7: lane l writes row 8q + l/8, chunk position l%8, which holds the
  // row's global chunk (l%8) ^ ((row/2) % 8).
  auto weight_row = [&](int r) {
    if (SWIGLU) return r < DR / 2 ? nt * (DR / 2) + r : a.f + nt * (DR / 2) + (r - DR / 2);
    return nt * DR + r;
  };
  const uint16_t* wseg = a.W + (long long)seg * a.Wrows * a.K + k0;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)wseg, (short)0, (int)(((long long)a.Wrows * a.K - k0) * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.X + k0), (short)0, (int)(a.xbytes - (long long)k0 * 2), 0x00020000);
  uint32_t soff[NDMA], xoff[2];
#pragma unroll
  for (int q = 0; q < NDMA; ++q) {
    const int r = 8 * q + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    soff[q] = ((uint32_t)weight_row(r) * (uint32_t)a.K + (uint32_t)c * 8u) * 2u;
  }
  // token rows: x gathered through sorted_assign (up) or h (down); rows past
  // the segment's count repeat a valid row and their outputs are not stored
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int t = 8 * q + (lane >> 3);
    const int tt = t < rows ? t : 0;
    uint32_t brow;
    if (DOWN) brow = (uint32_t)(start + tt);
    else brow = (uint32_t)(seg < a.E ? a.sorted_assign[start + tt] / a.k : tt);
    const int c = (lane & 7) ^ (((DR + t) >> 1) & 7);
    xoff[q] = (brow * (uint32_t)a.K + (uint32_t)c * 8u) * 2u;
  }
  // fragment reads: A row 16q + tl and B row DR + tl, chunk 4h + g of half h
  const int tl = lane & 15, g = lane >> 4;
  const bool tvalid = tl < rows;
  int fpos[RG][2], bpos[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int q = 0; q < RG; ++q) {
      const int r = 16 * q + tl;
      fpos[q][h] = r * 8 + ((4 * h + g) ^ ((r >> 1) & 7));
    }
    const int rb = DR + tl;
    bpos[h] = rb * 8 + ((4 * h + g) ^ ((rb >> 1) & 7));
  }

  typedef __attribute__((address_space(3))) void lds_void_t;
  // called with indices that are constants after unrolling
  auto slot = [&](int i) -> u32x4* { return i == 0 ? ring0 : i == 1 ? ring1 : i == 2 ? ring2 : ring3; };
  f32x4 acc[RG];
#pragma unroll
  for (int q = 0; q < RG; ++q) acc[q] = f32x4{};

  auto issue = [&](u32x4* buf, int j) {
#pragma unroll
    for (int q = 0; q < NDMA; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, (lds_void_t*)(buf + q * 64), 16, soff[q],
                                               j * DK * 2, 0, 2 /* nt */);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (lds_void_t*)(buf + (DR / 8 + q) * 64), 16,
                                               xoff[q], j * DK * 2, 0, 0);
  };
  auto compute = [&](const u32x4* buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 xv = buf[bpos[h]];
#pragma unroll
      for (int q = 0; q < RG; ++q) {
        const u32x4 w = buf[fpos[q][h]];
        if (DOWN)
          acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              __builtin_bit_cast(f16x8, bf16x8_to_f16x8(w)), __builtin_bit_cast(f16x8, xv),
              acc[q], 0, 0, 0);
        else
          acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, w), __builtin_bit_cast(bf16x8, xv), acc[q], 0, 0, 0);
      }
    }
  };
  // Each stage is NDMA + 2 DMA loads; they complete in issue order.
  constexpr int PER = NDMA + 2;
  auto wait_stage = [&](int ahead) {   // stages issued after the one to consume
    if (NST >= 4 && ahead >= 3) wait_vm<3 * PER>();
    else if (NST >= 3 && ahead >= 2) wait_vm<2 * PER>();
    else if (ahead >= 1) wait_vm<PER>();
    else wait_vm<0>();
    __asm__ volatile("" ::: "memory");
  };

#pragma unroll
  for (int j = 0; j < NST - 1; ++j)
    if (j < nk) issue(slot(j), j);
  // Stage j lives in ring slot j % NST (loops unrolled over the slots).
  // Steady state: every step issues stage j + NST - 1 and waits for stage j
  // with NST - 1 stages still in flight.
  int j0 = 0;
  for (; j0 + 2 * NST - 1 <= nk; j0 += NST) {
#pragma unroll
    for (int sl = 0; sl < NST; ++sl) {
      __asm__ volatile("" ::: "memory");   // slot (j-1) % NST has been read
      issue(slot((sl + NST - 1) % NST), j0 + sl + NST - 1);
      wait_vm<(NST - 1) * PER>();
      __asm__ volatile("" ::: "memory");
      compute(slot(sl));
    }
  }
  // the last (fewer than 2 NST - 1) stages
  for (; j0 < nk; j0 += NST) {
#pragma unroll
    for (int sl = 0; sl < NST; ++sl) {
      const int j = j0 + sl;
      if (j < nk) {
        __asm__ volatile("" ::: "memory");
        if (j + NST - 1 < nk) issue(slot((sl + NST - 1) % NST), j + NST - 1);
        wait_stage(min(NST - 1, nk - 1 - j));
        compute(slot(sl));
      }
    }
  }
  if (!tvalid) return;

  // D[row][token]: lane holds token tl and rows 16q + 4g + 0..3 of group q.
  const long long orow = start + tl;
  if (DOWN) {
    float* out = (float*)a.out + ks * a.part_stride + orow * a.Wrows + nt * DR + 4 * g;
#pragma unroll
    for (int q = 0; q < RG; ++q) *(f32x4*)(out + 16 * q) = acc[q];
  } else if (SWIGLU) {
    _Float16* hrow = (_Float16*)a.out + orow * a.f + nt * (DR / 2) + 4 * g;
#pragma unroll
    for (int q = 0; q < RG / 2; ++q) {
      f16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (_Float16)(silu_f(acc[q][r]) * acc[q + RG / 2][r]);
      *(f16x4*)(hrow + 16 * q) = v;
    }
  } else {
    _Float16* hrow = (_Float16*)a.out + orow * a.f + nt * DR + 4 * g;
#pragma unroll
    for (int q = 0; q < RG; ++q) {
      f16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float z = acc[q][r];
        if (a.bias) z += bf16_to_f32(a.bias[(long long)seg * a.Wrows + nt * DR + 16 * q + 4 * g + r]);
        v[r] = (_Float16)(MODE == MOE_RELU ? fmaxf(z, 0.f) : gelu_f(z));
      }
      *(f16x4*)(hrow + 16 * q) = v;
    }
  }
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
  const int items_per_seg = s.act == MOE_SWIGLU ? s.f / (DR / 2) : s.f / DR;
  const long long items = (long long)nseg * items_per_seg;
  DecodeArgs a{(const uint16_t*)x, (const uint16_t*)w_up,
               s.expert_bias() ? (const uint16_t*)b_up : nullptr, h, offsets, sorted_assign,
               s.T, s.k, s.E, s.S, s.d, s.up_rows(), s.f, 1, items_per_seg, 0,
               (long long)s.T * s.d * 2};
  if (s.act == MOE_SWIGLU) decode_kernel<MOE_SWIGLU><<<(int)items, 64, 0, st>>>(a);
  else if (s.act == MOE_GELU) decode_kernel<MOE_GELU><<<(int)items, 64, 0, st>>>(a);
  else decode_kernel<MOE_RELU><<<(int)items, 64, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_decode_down(const Shape& s, const void* h, const void* w_down,
                              const void* b_down, const int32_t* offsets, float* y_exp,
                              float* y_part, hipStream_t st) {
  const int nseg = s.E + s.S;
  // K slices of a multiple of 64 elements (f is a multiple of 64)
  const int nsplit = (s.f % (64 * kDecodeSplitK) == 0) ? kDecodeSplitK
                     : (s.f % 128 == 0 ? 2 : 1);
  const int items_per_seg = (s.d / DR) * nsplit;
  const long long items = (long long)nseg * items_per_seg;
  const long long part_stride = s.max_rows() * s.d;
  DecodeArgs a{(const uint16_t*)h, (const uint16_t*)w_down, nullptr, y_part, offsets, nullptr,
               s.T, s.k, s.E, s.S, s.f, s.d, s.f, nsplit, items_per_seg, part_stride,
               s.max_rows() * s.f * 2};
  decode_kernel<DEC_DOWN><<<(int)items, 64, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n = s.max_rows() * (s.d / 4);
  const uint16_t* b = s.expert_bias() ? (const uint16_t*)b_down : nullptr;
  split_reduce_kernel<<<(int)((n + 255) / 256), 256, 0, st>>>(y_part, b, y_exp, offsets, s.T, s.E,
                                                             s.S, s.d, nsplit, part_stride);
  return hipGetLastError();
}

}  // namespace moe
