// Expert FFNs for decode-sized batches (T <= 128): the sparse-GEMV regime
// ("MoE混合专家模型" 5.2: with few tokens the layer is a stream of the
// touched experts' weights).
//
// Each expert sees at most T <= 128 rows, so the work is a stream of the
// touched experts' weights through the matrix cores with the (few) token
// rows as the 16-wide MFMA operand, in up to 4 groups of 16 (a segment with
// more than 64 rows takes several passes, each streaming the weights): bf16 MFMA
// 16x16x32 for the up projection, fp16 MFMA 16x16x32 for the down projection
// (W2 converted to fp16 in registers).  Every weight byte of a touched
// expert is read from HBM once per pass (once when the expert has at most 64
// rows); experts with no rows are skipped without reading their weights.
//
// One 64-lane wave (its own block) is one work item: DR consecutive rows of
// one weight matrix (for SwiGLU DR/2 gate rows and the DR/2 matching up
// rows) over a range of K.  The weights move from HBM straight into LDS by
// buffer_load ... lds (one 128-byte line of one row per 8 lanes, so every
// instruction consumes whole lines; non-temporal, since nothing re-reads
// them), through a ring of NST stages of 64 K-elements, NST-1 stages in
// flight.  The 16 token rows (x gathered through sorted_assign, or h) are
// the MFMA "B" operand: each stage also carries their K range in LDS, or,
// for the FP8 up projection, loads it straight into registers (16 bytes per
// lane and k-substep, beside the weight DMA; the rows stay in L2), which
// halves the wave's LDS ring and lets twice as many waves share a unit.
// LDS rows are XOR-swizzled in 16-byte chunks ((row/2) % 8) so the fragment
// reads are free of bank conflicts.
//
// Up:   item = (segment, DR rows of W1) -> h columns, bias + activation.
// Down: item = (segment, DR rows of W2 = DR columns of y, one of nsplit
//       slices of K); slice 0 (with the bias) writes y_exp, the others
//       partials that are added to it in slice order (by the combine, or by
//       part_add_kernel when y_exp must be whole).
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
#ifndef MOE_DECODE_ROWS_F8
#define MOE_DECODE_ROWS_F8 32
#endif
#ifndef MOE_DECODE_STAGES_F8
#define MOE_DECODE_STAGES_F8 3
#endif
// token rows in registers: 0 never, 1 for the FP8 up projection, 2 always
#ifndef MOE_DECODE_XREG
#define MOE_DECODE_XREG 1
#endif
// Weight rows per work item and LDS ring stages, for bf16 and FP8 weights.
template <bool F8> struct DecodeTile {
  static constexpr int DR = F8 ? MOE_DECODE_ROWS_F8 : MOE_DECODE_ROWS;
  static constexpr int NST = F8 ? MOE_DECODE_STAGES_F8 : MOE_DECODE_STAGES;
  static_assert(DR % 16 == 0 && DR <= 64 && NST >= 2 && NST <= 4, "decode tiling");
};

struct DecodeArgs {
  const uint16_t* X;       // up: x [T, d] bf16; down: h [rows, f] fp16
  const void* W;           // [segments][Wrows][K] bf16, or FP8 E4M3 codes
  const float* wscale;     // FP8 only: [segments][Wrows] row scales
  const uint16_t* bias;    // [segments][Wrows] bf16, or null (down: added by K slice 0)
  void* out;               // up: h [rows, f] fp16; down: y_exp [rows, d] fp32 (K slice 0)
  float* part;             // down: K slices 1.. at part + (slice - 1) * part_stride
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

// Eight E4M3 codes -> eight bf16 (up) or fp16 (down) values, exactly (the
// hardware conversions decode OCP E4M3; every E4M3 value is representable).
template <bool TO_F16>
__device__ __forceinline__ u32x4 e4m3x8_to_16(u32x2 c) {
  u32x4 r = {};
#if __HIP_DEVICE_COMPILE__   // the host pass of the kernel does not see the gfx950 builtins
  const int w0 = (int)c[0], w1 = (int)c[1];
  if (TO_F16) {
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true));
  } else {
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  }
#endif
  return r;
}

// F8: the weights are E4M3 codes with per-row scales (applied to the
// accumulated sums); a stage then covers 128 K-elements (128 weight bytes
// per row, as for bf16 with 64) and carries 256 bytes of each token row.
// TG: groups of 16 token rows (a segment of up to 16 TG rows); each weight
// stage feeds the MFMAs of every group that holds rows of the segment.
template <int MODE, bool F8, int TG>
__global__ __launch_bounds__(64) void decode_kernel(DecodeArgs a) {
  constexpr bool DOWN = MODE == DEC_DOWN, SWIGLU = MODE == MOE_SWIGLU;
  constexpr int DR = DecodeTile<F8>::DR;    // weight rows per work item
  // LDS ring stages; with four token groups a stage carries 64 token rows, so
  // 3 stages (four waves per compute unit instead of three) measured 5%
  // faster at T = 48 ... 128 (2 groups: 4 stages stay faster)
  constexpr int NST = TG >= 4 ? 3 : DecodeTile<F8>::NST;
  constexpr int RG = DR / 16;               // MFMA row groups
  constexpr int NDMA = DR / 8;              // weight DMA instructions per stage (8 rows each)
  static_assert(!SWIGLU || RG % 2 == 0, "SwiGLU pairs MFMA row groups of gate and up rows");
  constexpr int WB = F8 ? 1 : 2;         // weight bytes
  constexpr int SK = F8 ? 128 : 64;      // K elements per stage
  constexpr int NSUBK = SK / 32;         // MFMA k-substeps per stage
  // token rows in registers (XREG) or as XR 128-byte LDS rows per stage
  constexpr bool XREG = TG == 1 && (MOE_DECODE_XREG == 2 || (MOE_DECODE_XREG == 1 && F8 && !DOWN));
  constexpr int XR = XREG ? 0 : (F8 ? 32 : 16) * TG;
  constexpr int NDX = XR / 8;            // their DMA instructions
  constexpr int LR = DR + XR;            // LDS rows per stage: weights, then token rows
  // The ring as distinct arrays ([row][8 chunks of 16 bytes] each): the
  // compiler then sees that a DMA into one stage never aliases the fragment
  // reads of another and keeps its own waits per stage.
  __shared__ u32x4 ring0[LR * 8], ring1[LR * 8], ring2[NST > 2 ? LR * 8 : 1],
      ring3[NST > 3 ? LR * 8 : 1];
  const int lane = threadIdx.x;
  const int seg = blockIdx.x / a.items_per_seg, it = blockIdx.x % a.items_per_seg;
  if (seg >= a.E + a.S) return;
  int rows_all, start_all;
  seg_info(a.offsets, seg, a.E, a.T, rows_all, start_all);
  if (rows_all <= 0) return;   // untouched expert: its weights are never read

  const int nt = DOWN ? it / a.nsplit : it;       // row block of the weight matrix
  const int ks = DOWN ? it % a.nsplit : 0;        // K slice
  const int klen = DOWN ? a.K / a.nsplit : a.K;
  const int k0 = ks * klen;
  const int nk = klen / SK;
  // Up projection: stage j of item i reads K stage (j + i) mod nk, so the
  // items in flight at one moment read different columns of their rows.
  // With every item at the same column (all rows of a matrix share their low
  // address bits) the requests of a moment crowd the same DRAM channels:
  // measured on the 8-expert d = 4096, f = 14336 layer, the bf16 up
  // projection went from 0.77 to 0.83 of 8 TB/s and the FP8 one from 0.68 to
  // 0.78.  The down projection's consecutive items are already different K
  // slices (the same order there measured 1% slower).
  const int rot = !DOWN && nk > 1 ? (int)(blockIdx.x % (unsigned)nk) : 0;
  auto kpos = [&](int j) { const int p = j + rot; return p >= nk ? p - nk : p; };

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
  const char* wseg = (const char*)a.W + ((long long)seg * a.Wrows * a.K + k0) * WB;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)wseg, (short)0, (int)(((long long)a.Wrows * a.K - k0) * WB), 0x00020000);
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.X + k0), (short)0, (int)(a.xbytes - (long long)k0 * 2), 0x00020000);
  uint32_t soff[NDMA], xoff[NDX > 0 ? NDX : 1];
#pragma unroll
  for (int q = 0; q < NDMA; ++q) {
    const int r = 8 * q + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    soff[q] = (uint32_t)weight_row(r) * (uint32_t)a.K * WB + (uint32_t)c * 16u;
  }
  // Passes over the segment's rows, 16 TG at a time: a segment with more rows
  // than one pass holds streams the item's weights once per pass.
  for (int p0 = 0; p0 < rows_all; p0 += 16 * TG) {
    const int rows = min(16 * TG, rows_all - p0), start = start_all + p0;
    const int ntg = (rows + 15) >> 4;   // token groups holding rows of this pass (<= TG)
    // token rows: x gathered through sorted_assign (up) or h (down); rows past
    // the pass's count repeat a valid row and their outputs are not stored.
    // With F8 each token row of a stage spans two LDS rows (halves of 64).
#pragma unroll
    for (int q = 0; q < NDX; ++q) {
      const int rl = 8 * q + (lane >> 3);
      const int t = F8 ? rl >> 1 : rl, half = F8 ? rl & 1 : 0;
      const int tt = t < rows ? t : 0;
      uint32_t brow;
      if (DOWN) brow = (uint32_t)(start + tt);
      else brow = (uint32_t)(seg < a.E ? a.sorted_assign[start + tt] / a.k : p0 + tt);
      const int c = (lane & 7) ^ (((DR + rl) >> 1) & 7);
      xoff[q] = (brow * (uint32_t)a.K + (uint32_t)(half * 64 + c * 8)) * 2u;
    }
    // fragment reads (byte offsets in a stage): A rows 16q + tl, B token row
    // 16 tg + tl; k-substep u covers K elements 32u .. 32u+31 of the stage
    const int tl = lane & 15, g = lane >> 4;
    const bool tvalid = tl < rows;
    // XREG: the lane's token row (K elements 32u + 8g .. +7 of substep u)
    uint32_t xroff = 0;
    if (XREG) {
      const int tt = tvalid ? tl : 0;
      uint32_t brow;
      if (DOWN) brow = (uint32_t)(start + tt);
      else brow = (uint32_t)(seg < a.E ? a.sorted_assign[start + tt] / a.k : p0 + tt);
      xroff = (brow * (uint32_t)a.K + (uint32_t)(8 * g)) * 2u;
    }
    (void)xroff;   // read by the device pass only
    int fpos[RG][NSUBK], bpos[TG][NSUBK];
#pragma unroll
    for (int u = 0; u < NSUBK; ++u) {
#pragma unroll
      for (int q = 0; q < RG; ++q) {
        const int r = 16 * q + tl;
        if (F8) fpos[q][u] = r * 128 + (((2 * u + (g >> 1)) ^ ((r >> 1) & 7)) * 16) + 8 * (g & 1);
        else fpos[q][u] = r * 128 + (((4 * u + g) ^ ((r >> 1) & 7)) * 16);
      }
#pragma unroll
      for (int tg = 0; tg < TG; ++tg) {
        const int tr = 16 * tg + tl;
        const int rb = F8 ? DR + 2 * tr + (u >> 1) : DR + tr;
        const int cb = F8 ? 4 * (u & 1) + g : 4 * u + g;
        bpos[tg][u] = rb * 128 + ((cb ^ ((rb >> 1) & 7)) * 16);
      }
    }

    // called with indices that are constants after unrolling
    auto slot = [&](int i) -> u32x4* { return i == 0 ? ring0 : i == 1 ? ring1 : i == 2 ? ring2 : ring3; };
    f32x4 acc[TG][RG];
#pragma unroll
    for (int tg = 0; tg < TG; ++tg)
#pragma unroll
      for (int q = 0; q < RG; ++q) acc[tg][q] = f32x4{};
    // XREG: token fragments of the stages in flight, one set per ring slot
    u32x4 xr[XREG ? NST : 1][NSUBK];

    auto issue = [&](u32x4* buf, u32x4 (&xs)[NSUBK], int j) {
#if __HIP_DEVICE_COMPILE__   // (with template-dependent operands the host pass drops the kernel)
      typedef __attribute__((address_space(3))) void lds_void_t;
#pragma unroll
      for (int q = 0; q < NDMA; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wres, (lds_void_t*)(buf + q * 64), 16, soff[q],
                                                 kpos(j) * SK * WB, 0, 2 /* nt */);
#pragma unroll
      for (int q = 0; q < NDX; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (lds_void_t*)(buf + (DR / 8 + q) * 64), 16,
                                                 xoff[q], kpos(j) * SK * 2, 0, 0);
      if (XREG) {
#pragma unroll
        for (int u = 0; u < NSUBK; ++u)
          xs[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                xres, xroff + u * 64, kpos(j) * SK * 2, 0));
      }
#endif
    };
    auto compute = [&](const u32x4* buf, const u32x4 (&xs)[NSUBK]) {
      const char* b = (const char*)buf;
#pragma unroll
      for (int u = 0; u < NSUBK; ++u) {
        u32x4 w[RG];
#pragma unroll
        for (int q = 0; q < RG; ++q) {
          if (F8) w[q] = e4m3x8_to_16<DOWN>(*(const u32x2*)(b + fpos[q][u]));
          else w[q] = DOWN ? bf16x8_to_f16x8(*(const u32x4*)(b + fpos[q][u])) : *(const u32x4*)(b + fpos[q][u]);
        }
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) {
          if (tg >= ntg) break;   // uniform: no rows of the segment in this group
          const u32x4 xv = XREG ? xs[u] : *(const u32x4*)(b + bpos[tg][u]);
#pragma unroll
          for (int q = 0; q < RG; ++q) {
            if (DOWN)
              acc[tg][q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  __builtin_bit_cast(f16x8, w[q]), __builtin_bit_cast(f16x8, xv), acc[tg][q], 0, 0, 0);
            else
              acc[tg][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8, w[q]), __builtin_bit_cast(bf16x8, xv), acc[tg][q], 0, 0,
                  0);
          }
        }
      }
    };
    // Each stage is NDMA + NDX DMA loads (+ NSUBK token loads with XREG); they
    // complete in issue order.
    constexpr int PER = NDMA + NDX + (XREG ? NSUBK : 0);
    auto xslot = [&](int i) -> u32x4(&)[NSUBK] { return xr[XREG ? i : 0]; };
    auto wait_stage = [&](int ahead) {   // stages issued after the one to consume
      if (NST >= 4 && ahead >= 3) wait_vm<3 * PER>();
      else if (NST >= 3 && ahead >= 2) wait_vm<2 * PER>();
      else if (ahead >= 1) wait_vm<PER>();
      else wait_vm<0>();
      __asm__ volatile("" ::: "memory");
    };

#pragma unroll
    for (int j = 0; j < NST - 1; ++j)
      if (j < nk) issue(slot(j), xslot(j), j);
    // Stage j lives in ring slot j % NST (loops unrolled over the slots).
    // Steady state: every step issues stage j + NST - 1 and waits for stage j
    // with NST - 1 stages still in flight.
    int j0 = 0;
    for (; j0 + 2 * NST - 1 <= nk; j0 += NST) {
#pragma unroll
      for (int sl = 0; sl < NST; ++sl) {
        __asm__ volatile("" ::: "memory");   // slot (j-1) % NST has been read
        issue(slot((sl + NST - 1) % NST), xslot((sl + NST - 1) % NST), j0 + sl + NST - 1);
        wait_vm<(NST - 1) * PER>();
        __asm__ volatile("" ::: "memory");
        compute(slot(sl), xslot(sl));
      }
    }
    // the last (fewer than 2 NST - 1) stages
    for (; j0 < nk; j0 += NST) {
#pragma unroll
      for (int sl = 0; sl < NST; ++sl) {
        const int j = j0 + sl;
        if (j < nk) {
          __asm__ volatile("" ::: "memory");
          if (j + NST - 1 < nk)
            issue(slot((sl + NST - 1) % NST), xslot((sl + NST - 1) % NST), j + NST - 1);
          wait_stage(min(NST - 1, nk - 1 - j));
          compute(slot(sl), xslot(sl));
        }
      }
    }
    // D[row][token]: lane holds token 16 tg + tl and rows 16q + 4g + 0..3 of
    // group q (consecutive weight rows, so their FP8 scales are one 16-byte load).
    f32x4 sc[RG];
    if (F8) {
#pragma unroll
      for (int q = 0; q < RG; ++q)
        sc[q] = *(const f32x4*)(a.wscale + (long long)seg * a.Wrows + weight_row(16 * q + 4 * g));
    }
#pragma unroll
    for (int tg = 0; tg < TG; ++tg) {
      const int t = 16 * tg + tl;
      if (t >= rows) break;   // the rows of a segment are 0 .. rows - 1
      f32x4* ac = acc[tg];
      if (F8) {
#pragma unroll
        for (int q = 0; q < RG; ++q) ac[q] *= sc[q];
      }
      const long long orow = start + t;
      if (DOWN) {
        float* out = (ks == 0 ? (float*)a.out : a.part + (ks - 1) * a.part_stride) + orow * a.Wrows +
                     nt * DR + 4 * g;
#pragma unroll
        for (int q = 0; q < RG; ++q) {
          f32x4 v = ac[q] * kHLoadScale;   // h was stored scaled by 2^-8
          if (ks == 0 && a.bias) {
            const uint16_t* b = a.bias + (long long)seg * a.Wrows + nt * DR + 16 * q + 4 * g;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] += bf16_to_f32(b[r]);
          }
          *(f32x4*)(out + 16 * q) = v;
        }
      } else if (SWIGLU) {
        _Float16* hrow = (_Float16*)a.out + orow * a.f + nt * (DR / 2) + 4 * g;
#pragma unroll
        for (int q = 0; q < RG / 2; ++q) {
          f16x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = h_to_f16(silu_f(ac[q][r]) * ac[q + RG / 2][r]);
          *(f16x4*)(hrow + 16 * q) = v;
        }
      } else {
        _Float16* hrow = (_Float16*)a.out + orow * a.f + nt * DR + 4 * g;
#pragma unroll
        for (int q = 0; q < RG; ++q) {
          f16x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float z = ac[q][r];
            if (a.bias) z += bf16_to_f32(a.bias[(long long)seg * a.Wrows + nt * DR + 16 * q + 4 * g + r]);
            v[r] = h_to_f16(MODE == MOE_RELU ? fmaxf(z, 0.f) : gelu_f(z));
          }
          *(f16x4*)(hrow + 16 * q) = v;
        }
      }
    }
  }   // passes
}

// y_exp[r, :] += the partials of K slices 1 .. nparts, in slice order.
__global__ __launch_bounds__(256) void part_add_kernel(float* __restrict__ y_exp,
                                                       const float* __restrict__ y_part,
                                                       const int32_t* offsets, int T, int E,
                                                       int S, int d, int nparts,
                                                       long long part_stride) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int d4 = d / 4;
  const long long r = gid / d4;
  const int c = (int)(gid % d4) * 4;
  if (r >= (long long)offsets[E] + (long long)S * T) return;
  f32x4 acc = *(const f32x4*)(y_exp + r * d + c);
  for (int p = 0; p < nparts; ++p) acc += *(const f32x4*)(y_part + p * part_stride + r * d + c);
  *(f32x4*)(y_exp + r * d + c) = acc;
}

}  // namespace

// Groups of 16 token rows the decode kernels carry: enough for any segment
// (a routed expert holds at most T rows, a shared one exactly T).
static int decode_token_groups(const Shape& s) { return s.T <= 16 ? 1 : s.T <= 32 ? 2 : 4; }

hipError_t launch_decode_up(const Shape& s, const void* x, const void* w_up, const void* b_up,
                            const float* s_up, const int32_t* offsets,
                            const int32_t* sorted_assign, void* h, hipStream_t st) {
  const int nseg = s.E + s.S;
  const int DR = s.w_fp8() ? DecodeTile<true>::DR : DecodeTile<false>::DR;
  const int items_per_seg = s.act == MOE_SWIGLU ? s.f / (DR / 2) : s.f / DR;
  const long long items = (long long)nseg * items_per_seg;
  DecodeArgs a{(const uint16_t*)x, w_up, s_up,
               s.expert_bias() ? (const uint16_t*)b_up : nullptr, h, nullptr, offsets, sorted_assign,
               s.T, s.tok_div(), s.E, s.S, s.d, s.up_rows(), s.f, 1, items_per_seg, 0,
               (long long)s.T * s.d * 2};
  const int tg = decode_token_groups(s);
#define MOE_DECODE_UP(A, F)                                                      \
  (tg == 1   ? decode_kernel<A, F, 1><<<(int)items, 64, 0, st>>>(a)              \
   : tg == 2 ? decode_kernel<A, F, 2><<<(int)items, 64, 0, st>>>(a)              \
             : decode_kernel<A, F, 4><<<(int)items, 64, 0, st>>>(a))
  if (s.w_fp8()) {
    if (s.act == MOE_SWIGLU) MOE_DECODE_UP(MOE_SWIGLU, true);
    else if (s.act == MOE_GELU) MOE_DECODE_UP(MOE_GELU, true);
    else MOE_DECODE_UP(MOE_RELU, true);
  } else {
    if (s.act == MOE_SWIGLU) MOE_DECODE_UP(MOE_SWIGLU, false);
    else if (s.act == MOE_GELU) MOE_DECODE_UP(MOE_GELU, false);
    else MOE_DECODE_UP(MOE_RELU, false);
  }
#undef MOE_DECODE_UP
  return hipGetLastError();
}

int decode_nsplit(const Shape& s) {
  // K slices of a whole number of stages (64 elements; 128 for FP8 weights)
  const int sk = s.w_fp8() ? 128 : 64;
  const int want = s.w_fp8() ? kDecodeSplitK8 : kDecodeSplitK;
  for (int n = want; n > 1; n /= 2)
    if (s.f % (sk * n) == 0) return n;
  return 1;
}

hipError_t launch_decode_down(const Shape& s, const void* h, const void* w_down,
                              const void* b_down, const float* s_down, const int32_t* offsets,
                              float* y_exp, float* y_part, bool complete, hipStream_t st) {
  const int nseg = s.E + s.S;
  const int nsplit = decode_nsplit(s);
  const int DR = s.w_fp8() ? DecodeTile<true>::DR : DecodeTile<false>::DR;
  const int items_per_seg = (s.d / DR) * nsplit;
  const long long items = (long long)nseg * items_per_seg;
  const long long part_stride = s.max_rows() * s.d;
  const uint16_t* b = s.expert_bias() ? (const uint16_t*)b_down : nullptr;
  DecodeArgs a{(const uint16_t*)h, w_down, s_down, b, y_exp, y_part, offsets, nullptr,
               s.T, s.tok_div(), s.E, s.S, s.f, s.d, s.f, nsplit, items_per_seg, part_stride,
               s.max_rows() * s.f * 2};
  const int tg = decode_token_groups(s);
#define MOE_DECODE_DOWN(F)                                                       \
  (tg == 1   ? decode_kernel<DEC_DOWN, F, 1><<<(int)items, 64, 0, st>>>(a)       \
   : tg == 2 ? decode_kernel<DEC_DOWN, F, 2><<<(int)items, 64, 0, st>>>(a)       \
             : decode_kernel<DEC_DOWN, F, 4><<<(int)items, 64, 0, st>>>(a))
  if (s.w_fp8()) MOE_DECODE_DOWN(true);
  else MOE_DECODE_DOWN(false);
#undef MOE_DECODE_DOWN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !complete || nsplit == 1) return e;
  const long long n = s.max_rows() * (s.d / 4);
  part_add_kernel<<<(int)((n + 255) / 256), 256, 0, st>>>(y_exp, y_part, offsets, s.T, s.E, s.S,
                                                         s.d, nsplit - 1, part_stride);
  return hipGetLastError();
}

}  // namespace moe
