// Router + gate + top-k + renormalization, fused in one kernel.
//
//   logits[t, e] = sum_j x[t, j] Wr[e, j] + br[e]           (0539edu 2.1; kamacoder 三)
//   softmax p = exp(l - max) / sum, or normalized sigmoid p = s / sum s
//                                                            ("MoE架构解析" 四 技术飞跃③)
//   top-k by descending score, ties to the lower expert index; weights =
//   selected scores / their sum                              (0539edu 2.1; kamacoder 三)
//
// A block handles 16 tokens with 8 waves (16 when there are at most 64
// blocks, i.e. T <= 1024).  For bf16 inputs the router
// product runs on bf16 MFMA 16x16x32 (A = 16 router rows, B = 16 token rows),
// each wave covering every 8th (16th) 32-wide K step and issuing the loads of 8
// steps at once (4 with three or four expert tiles); the partial logit tiles
// of the waves are summed in LDS in a fixed order.  The gate and the top-k
// then run one token per wave pass (two tokens per wave, or one with 16
// waves) with one lane per expert (E <= 64): wave-wide max and sum by DPP
// row steps and scalar reads of the row results.  Up to 16 experts,
// each lane counts the experts that beat it (a larger logit, or an equal one
// at a lower index), reading their logits as scalars, so the experts of rank
// 0 .. k-1 are the top k in order (ties to the lower index); with more, the
// k selections are taken one at a time as the largest remaining logit at its
// lowest lane (a wave max, then a ballot).  Experts are ranked by logit
// (monotone in both gates, so ranking and weights match ranking by score).
// No step goes through the LDS crossbar.  Each block also
// writes the sum of its 16 tokens' probabilities per expert (token order);
// these partial sums are reduced in block order for P.  It also writes the
// number of selections of each expert in its 16 tokens (the dispatch's
// per-chunk counts).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int RT = kRouterTokens;  // 16 tokens per block
// waves per block: 8, or 16 when there are few blocks (small T), so a block's
// K steps spread over more waves (one token per wave in the gate)
constexpr int RB = 8;              // K steps whose loads a wave issues together

struct RouterArgs {
  const void* x;
  const void* wr;
  const void* br;       // null if no router bias
  int32_t* topk_idx;
  float* topk_w;
  float* probs;         // null if not requested
  float* prob_part;     // [blocks, E]
  int32_t* chunk_counts;  // [blocks, E]: selections of each expert in the block's tokens
  float* logits;        // [T, E] logits incl. bias, or null (the backward pass recomputes them)
  int T, d, E, k, gating, dtype;
};

// At least 4 waves per SIMD (at most 128 VGPRs): two 8-wave blocks share a
// compute unit, so T = 8192 (512 blocks) runs in one round also with four
// expert tiles (measured at 64 experts, d = 2048: 41.7 -> 36.4 us).
template <int NE16, int RW>  // expert tiles of 16 (bf16 path; 0 = fp32 path), waves
__global__ __launch_bounds__(64 * RW) __attribute__((amdgpu_waves_per_eu(4))) void router_kernel(
    RouterArgs a) {
  __shared__ float red[RW][RT][kMaxExperts + 1];
  __shared__ float colp[RW][kMaxExperts];
  __shared__ int cntp[RW][kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * RT;
  const int E = a.E;

  if (NE16 > 0) {
    // ---- logits on the matrix cores
    const uint16_t* x = (const uint16_t*)a.x;
    const uint16_t* wr = (const uint16_t*)a.wr;
    const int tl = lane & 15, kg = lane >> 4;
    const int t = min(t0 + tl, a.T - 1);
    const uint16_t* xp = x + (long long)t * a.d + kg * 8;
    const uint16_t* wp[NE16 > 0 ? NE16 : 1];
#pragma unroll
    for (int j = 0; j < NE16; ++j) {
      const int e = min(j * 16 + (lane & 15), E - 1);
      wp[j] = wr + (long long)e * a.d + kg * 8;
    }
    f32x4 acc[NE16 > 0 ? NE16 : 1];
#pragma unroll
    for (int j = 0; j < NE16; ++j) acc[j] = f32x4{};
    const int nsteps = a.d / 32;
    if constexpr (NE16 <= 2) {
      for (int s0 = wave; s0 < nsteps; s0 += RW * RB) {
        u32x4 xv[RB], wv[RB][NE16 > 0 ? NE16 : 1];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const int s = min(s0 + b * RW, nsteps - 1);   // clamped; masked below
          xv[b] = *(const u32x4*)(xp + s * 32);
#pragma unroll
          for (int j = 0; j < NE16; ++j) wv[b][j] = *(const u32x4*)(wp[j] + s * 32);
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          if (s0 + b * RW >= nsteps) break;   // uniform
#pragma unroll
          for (int j = 0; j < NE16; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, wv[b][j]), __builtin_bit_cast(bf16x8, xv[b]), acc[j],
                0, 0, 0);
        }
      }
    } else {
      // Many expert tiles: the loads of up to RB / 2 steps are issued
      // together (a uniform test skips the steps past the end, whose
      // products a select discards), all before the first product, so none
      // of them waits for an earlier one (measured: 35 -> 33 us at 64
      // experts, d = 2048; with one or two expert tiles the compiler's own
      // interleaving, which keeps more waves resident, is faster).
      constexpr int RBN = RB / 2;
      for (int s0 = wave; s0 < nsteps; s0 += RW * RBN) {
        u32x4 xv[RBN], wv[RBN][NE16 > 0 ? NE16 : 1];
#pragma unroll
        for (int b = 0; b < RBN; ++b) {
          const int s = s0 + b * RW;
          xv[b] = u32x4{0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < NE16; ++j) wv[b][j] = u32x4{0, 0, 0, 0};
          if (s < nsteps) {   // uniform
            xv[b] = *(const u32x4*)(xp + s * 32);
#pragma unroll
            for (int j = 0; j < NE16; ++j) wv[b][j] = *(const u32x4*)(wp[j] + s * 32);
          }
        }
        __builtin_amdgcn_sched_barrier(0);   // every load above is issued before the first product
#pragma unroll
        for (int b = 0; b < RBN; ++b) {
          const bool ok = s0 + b * RW < nsteps;   // uniform
#pragma unroll
          for (int j = 0; j < NE16; ++j) {
            const f32x4 r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, wv[b][j]), __builtin_bit_cast(bf16x8, xv[b]), acc[j], 0,
                0, 0);
            acc[j] = ok ? r : acc[j];
          }
        }
      }
    }
    // The last, partial K step when d is not a multiple of 32 (d is a
    // multiple of 8: a lane's 8 elements are all in the row or all past it,
    // and those past it count as zero), taken by the wave next in turn.
    if (a.d % 32 != 0 && wave == nsteps % RW) {
      const bool in = nsteps * 32 + kg * 8 < a.d;
      const u32x4 xv = in ? *(const u32x4*)(xp + nsteps * 32) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < NE16; ++j) {
        const u32x4 wv = in ? *(const u32x4*)(wp[j] + nsteps * 32) : u32x4{0, 0, 0, 0};
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, wv), __builtin_bit_cast(bf16x8, xv), acc[j], 0, 0, 0);
      }
    }
    // D[expert][token]: lane holds token lane & 15, experts 16j + 4*(lane>>4) + r
#pragma unroll
    for (int j = 0; j < NE16; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][tl][j * 16 + 4 * kg + r] = acc[j][r];
  } else {
    // ---- fp32: one thread per (token, expert) dot product
    const float* x = (const float*)a.x;
    const float* wr = (const float*)a.wr;
    for (int p = tid; p < RT * kMaxExperts; p += 64 * RW) {
      const int tl = p / kMaxExperts, e = p % kMaxExperts;
      float z = 0.f;
      if (e < E && t0 + tl < a.T) {
        const float* xr = x + (long long)(t0 + tl) * a.d;
        const float* wrow = wr + (long long)e * a.d;
        for (int j = 0; j < a.d; ++j) z = fmaf(xr[j], wrow[j], z);
      }
      red[0][tl][e] = z;
#pragma unroll
      for (int w = 1; w < RW; ++w) red[w][tl][e] = 0.f;
    }
  }
  __syncthreads();

  // ---- gate + top-k: wave w handles tokens 2w, 2w+1; lane = expert
  float bias = 0.f;
  if (a.br && lane < E)
    bias = a.dtype == MOE_BF16 ? bf16_to_f32(((const uint16_t*)a.br)[lane])
                               : ((const float*)a.br)[lane];
  const float NEG_INF = -__builtin_inff();
  float psum = 0.f;
  int nsel = 0;   // lane e: selections of expert e by this wave's tokens
#pragma unroll 1
  for (int i = 0; i < RT / RW; ++i) {
    const int tl = wave * (RT / RW) + i;
    const int t = t0 + tl;
    if (t >= a.T) break;
    float l = NEG_INF;
    if (lane < E) {
      float z = red[0][tl][lane];
#pragma unroll
      for (int w = 1; w < RW; ++w) z += red[w][tl][lane];   // fixed order
      l = z + bias;
      if (a.logits) a.logits[(long long)t * E + lane] = l;
    }
    float score, denom;
    if (a.gating == MOE_SOFTMAX) {
      const float mx = wave_max_dpp(l);
      score = lane < E ? fast_exp(l - mx) : 0.f;   // unnormalized, exp(l - max)
      denom = wave_sum_dpp(score);
    } else {
      score = lane < E ? __builtin_amdgcn_rcpf(1.0f + fast_exp(-l)) : 0.f;   // sigma(l)
      denom = wave_sum_dpp(score);
    }
    const float p = score / denom;
    if (lane < E) {
      if (a.probs) a.probs[(long long)t * E + lane] = p;
      psum += p;
    }
    // rank of each expert: the experts with a larger logit, or an equal one
    // and a lower index (a NaN logit ranks below every number); lanes >= E
    // rank E or more.  The experts of rank 0 .. k-1 are the top k, in order.
    const float key = (l == l) ? l : NEG_INF;
    int rank = a.k;
    int my_idx = 0;
    float my_score = 0.f, sel_sum = 0.f;
    if (E <= 16) {
      rank = 0;
      for (int j = 0; j < E; ++j) {
        const float kj = lane_f(key, j);
        rank += (kj > key || (kj == key && j < lane)) ? 1 : 0;
      }
      for (int s = 0; s < a.k; ++s) {
        const uint64_t m = __ballot(rank == s);   // exactly one lane
        const int bi = m ? __builtin_ctzll(m) : 0;
        const float bs = lane_f(score, bi);
        sel_sum += bs;
        if (lane == s) { my_idx = bi; my_score = bs; }
      }
    } else {
      // Many experts: the k selections one at a time, each the largest
      // remaining key (a wave max over DPP row steps) at its lowest lane
      // (ballot of the lanes holding it among the remaining experts); the
      // q-th selection is the expert of rank q.
      uint64_t left = __ballot(lane < E);
      for (int q = 0; q < a.k; ++q) {
        const bool in = (left >> lane) & 1;
        const float mx = wave_max_dpp(in ? key : NEG_INF);
        const int j = __builtin_ctzll(__ballot(in && key == mx) & left);
        const float bs = lane_f(score, j);
        sel_sum += bs;
        if (lane == j) rank = q;
        if (lane == q) { my_idx = j; my_score = bs; }
        left &= ~(1ull << j);
      }
    }
    if (rank < a.k) ++nsel;
    if (lane < a.k && a.topk_idx) {   // (expert-choice routing uses the probabilities only)
      a.topk_idx[(long long)t * a.k + lane] = my_idx;
      a.topk_w[(long long)t * a.k + lane] = my_score / sel_sum;
    }
  }
  colp[wave][lane] = psum;
  cntp[wave][lane] = nsel;
  __syncthreads();
  if (tid < E) {
    float c = colp[0][tid];
    int n = cntp[0][tid];
#pragma unroll
    for (int w = 1; w < RW; ++w) {
      c += colp[w][tid];   // wave order = token order
      n += cntp[w][tid];
    }
    a.prob_part[(long long)blockIdx.x * E + tid] = c;
    a.chunk_counts[(long long)blockIdx.x * E + tid] = n;
  }
}

// colsum[e] = sum over router blocks b (in order, 256 strided partial sums
// then a fixed tree) of prob_part[b, e].  One block per expert.
__global__ __launch_bounds__(256) void colsum_kernel(const float* prob_part, int nblk, int E,
                                                     float* colsum) {
  __shared__ float s[256];
  const int e = blockIdx.x, tid = threadIdx.x;
  float v = 0.f;
  for (int b = tid; b < nblk; b += 256) v += prob_part[(long long)b * E + e];
  s[tid] = v;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) s[tid] += s[tid + o];
    __syncthreads();
  }
  if (tid == 0) colsum[e] = s[0];
}

}  // namespace

hipError_t launch_router(const Shape& s, const void* x, const void* wr, const void* br,
                         int32_t* topk_idx, float* topk_w, float* probs, float* prob_part,
                         int32_t* chunk_counts, hipStream_t st, float* logits) {
  RouterArgs a{x, wr, s.router_bias() ? br : nullptr, topk_idx, topk_w, probs, prob_part,
               chunk_counts, logits, s.T, s.d, s.E, s.k, s.gating, s.dtype};
  const int blocks = router_blocks(s);
  const bool wide = blocks <= 64;   // few blocks: 16 waves each
#define MOE_ROUTER(NE)                                            \
  do {                                                            \
    if (wide) router_kernel<NE, 16><<<blocks, 1024, 0, st>>>(a);  \
    else router_kernel<NE, 8><<<blocks, 512, 0, st>>>(a);         \
  } while (0)
  if (s.dtype == MOE_F32) {
    router_kernel<0, 8><<<blocks, 512, 0, st>>>(a);
  } else {
    const int ne16 = (s.E + 15) / 16;
    if (ne16 == 1) MOE_ROUTER(1);
    else if (ne16 == 2) MOE_ROUTER(2);
    else if (ne16 == 3) MOE_ROUTER(3);
    else MOE_ROUTER(4);
  }
#undef MOE_ROUTER
  return hipGetLastError();
}

hipError_t launch_colsum(const Shape& s, const float* prob_part, float* colsum, hipStream_t st) {
  colsum_kernel<<<s.E, 256, 0, st>>>(prob_part, router_blocks(s), s.E, colsum);
  return hipGetLastError();
}

}  // namespace moe
