// Capacity-limited dispatch ("MoE架构解析", 三 关键技术①) and the load-balance
// statistics (0539edu 2.3; kamacoder 七).
//
// Dispatch is a stable counting sort of the T*k assignments a = t*k + s by
// expert, in two kernels with no inter-block waiting:
//   1. per-chunk expert counts: chunk c = tokens 16c .. 16c+15 (the router
//      kernel writes them in the fused forward; chunk_count_kernel otherwise);
//   2. dispatch_kernel (one block per 512 tokens): from the chunk counts
//      each block forms the expert totals (so kept = min(count, capacity)
//      and the row offsets, an exclusive scan of kept) and its own base
//      ranks, then ranks and scatters its assignments; block 0 writes
//      counts, kept and offsets.  Given the router's per-chunk probability
//      sums, one extra block (the last) forms the totals the same way and
//      reduces them in a fixed order to colsum, f, P and L_aux, beside the
//      scatter rather than after block 0's share of it.
// Ranks are the token order within each expert, so an expert keeps its C
// lowest-token assignments, bit-exactly and independently of scheduling.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int SW = 16;               // waves of the scan and scatter blocks
constexpr int ST = SW * 64;          // threads

struct Bits {   // the bit-plane ballots of one chunk of 64 ids
  uint64_t valid, b[6];
};
__device__ __forceinline__ Bits ballots(int e, bool valid) {
  Bits r;
  r.valid = __ballot(valid);
#pragma unroll
  for (int i = 0; i < 6; ++i) r.b[i] = __ballot(valid && ((e >> i) & 1));
  return r;
}
// Valid lanes of the chunk whose id equals `key`.
__device__ __forceinline__ uint64_t lanes_with(const Bits& r, int key) {
  uint64_t m = r.valid;
#pragma unroll
  for (int i = 0; i < 6; ++i) m &= ((key >> i) & 1) ? r.b[i] : ~r.b[i];
  return m;
}
// Expert ids outside [0, E) are clamped (the router never produces them).
__device__ __forceinline__ int clamp_id(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

// ---- 1. counts of each 16-token chunk: one wave per chunk, lane e counts e
__global__ __launch_bounds__(256) void chunk_count_kernel(const int32_t* __restrict__ topk_idx,
                                                          int32_t* __restrict__ chunk_counts,
                                                          int T, int k, int E, int nchunk) {
  const int lane = threadIdx.x & 63;
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (c >= nchunk) return;
  const long long n = (long long)T * k;
  const long long a0 = (long long)c * kRouterTokens * k;
  const long long a1 = a0 + (long long)kRouterTokens * k < n ? a0 + (long long)kRouterTokens * k : n;
  int cnt = 0;
  for (long long b = a0; b < a1; b += 64) {
    const long long i = b + lane;
    const bool valid = i < a1;
    const int e = valid ? clamp_id(topk_idx[i], E) : 0;
    cnt += __popcll(lanes_with(ballots(e, valid), lane));
  }
  if (lane < E) chunk_counts[(long long)c * E + lane] = cnt;
}

// Routing health indicators (moe_route_stats) computed by one wave, lane e
// holding expert e's routed count c, kept count kp and mean probability pe
// (lanes >= E pass zeros).  Wave sums run in a fixed xor-butterfly order.
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ void route_stats_wave(int lane, int E, int c, int kp, float pe, moe_route_stats* out) {
  const bool on = lane < E;
  const int total = wave_sum_i(on ? c : 0);
  const float share = (on && total > 0) ? (float)c / (float)total : 0.f;
  const float h = wave_sum_f(share > 0.f ? -share * logf(share) : 0.f);
  const float hp = wave_sum_f((on && pe > 0.f) ? -pe * logf(pe) : 0.f);
  const float mean = (float)wave_sum_i(on ? kp : 0) / (float)E;
  const float dv = on ? (float)kp - mean : 0.f;
  const float var = wave_sum_f(dv * dv) / (float)E;
  const int dropped = wave_sum_i(on ? c - kp : 0);
  const int idle = wave_sum_i((on && kp == 0) ? 1 : 0);
  if (lane == 0) {
    out->entropy = h;
    out->entropy_p = hp;
    out->entropy_max = logf((float)E);
    out->util_mean = mean;
    out->util_var = var;
    out->util_cv = mean > 0.f ? sqrtf(var) / mean : 0.f;
    out->dropped = dropped;
    out->idle = idle;
  }
}

struct DispatchArgs {
  const int32_t* topk_idx;
  const int32_t* chunk_counts;   // [nchunk, E]
  int32_t *counts, *kept, *offsets;
  int32_t *sorted_assign, *assign_row;
  uint8_t* drop_mask;
  const float* prob_part;        // [nchunk, E] or null (no aux statistics)
  float *colsum, *f, *P, *l_aux;
  moe_route_stats* stats;        // or null
  int T, k, E, cap, nchunk;
};

constexpr int PMAX = 32;   // per-thread probability partial sums prefetched

// Aux statistics (the extra last block): colsum, f, P, L_aux and the routing health
// indicators from the router's per-chunk probability sums and the routed
// counts tot_s.  Sums run per thread in chunk order, over the wave's j in
// xor-butterfly order, then over the waves in order.  Thread (e, j) as in
// dispatch_kernel.
__device__ void aux_block(const DispatchArgs& a, const int* tot_s, int e, int j, int EP, int J,
                          float (*wsum)[kMaxExperts], int* scratch) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E;
  const bool act = e < E;
  float v = 0.f;
  if (act) {
    float pv[PMAX];
#pragma unroll
    for (int q = 0; q < PMAX; ++q) {   // independent loads, all in flight
      const int b = j + q * J;
      pv[q] = (b < a.nchunk) ? a.prob_part[(long long)b * E + e] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < PMAX; ++q) v += pv[q];
    for (int b = j + PMAX * J; b < a.nchunk; b += J) v += a.prob_part[(long long)b * E + e];
  }
  for (int o = EP; o < 64; o <<= 1) v += __shfl_xor(v, o);
  if (lane < EP) wsum[wave][lane] = v;
  __syncthreads();
  float pe = 0.f;
  if (tid < E) {
    float cs = 0.f;
    for (int w = 0; w < SW; ++w) cs += wsum[w][tid];
    const float fe = (float)tot_s[tid] / (float)((long long)a.T * a.k);
    pe = cs / (float)a.T;
    if (a.colsum) a.colsum[tid] = cs;
    if (a.f) a.f[tid] = fe;
    if (a.P) a.P[tid] = pe;
    scratch[tid] = __float_as_int(fe * pe);
  }
  if (wave == 0 && a.stats) {
    const int c = lane < E ? tot_s[lane] : 0;
    route_stats_wave(lane, E, c, (a.cap > 0 && c > a.cap) ? a.cap : c, pe, a.stats);
  }
  __syncthreads();
  if (tid == 0 && a.l_aux) {
    float l = 0.f;
    for (int ee = 0; ee < E; ++ee) l += __int_as_float(scratch[ee]);
    a.l_aux[0] = (float)E * l;
  }
}

// ---- 2. one block per kScatterTokens tokens.  Each block sums the chunk
// counts itself: over all chunks (the expert totals, hence kept = min(total,
// capacity) and the row offsets) and over the chunks before its tokens (its
// base ranks).  It then ranks each of its assignments within its expert —
// base rank, plus the counts of earlier waves and passes of the block, plus
// the lanes below it in its wave holding the same expert (six bit-plane
// ballots) — and scatters: rank < kept gives row offsets[e] + rank,
// otherwise the assignment is dropped and goes after all kept rows, grouped
// by expert.  Block 0 also writes counts, kept and offsets.  Given the
// router's probability sums, the grid has one more block, which computes
// the aux statistics and scatters nothing.
// Thread (e, j) = (tid % EP, tid / EP) while summing, EP = E rounded up to a
// power of two, J = ST / EP threads per expert.
__global__ __launch_bounds__(ST) void dispatch_kernel(DispatchArgs a) {
  __shared__ int sp[ST], stot[ST];
  __shared__ int kept_s[kMaxExperts], off_s[kMaxExperts], drop_s[kMaxExperts], run_s[kMaxExperts];
  __shared__ int tot_s[kMaxExperts];
  __shared__ int wc[SW][kMaxExperts];
  __shared__ float wsum[SW][kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E;
  const long long n = (long long)a.T * a.k;
  // with aux statistics the last block computes them and scatters nothing
  const bool aux_blk = a.prob_part && blockIdx.x == gridDim.x - 1;
  const long long A0 = aux_blk ? n : (long long)blockIdx.x * kScatterTokens * a.k;
  const long long A1 = A0 + (long long)kScatterTokens * a.k < n ? A0 + (long long)kScatterTokens * a.k : n;
  // this block's expert ids, loaded before anything waits
  constexpr int MAXP = kScatterTokens * kMaxTopK / ST;   // passes of ST assignments
  int ids[MAXP];
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    const long long asg = A0 + (long long)p * ST + tid;
    ids[p] = asg < A1 ? clamp_id(a.topk_idx[asg], E) : -1;
  }

  // expert totals and this block's base ranks from the chunk counts
  const int EP = E <= 1 ? 1 : (E <= 2 ? 2 : (E <= 4 ? 4 : (E <= 8 ? 8 : (E <= 16 ? 16 : (E <= 32 ? 32 : 64)))));
  const int J = ST / EP;
  const int e = tid % EP, j = tid / EP;
  const int cb = blockIdx.x * (kScatterTokens / kRouterTokens);   // chunks before this block
  int pre = 0, tot = 0;
  if (e < E) {
    constexpr int U = 8;
    int c = j;
    for (; c + (U - 1) * J < a.nchunk; c += U * J) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = a.chunk_counts[(long long)(c + u * J) * E + e];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        tot += v[u];
        if (c + u * J < cb) pre += v[u];
      }
    }
    for (; c < a.nchunk; c += J) {
      const int v = a.chunk_counts[(long long)c * E + e];
      tot += v;
      if (c < cb) pre += v;
    }
  }
  sp[tid] = pre;
  stot[tid] = tot;
  __syncthreads();
  for (int o = J >> 1; o >= 1; o >>= 1) {   // integer sums: exact in any order
    if (j < o) {
      sp[tid] += sp[tid + o * EP];
      stot[tid] += stot[tid + o * EP];
    }
    __syncthreads();
  }
  if (wave == 0) {   // lane e: kept count, row offset, base rank, dropped start
    const int c = lane < E ? stot[lane] : 0;
    const int kp = (a.cap > 0 && c > a.cap) ? a.cap : c;
    int incl = kp;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o);
      if (lane >= o) incl += u;
    }
    const int offE = __shfl(incl, 63);
    const int dc = c - kp;
    int dincl = dc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(dincl, o);
      if (lane >= o) dincl += u;
    }
    if (lane < E) {
      tot_s[lane] = c;
      kept_s[lane] = kp;
      off_s[lane] = incl - kp;
      run_s[lane] = sp[lane];
      drop_s[lane] = offE + dincl - dc;   // dropped groups follow all kept rows, by expert
      if (blockIdx.x == 0) {
        a.counts[lane] = c;
        a.kept[lane] = kp;
        a.offsets[lane] = incl - kp;
      }
    }
    if (blockIdx.x == 0 && lane == 0) a.offsets[E] = offE;
  }
  __syncthreads();
  if (aux_blk) {   // uniform over the block
    aux_block(a, tot_s, e, j, EP, J, wsum, sp);
    return;
  }

  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    const long long p0 = A0 + (long long)p * ST;
    if (p0 >= A1) break;   // uniform
    const long long asg = p0 + tid;
    const bool valid = ids[p] >= 0;
    const int ee = valid ? ids[p] : 0;
    const Bits r = ballots(ee, valid);
    const int rank_w = __popcll(lanes_with(r, ee) & lower);
    wc[wave][lane] = __popcll(lanes_with(r, lane));
    __syncthreads();
    if (tid < E) {   // per-wave base ranks: earlier blocks and passes, then earlier waves
      int run = run_s[tid];
      for (int w = 0; w < SW; ++w) {
        const int v = wc[w][tid];
        wc[w][tid] = run;
        run += v;
      }
      run_s[tid] = run;
    }
    __syncthreads();
    if (valid) {
      const int rank = wc[wave][ee] + rank_w;
      int row;
      if (rank < kept_s[ee]) {
        row = off_s[ee] + rank;
        a.assign_row[asg] = row;
        if (a.drop_mask) a.drop_mask[asg] = 0;
      } else {
        row = drop_s[ee] + (rank - kept_s[ee]);
        a.assign_row[asg] = -1;
        if (a.drop_mask) a.drop_mask[asg] = 1;
      }
      a.sorted_assign[row] = (int32_t)asg;
    }
    __syncthreads();   // wc is rewritten by the next pass
  }
}

// Routing health indicators from given counts, kept and P (one wave).
__global__ __launch_bounds__(64) void routing_stats_kernel(const int32_t* counts,
                                                           const int32_t* kept, const float* P,
                                                           int E, moe_route_stats* out) {
  const int lane = threadIdx.x;
  const bool on = lane < E;
  route_stats_wave(lane, E, on ? counts[lane] : 0, on ? kept[lane] : 0, on ? P[lane] : 0.f, out);
}

// f, P, L_aux from given column sums and counts (one block).
__global__ __launch_bounds__(64) void aux_kernel(const float* colsum, const int32_t* counts,
                                                 float* f, float* P, float* l_aux, int T,
                                                 long long total, int E) {
  __shared__ float prod[kMaxExperts];
  const int e = threadIdx.x;
  if (e < E) {
    const float fe = (float)counts[e] / (float)total;   // share of the routing decisions
    const float pe = colsum[e] / (float)T;
    f[e] = fe;
    P[e] = pe;
    prod[e] = fe * pe;
  }
  __syncthreads();
  if (e == 0) {
    float l = 0.f;
    for (int i = 0; i < E; ++i) l += prod[i];
    l_aux[0] = (float)E * l;
  }
}

}  // namespace

hipError_t launch_dispatch(const Shape& s, const int32_t* topk_idx, int32_t* chunk_counts,
                           bool counted, int32_t* counts, int32_t* kept, int32_t* offsets,
                           int32_t* sorted_assign, int32_t* assign_row, uint8_t* drop_mask,
                           const float* prob_part, float* colsum, float* f, float* P,
                           float* l_aux, moe_route_stats* stats, hipStream_t st) {
  const int nchunk = router_blocks(s), nsb = scatter_blocks(s);
  if (!counted) {
    chunk_count_kernel<<<(nchunk + 3) / 4, 256, 0, st>>>(topk_idx, chunk_counts, s.T, s.k, s.E,
                                                         nchunk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  DispatchArgs da{topk_idx, chunk_counts, counts, kept, offsets, sorted_assign, assign_row,
                  drop_mask, prob_part, colsum, f, P, l_aux, prob_part ? stats : nullptr,
                  s.T, s.k, s.E, s.cap, nchunk};
  dispatch_kernel<<<nsb + (prob_part ? 1 : 0), ST, 0, st>>>(da);
  return hipGetLastError();
}

hipError_t launch_aux(const Shape& s, const float* colsum, const int32_t* counts, float* f,
                      float* P, float* l_aux, hipStream_t st) {
  aux_kernel<<<1, 64, 0, st>>>(colsum, counts, f, P, l_aux, s.T, s.routed_rows(), s.E);
  return hipGetLastError();
}

hipError_t launch_routing_stats(const Shape& s, const int32_t* counts, const int32_t* kept,
                                const float* P, moe_route_stats* stats, hipStream_t st) {
  routing_stats_kernel<<<1, 64, 0, st>>>(counts, kept, P, s.E, stats);
  return hipGetLastError();
}

}  // namespace moe
