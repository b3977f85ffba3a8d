// Capacity-limited dispatch ("MoE架构解析", 三 关键技术①) and the load-balance
// statistics (0539edu 2.3; kamacoder 七).
//
// Dispatch is a stable counting sort of the T*k assignments a = t*k + s by
// expert, in three kernels with no inter-block waiting:
//   1. per-chunk expert counts: chunk c = tokens 16c .. 16c+15 (the router
//      kernel writes them in the fused forward; chunk_count_kernel otherwise);
//   2. dispatch_scan_kernel (one block): sums the chunk counts of each
//      scatter block (512 tokens), turns them into per-block exclusive
//      prefixes per expert, and writes counts, kept = min(count, capacity),
//      offsets (exclusive scan of kept); with the router's per-block
//      probability sums it also reduces them in a fixed order and writes
//      colsum, f, P and L_aux;
//   3. dispatch_scatter_kernel (one block per 512 tokens): ranks each of its
//      assignments within its expert — the block's prefix, plus the counts
//      of earlier waves of the block, plus the lanes below it in its wave
//      holding the same expert (six bit-plane ballots) — and scatters:
//      rank < kept gives row offsets[e] + rank, otherwise the assignment is
//      dropped and goes after all kept rows, grouped by expert.
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

struct ScanArgs {
  const int32_t* chunk_counts;   // [nchunk, E]
  int32_t* sb_prefix;            // [nsb, E] out: per scatter block exclusive prefix
  int32_t *counts, *kept, *offsets;
  const float* prob_part;        // [nchunk, E] or null (no aux statistics)
  float *colsum, *f, *P, *l_aux;
  int T, k, E, cap, nchunk, nsb;
};

constexpr int PMAX = 32;   // per-thread probability partial sums prefetched

// ---- 2. one block: block prefixes, counts/kept/offsets, aux statistics
__global__ __launch_bounds__(ST) void dispatch_scan_kernel(ScanArgs a) {
  __shared__ int part[SW][kMaxExperts];
  __shared__ int tot_s[kMaxExperts];
  __shared__ float red[ST];
  const int tid = threadIdx.x;
  const int E = a.E;

  // prefetch the router's per-chunk probability sums: thread (pe, pj),
  // pe = tid % EP, sums chunks pj, pj + J, pj + 2J, ... in order
  const int EP = E <= 1 ? 1 : (E <= 2 ? 2 : (E <= 4 ? 4 : (E <= 8 ? 8 : (E <= 16 ? 16 : (E <= 32 ? 32 : 64)))));
  const int J = ST / EP;
  const int pe = tid % EP, pj = tid / EP;
  float pv[PMAX];
  int pcount = 0;
  if (a.prob_part && pe < E) {
#pragma unroll
    for (int q = 0; q < PMAX; ++q) {
      const int b = pj + q * J;
      pv[q] = (b < a.nchunk) ? a.prob_part[(long long)b * E + pe] : 0.f;
    }
    pcount = (a.nchunk + J - 1) / J;
  }

  // thread (e, j) owns the contiguous range [b0, b1) of scatter blocks
  const int e = tid & 63, j = tid >> 6;
  const int R = (a.nsb + SW - 1) / SW;
  const int b0 = j * R, b1 = min(a.nsb, b0 + R);
  constexpr int CPB = kScatterTokens / kRouterTokens;   // chunks per scatter block
  int acc = 0;
  if (e < E) {
    for (int b = b0; b < b1; ++b) {
      const int c0 = b * CPB, c1 = min(a.nchunk, c0 + CPB);
      int sum = 0;
      for (int c = c0; c < c1; ++c) sum += a.chunk_counts[(long long)c * E + e];
      a.sb_prefix[(long long)b * E + e] = sum;   // block sum; made a prefix below
      acc += sum;
    }
  }
  part[j][e] = acc;
  __syncthreads();
  if (tid < kMaxExperts) {
    int run = 0;
    for (int jj = 0; jj < SW; ++jj) {
      const int v = part[jj][tid];
      part[jj][tid] = run;
      run += v;
    }
    tot_s[tid] = run;
  }
  __syncthreads();
  if (e < E) {
    int run = part[j][e];
    for (int b = b0; b < b1; ++b) {
      const int v = a.sb_prefix[(long long)b * E + e];
      a.sb_prefix[(long long)b * E + e] = run;
      run += v;
    }
  }
  if (tid == 0) {
    int off = 0;
    for (int ee = 0; ee < E; ++ee) {
      const int c = tot_s[ee];
      const int kk = (a.cap > 0 && c > a.cap) ? a.cap : c;
      a.counts[ee] = c;
      a.kept[ee] = kk;
      a.offsets[ee] = off;
      off += kk;
    }
    a.offsets[E] = off;
  }

  // ---- aux statistics (f, P, L_aux) when the router's partial sums are given
  if (a.prob_part) {
    float v = 0.f;
    if (pe < E) {
#pragma unroll
      for (int q = 0; q < PMAX; ++q)
        if (q < pcount) v += pv[q];
      for (int b = pj + PMAX * J; b < a.nchunk; b += J) v += a.prob_part[(long long)b * E + pe];
    }
    red[tid] = v;
    __syncthreads();
    // fixed tree over j: red[j*EP + e] for j = 0..J-1
    for (int h = J / 2; h > 0; h >>= 1) {
      if (pj < h) red[tid] += red[tid + h * EP];
      __syncthreads();
    }
    if (tid < E) {
      const float cs = red[tid];
      const float fe = (float)tot_s[tid] / (float)((long long)a.T * a.k);
      const float pe_ = cs / (float)a.T;
      if (a.colsum) a.colsum[tid] = cs;
      if (a.f) a.f[tid] = fe;
      if (a.P) a.P[tid] = pe_;
      red[ST - 1 - tid] = fe * pe_;
    }
    __syncthreads();
    if (tid == 0 && a.l_aux) {
      float l = 0.f;
      for (int ee = 0; ee < E; ++ee) l += red[ST - 1 - ee];
      a.l_aux[0] = (float)E * l;
    }
  }
}

struct ScatterArgs {
  const int32_t* topk_idx;
  const int32_t *sb_prefix, *counts, *kept, *offsets;
  int32_t *sorted_assign, *assign_row;
  uint8_t* drop_mask;
  int T, k, E;
};

// ---- 3. ranks and scatter, one block per kScatterTokens tokens
__global__ __launch_bounds__(ST) void dispatch_scatter_kernel(ScatterArgs a) {
  __shared__ int kept_s[kMaxExperts], off_s[kMaxExperts], drop_s[kMaxExperts], run_s[kMaxExperts];
  __shared__ int wc[SW][kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E;
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (tid < E) {
    kept_s[tid] = a.kept[tid];
    off_s[tid] = a.offsets[tid];
    run_s[tid] = a.sb_prefix[(long long)blockIdx.x * E + tid];
  }
  if (tid == 0) {   // start of each expert's dropped group, after all kept rows
    int d = a.offsets[E];
    for (int e = 0; e < E; ++e) {
      drop_s[e] = d;
      d += a.counts[e] - a.kept[e];
    }
  }
  __syncthreads();
  const long long n = (long long)a.T * a.k;
  const long long A0 = (long long)blockIdx.x * kScatterTokens * a.k;
  const long long A1 = A0 + (long long)kScatterTokens * a.k < n ? A0 + (long long)kScatterTokens * a.k : n;
  for (long long p0 = A0; p0 < A1; p0 += ST) {
    const long long asg = p0 + tid;
    const bool valid = asg < A1;
    const int e = valid ? clamp_id(a.topk_idx[asg], E) : 0;
    const Bits r = ballots(e, valid);
    const int rank_w = __popcll(lanes_with(r, e) & lower);
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
      const int rank = wc[wave][e] + rank_w;
      int row;
      if (rank < kept_s[e]) {
        row = off_s[e] + rank;
        a.assign_row[asg] = row;
        if (a.drop_mask) a.drop_mask[asg] = 0;
      } else {
        row = drop_s[e] + (rank - kept_s[e]);
        a.assign_row[asg] = -1;
        if (a.drop_mask) a.drop_mask[asg] = 1;
      }
      a.sorted_assign[row] = (int32_t)asg;
    }
    __syncthreads();   // wc is rewritten by the next pass
  }
}

// f, P, L_aux from given column sums and counts (one block).
__global__ __launch_bounds__(64) void aux_kernel(const float* colsum, const int32_t* counts,
                                                 float* f, float* P, float* l_aux, int T, int k,
                                                 int E) {
  __shared__ float prod[kMaxExperts];
  const int e = threadIdx.x;
  if (e < E) {
    const float fe = (float)counts[e] / (float)((long long)T * k);
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
                           bool counted, int32_t* sb_prefix, int32_t* counts, int32_t* kept,
                           int32_t* offsets, int32_t* sorted_assign, int32_t* assign_row,
                           uint8_t* drop_mask, const float* prob_part, float* colsum, float* f,
                           float* P, float* l_aux, hipStream_t st) {
  const int nchunk = router_blocks(s), nsb = scatter_blocks(s);
  if (!counted) {
    chunk_count_kernel<<<(nchunk + 3) / 4, 256, 0, st>>>(topk_idx, chunk_counts, s.T, s.k, s.E,
                                                         nchunk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  ScanArgs sa{chunk_counts, sb_prefix, counts, kept, offsets, prob_part, colsum, f, P, l_aux,
              s.T, s.k, s.E, s.cap, nchunk, nsb};
  dispatch_scan_kernel<<<1, ST, 0, st>>>(sa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ScatterArgs ca{topk_idx, sb_prefix, counts, kept, offsets, sorted_assign, assign_row, drop_mask,
                 s.T, s.k, s.E};
  dispatch_scatter_kernel<<<nsb, ST, 0, st>>>(ca);
  return hipGetLastError();
}

hipError_t launch_aux(const Shape& s, const float* colsum, const int32_t* counts, float* f,
                      float* P, float* l_aux, hipStream_t st) {
  aux_kernel<<<1, 64, 0, st>>>(colsum, counts, f, P, l_aux, s.T, s.k, s.E);
  return hipGetLastError();
}

}  // namespace moe
