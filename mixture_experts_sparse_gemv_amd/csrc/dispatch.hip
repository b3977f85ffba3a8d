// Capacity-limited dispatch ("MoE架构解析", 三 关键技术①) and the load-balance
// statistics (0539edu 2.3; kamacoder 七).
//
// Dispatch is a stable counting sort of the T*k assignments a = t*k + s by
// expert, done by one block of 16 waves so that the order is fixed without
// any inter-block protocol:
//   1. the expert ids of a segment of up to 64K assignments are staged in LDS
//      as bytes;
//   2. each wave walks a contiguous range in chunks of 64; a lane finds the
//      lanes holding the same expert with six ballots (one per bit of the
//      id), its rank among them is a popcount of the lower lanes, and the
//      group's first lane adds the group size to the wave's running count of
//      that expert (LDS, no atomics);
//   3. counts -> kept = min(count, capacity) -> offsets (exclusive scan) and
//      the start of each expert's dropped group;
//   4. a second walk recomputes the same ranks and scatters: rank < kept
//      gives row offsets[e] + rank, otherwise the assignment is dropped.
// Ranks are therefore the token order within each expert, so an expert keeps
// its C lowest-token assignments, bit-exactly.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int DW = 16;               // waves
constexpr int DT = DW * 64;          // threads
constexpr int SEG = 65536;           // assignments staged in LDS per segment

struct DispatchArgs {
  const int32_t* topk_idx;
  int32_t *counts, *kept, *offsets, *sorted_assign, *assign_row;
  uint8_t* drop_mask;
  const float* prob_part;   // null: no aux statistics
  float *colsum, *f, *P, *l_aux;
  int T, k, E, cap, nblk;
};

// Lanes of this wave whose (valid) key equals mine.
__device__ __forceinline__ uint64_t match_lanes(int e, bool valid) {
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 6; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

__global__ __launch_bounds__(DT) void dispatch_kernel(DispatchArgs a) {
  __shared__ uint8_t ids[SEG];
  __shared__ int run[DW][kMaxExperts];      // per-wave running counts
  __shared__ int base[DW][kMaxExperts];     // per-wave base rank in the current segment
  __shared__ int total_run[kMaxExperts];    // counts of earlier segments
  __shared__ int cnt_s[kMaxExperts], kept_s[kMaxExperts], off_s[kMaxExperts + 1],
      drop_s[kMaxExperts];
  __shared__ float tmp[DW][kMaxExperts];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E;
  const long long n = (long long)a.T * a.k;
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  auto stage = [&](long long s0, int len) {
    for (int i = tid; i < len; i += DT) {
      int e = a.topk_idx[s0 + i];
      e = e < 0 ? 0 : (e >= E ? E - 1 : e);   // out-of-range ids are clamped
      ids[i] = (uint8_t)e;
    }
  };
  // Count a segment per wave into run[wave][*] (which the caller zeroed).
  auto count_segment = [&](int len) {
    const int per = ((len + DW * 64 - 1) / (DW * 64)) * 64;
    const int lo = wave * per, hi = min(len, lo + per);
    for (int c = lo; c < hi; c += 64) {
      const int i = c + lane;
      const bool valid = i < hi;
      const int e = valid ? ids[i] : 0;
      const uint64_t m = match_lanes(e, valid);
      if (valid && (m & lower) == 0) run[wave][e] += __popcll(m);
    }
  };

  // ---- pass 1: counts
  if (tid < kMaxExperts) total_run[tid] = 0;
  for (long long s0 = 0; s0 < n; s0 += SEG) {
    const int len = (int)((n - s0) < SEG ? (n - s0) : SEG);
    for (int i = tid; i < DW * kMaxExperts; i += DT) run[i / kMaxExperts][i % kMaxExperts] = 0;
    stage(s0, len);
    __syncthreads();
    count_segment(len);
    __syncthreads();
    if (tid < E) {
      int c = 0;
      for (int w = 0; w < DW; ++w) c += run[w][tid];
      total_run[tid] += c;
    }
    __syncthreads();
  }
  if (tid == 0) {
    int off = 0;
    for (int e = 0; e < E; ++e) {
      const int c = total_run[e];
      const int kk = (a.cap > 0 && c > a.cap) ? a.cap : c;
      cnt_s[e] = c;
      kept_s[e] = kk;
      off_s[e] = off;
      off += kk;
    }
    off_s[E] = off;
    int d = off;
    for (int e = 0; e < E; ++e) {
      drop_s[e] = d;
      d += cnt_s[e] - kept_s[e];
    }
  }
  __syncthreads();
  if (tid < E) {
    if (a.counts) a.counts[tid] = cnt_s[tid];
    if (a.kept) a.kept[tid] = kept_s[tid];
    total_run[tid] = 0;
  }
  if (tid <= E && a.offsets) a.offsets[tid] = off_s[tid];

  // ---- pass 2: ranks and scatter
  for (long long s0 = 0; s0 < n; s0 += SEG) {
    const int len = (int)((n - s0) < SEG ? (n - s0) : SEG);
    __syncthreads();
    for (int i = tid; i < DW * kMaxExperts; i += DT) run[i / kMaxExperts][i % kMaxExperts] = 0;
    stage(s0, len);
    __syncthreads();
    count_segment(len);
    __syncthreads();
    if (tid < E) {   // per-wave base ranks: earlier segments + earlier waves
      int b = total_run[tid];
      for (int w = 0; w < DW; ++w) {
        base[w][tid] = b;
        b += run[w][tid];
        run[w][tid] = 0;
      }
      total_run[tid] = b;
    }
    __syncthreads();
    const int per = ((len + DW * 64 - 1) / (DW * 64)) * 64;
    const int lo = wave * per, hi = min(len, lo + per);
    for (int c = lo; c < hi; c += 64) {
      const int i = c + lane;
      const bool valid = i < hi;
      const int e = valid ? ids[i] : 0;
      const uint64_t m = match_lanes(e, valid);
      if (valid) {
        const int rank = base[wave][e] + run[wave][e] + __popcll(m & lower);
        const long long asg = s0 + i;
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
      // every lane has read run[wave][e] above before the group's first lane updates it
      if (valid && (m & lower) == 0) run[wave][e] += __popcll(m);
    }
  }

  // ---- aux statistics (f, P, L_aux) when the router's partial sums are given
  if (a.prob_part) {
    const int e = tid & 63, j = tid >> 6;   // 16 strided partial sums per expert
    float v = 0.f;
    if (e < E)
      for (int b = j; b < a.nblk; b += DW) v += a.prob_part[(long long)b * E + e];
    tmp[j][e] = v;
    __syncthreads();
    if (tid < E) {
      float cs = 0.f;
      for (int jj = 0; jj < DW; ++jj) cs += tmp[jj][tid];
      const float fe = (float)cnt_s[tid] / (float)((long long)a.T * a.k);
      const float pe = cs / (float)a.T;
      if (a.colsum) a.colsum[tid] = cs;
      if (a.f) a.f[tid] = fe;
      if (a.P) a.P[tid] = pe;
      tmp[0][tid] = fe * pe;
    }
    __syncthreads();
    if (tid == 0 && a.l_aux) {
      float l = 0.f;
      for (int ee = 0; ee < E; ++ee) l += tmp[0][ee];
      a.l_aux[0] = (float)E * l;
    }
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

hipError_t launch_dispatch(const Shape& s, const int32_t* topk_idx, int32_t* counts,
                           int32_t* kept, int32_t* offsets, int32_t* sorted_assign,
                           int32_t* assign_row, uint8_t* drop_mask, const float* prob_part,
                           float* colsum, float* f, float* P, float* l_aux, hipStream_t st) {
  DispatchArgs a{topk_idx, counts, kept, offsets, sorted_assign, assign_row, drop_mask,
                 prob_part, colsum, f, P, l_aux, s.T, s.k, s.E, s.cap, router_blocks(s)};
  dispatch_kernel<<<1, DT, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_aux(const Shape& s, const float* colsum, const int32_t* counts, float* f,
                      float* P, float* l_aux, hipStream_t st) {
  aux_kernel<<<1, 64, 0, st>>>(colsum, counts, f, P, l_aux, s.T, s.k, s.E);
  return hipGetLastError();
}

}  // namespace moe
