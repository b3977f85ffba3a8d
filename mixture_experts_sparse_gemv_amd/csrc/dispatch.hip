// Capacity-limited dispatch ("MoE架构解析", 三 关键技术①) and the load-balance
// statistics (0539edu 2.3; kamacoder 七).
//
// Dispatch is a stable counting sort of the T*k assignments a = t*k + s by
// expert, done by one block of 16 waves so that the order is fixed without
// any inter-block protocol:
//   1. the expert ids of a segment of up to 64K assignments are staged in LDS
//      as bytes;
//   2. each wave walks a contiguous range in chunks of 64; six ballots (one
//      per bit of the id) give every lane the set of lanes holding its expert
//      (its rank in the chunk is a popcount of the lower ones) and the set
//      holding expert `lane`; lane e keeps the wave's running count of
//      expert e in a register, and a lane reads its own expert's count with a
//      lane shuffle;
//   3. counts -> kept = min(count, capacity) -> offsets (exclusive scan) and
//      the start of each expert's dropped group;
//   4. a second walk recomputes the same ranks and scatters: rank < kept
//      gives row offsets[e] + rank, otherwise the assignment is dropped.
// Ranks are therefore the token order within each expert, so an expert keeps
// its C lowest-token assignments, bit-exactly.
//
// With the router's per-block probability sums given, the kernel also
// reduces them (loads issued first, summed in a fixed tree order at the end)
// and writes f, P and L_aux.
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

constexpr int PMAX = 32;   // per-thread probability partial sums prefetched

__global__ __launch_bounds__(DT) void dispatch_kernel(DispatchArgs a) {
  __shared__ uint8_t ids[SEG];
  __shared__ int wcnt[DW][kMaxExperts];     // per-wave counts of the current segment
  __shared__ int base[DW][kMaxExperts];     // per-wave base rank in the current segment
  __shared__ int total_run[kMaxExperts];    // counts of earlier segments
  __shared__ int cnt_s[kMaxExperts], kept_s[kMaxExperts], off_s[kMaxExperts + 1],
      drop_s[kMaxExperts];
  __shared__ float red[DT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E;
  const long long n = (long long)a.T * a.k;
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  // ---- prefetch the router's per-block probability sums (aux statistics):
  // thread (e, j), e = tid % EP, sums blocks j, j + J, j + 2J, ... in order.
  const int EP = E <= 1 ? 1 : (E <= 2 ? 2 : (E <= 4 ? 4 : (E <= 8 ? 8 : (E <= 16 ? 16 : (E <= 32 ? 32 : 64)))));
  const int J = DT / EP;
  const int pe = tid % EP, pj = tid / EP;
  float pv[PMAX];
  int pcount = 0;
  if (a.prob_part && pe < E) {
#pragma unroll
    for (int q = 0; q < PMAX; ++q) {
      const int b = pj + q * J;
      pv[q] = (b < a.nblk) ? a.prob_part[(long long)b * E + pe] : 0.f;
    }
    pcount = (a.nblk + J - 1) / J;
  }

  auto stage = [&](long long s0, int len) {
    const int* src = a.topk_idx + s0;
    int i = tid;
    for (; i + 7 * DT < len; i += 8 * DT) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = src[i + u * DT];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = v[u] < 0 ? 0 : (v[u] >= E ? E - 1 : v[u]);   // out-of-range ids are clamped
        ids[i + u * DT] = (uint8_t)e;
      }
    }
    for (; i < len; i += DT) {
      const int e = src[i] < 0 ? 0 : (src[i] >= E ? E - 1 : src[i]);
      ids[i] = (uint8_t)e;
    }
  };
  // This wave's counts of each expert over its range of the segment: lane e
  // returns the count of expert e.
  auto count_segment = [&](int len) {
    const int per = ((len + DW * 64 - 1) / (DW * 64)) * 64;
    const int lo = wave * per, hi = min(len, lo + per);
    int cnt = 0;
    for (int c = lo; c < hi; c += 64) {
      const int i = c + lane;
      const bool valid = i < hi;
      const int e = valid ? ids[i] : 0;
      const Bits r = ballots(e, valid);
      cnt += __popcll(lanes_with(r, lane));
    }
    return cnt;
  };

  // ---- pass 1: counts
  if (tid < kMaxExperts) total_run[tid] = 0;
  for (long long s0 = 0; s0 < n; s0 += SEG) {
    const int len = (int)((n - s0) < SEG ? (n - s0) : SEG);
    stage(s0, len);
    __syncthreads();
    wcnt[wave][lane] = count_segment(len);
    __syncthreads();
    if (tid < E) {
      int c = 0;
      for (int w = 0; w < DW; ++w) c += wcnt[w][tid];
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
    stage(s0, len);
    __syncthreads();
    wcnt[wave][lane] = count_segment(len);
    __syncthreads();
    if (tid < E) {   // per-wave base ranks: earlier segments + earlier waves
      int b = total_run[tid];
      for (int w = 0; w < DW; ++w) {
        base[w][tid] = b;
        b += wcnt[w][tid];
      }
      total_run[tid] = b;
    }
    __syncthreads();
    const int per = ((len + DW * 64 - 1) / (DW * 64)) * 64;
    const int lo = wave * per, hi = min(len, lo + per);
    int run = lane < kMaxExperts ? base[wave][lane] : 0;   // lane e: next rank of expert e
    for (int c = lo; c < hi; c += 64) {
      const int i = c + lane;
      const bool valid = i < hi;
      const int e = valid ? ids[i] : 0;
      const Bits r = ballots(e, valid);
      const int before = __shfl(run, e);
      if (valid) {
        const int rank = before + __popcll(lanes_with(r, e) & lower);
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
      run += __popcll(lanes_with(r, lane));
    }
  }

  // ---- aux statistics (f, P, L_aux) when the router's partial sums are given
  if (a.prob_part) {
    float v = 0.f;
    if (pe < E) {
#pragma unroll
      for (int q = 0; q < PMAX; ++q)
        if (q < pcount) v += pv[q];
      for (int b = pj + PMAX * J; b < a.nblk; b += J) v += a.prob_part[(long long)b * E + pe];
    }
    __syncthreads();
    red[tid] = v;
    __syncthreads();
    // fixed tree over j: red[j*EP + e] for j = 0..J-1
    for (int h = J / 2; h > 0; h >>= 1) {
      if (pj < h) red[tid] += red[tid + h * EP];
      __syncthreads();
    }
    if (tid < E) {
      const float cs = red[tid];
      const float fe = (float)cnt_s[tid] / (float)((long long)a.T * a.k);
      const float pe_ = cs / (float)a.T;
      if (a.colsum) a.colsum[tid] = cs;
      if (a.f) a.f[tid] = fe;
      if (a.P) a.P[tid] = pe_;
      red[DT - 1 - tid] = fe * pe_;
    }
    __syncthreads();
    if (tid == 0 && a.l_aux) {
      float l = 0.f;
      for (int ee = 0; ee < E; ++ee) l += red[DT - 1 - ee];
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
