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
// Dense contractions, so they run on the matrix cores: bf16 MFMAs for the up
// projection, fp16 MFMAs for the down projection (h is fp16; each bf16 W2
// fragment is converted to fp16 in registers after its LDS read).
// Accumulation is fp32.  Block = 8 waves (WGM x WGN grid); block tile BM
// token rows x BN weight rows (256 x 256).  Two main loops: 16x16x32 MFMAs
// over 64-deep k-tiles in a 2-stage LDS ring (the DMA one k-tile ahead), for
// the up projection and long down-style launches; 32x32x16 MFMAs over
// 32-deep k-tiles in a 4-stage ring (the DMA three k-tiles ahead), for short
// ones.  Both accumulate every output in the same order (bit-identical
// results).  The ring is filled by direct global-to-LDS DMA, with an XOR
// swizzle of the 16-byte chunks that keeps fragment reads conflict-free.
// The MFMA "A" operand is the weight tile and "B" the token tile, so each
// lane's accumulators hold four consecutive output columns of one token row;
// the epilogue stages each wave's rows in LDS and stores whole row segments.
//
// The tile schedule is computed on the device from offsets[] (no host sync):
// every block derives the per-segment m-tile counts, their prefix sum, and its
// own (segment, n-tile, m-tile).  Block ids are remapped so that each of the 8
// XCDs (block b runs on XCD b % 8) gets a contiguous range of tiles: the tiles
// of one expert weight stay within one XCD's L2.  The launch is persistent
// (at most one block per compute unit, looping over its tiles), and a block's
// consecutive tiles overlap: the next tile's first k-tile loads while the
// current tile's epilogue runs.
#include <atomic>

#include "moe_internal.h"

// 1: a k-substep's fragment reads are issued first, MOE_SCHED_PER per MFMA,
// then the DMA; 0: one DMA and one fragment read after each MFMA.
#ifndef MOE_SCHED_FRONT
#define MOE_SCHED_FRONT 1
#endif
#ifndef MOE_SCHED_PER
#define MOE_SCHED_PER 2   // fragment reads per MFMA at the start of a k-substep
#endif

namespace moe {
namespace {

// Up projection with activation (RELU/GELU/SWIGLU, fp16 h out), down
// projection (DOWN: fp16 h times W2 converted to fp16, fp32 out).  The
// backward pass adds: LIN, gathered token rows times bf16 weights with an
// optional bias and fp32 out (no activation); DXB, like DOWN with bf16 rows
// and weights; WGRAD, the per-expert weight gradient, whose reduction runs
// over the expert's rows (see wgrad_* below).
enum {
  MODE_RELU = 0, MODE_GELU = 1, MODE_SWIGLU = 2, MODE_DOWN = 3, MODE_LIN = 4, MODE_DXB = 5,
  MODE_WGRAD = 6
};

struct GemmArgs {
  const uint16_t* X;       // up: x [T, K] bf16; down: h [rows, K] fp16
  const uint16_t* W;       // [segments][Wrows][K] bf16
  const uint16_t* bias;    // [segments][Wrows] bf16, or null
  void* out;               // up: h [rows, Nout] fp16; down: y_exp [rows, Nout] fp32
  const int32_t* offsets;  // [E + 1]
  const int32_t* sorted_assign;
  int T, k, E, S, K, Nout, Wrows, f;
  // DOWN / DXB: K slices; slice i > 0 writes to out2 + (i - 1) * part_elems
  int ksplit;
  float* out2;
  long long part_elems;
  // WGRAD: out[seg] = A_seg B_seg^T, [M, Nout] fp32, with A = X [M, K] and
  // B = W [Nout, K] (row stride K); segment seg reduces over its padded row
  // range of the columns (wgrad_pad / wgrad_poff)
  int M;
  // Bytes of X.  Below 2 GiB, the token-row loads of rows past a tile's
  // valid rows carry an out-of-range buffer offset (0x80000000): the
  // hardware returns zeros without reading memory, so ragged tiles fetch only
  // their valid rows.  Otherwise such rows repeat the last valid row.
  long long xbytes;
};

constexpr uint32_t kNoRow = 0x80000000u;   // out-of-range buffer offset (zeros, no fetch)


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

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100, SG_DS_WRITE = 0x200;
#define SGB(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)

// NM MFMAs, each followed by one instruction of group A (NA in total) and
// one of group B (NB in total); leftovers of A and B follow the last MFMA.
// N instructions of group A, the first NB of them each followed by one of group B.
template <int N, int MA, int MB, int NB, int I = 0>
__device__ __forceinline__ void sched_interleave_pair() {
  if constexpr (I < N) {
    SGB(MA, 1);
    if constexpr (I < NB) SGB(MB, (I + 1 < N) ? 1 : NB - I);
    sched_interleave_pair<N, MA, MB, NB, I + 1>();
  }
}

// NM MFMAs; while group A lasts (NA in total), each MFMA is followed by up
// to PER of its instructions, then each by one of group B (NB in total);
// leftovers follow the last MFMA.  Front-loading the fragment reads gives
// them the remaining MFMAs of the substep to complete in.
template <int NM, int MA, int NA, int PER, int MB, int NB, int I = 0, int A = 0, int B = 0>
__device__ __forceinline__ void sched_front() {
  if constexpr (I < NM) {
    SGB(SG_MFMA, 1);
    constexpr bool last = I + 1 == NM;
    constexpr int a = last ? NA - A : (NA - A < PER ? NA - A : PER);
    if constexpr (a > 0) SGB(MA, a);
    constexpr int b = last ? NB - B : ((a == 0 && NB > B) ? 1 : 0);
    if constexpr (b > 0) SGB(MB, b);
    sched_front<NM, MA, NA, PER, MB, NB, I + 1, A + a, B + b>();
  }
}

template <int NM, int MA, int NA, int MB, int NB, int I = 0>
__device__ __forceinline__ void sched_interleave() {
  if constexpr (I < NM) {
    SGB(SG_MFMA, 1);
    if constexpr (I < NA) SGB(MA, (I + 1 < NM) ? 1 : NA - I);
    if constexpr (I < NB) SGB(MB, (I + 1 < NM) ? 1 : NB - I);
    sched_interleave<NM, MA, NA, MB, NB, I + 1>();
  }
}

// Coordinates of one block tile: K slice, segment, n-tile and m-tile, and the
// segment's row count and first row.
struct TileCoord {
  int ks, seg, nt, mt, rows, start;
};

// OCC: waves per SIMD the register budget must allow.  MF: the MFMA shape,
// 16 (16x16x32) or 32 (32x32x16).  BK: the k-tile depth, 32 (4-stage LDS
// ring) or, with 16x16x32, 64 (2-stage ring, whole 128-byte rows per DMA).
template <int BM, int BN, int WGM, int WGN, int MODE, int OCC = 1, int MF = 16, int BK = 32>
__global__ __launch_bounds__(64 * WGM * WGN, OCC) void grouped_gemm_kernel(GemmArgs a) {
  constexpr int NSTAGE = BK == 64 ? 2 : 4;   // LDS ring stages
  constexpr int NW = WGM * WGN;            // waves: WGM along tokens x WGN along weights
  constexpr bool SWIGLU = MODE == MODE_SWIGLU;
  constexpr bool GATHER = MODE <= MODE_SWIGLU || MODE == MODE_LIN;   // token rows via sorted_assign
  constexpr bool CVT16 = MODE == MODE_DOWN;      // fp16 rows: W converted bf16 -> fp16
  constexpr bool OUT32 = MODE >= MODE_DOWN;      // fp32 output (else fp16 h)
  constexpr bool KSPLIT = MODE == MODE_DOWN || MODE == MODE_DXB;
  constexpr bool WG = MODE == MODE_WGRAD;
  constexpr bool BIAS = !SWIGLU && !WG;         // an optional per-column bias
  constexpr int WM = BM / WGM, WN = BN / WGN;  // wave tile: token rows x weight rows
  constexpr int MI = WM / MF, NI = WN / MF;
  typedef float accv __attribute__((ext_vector_type(MF * MF / 64)));
  constexpr int NOUT_TILE = SWIGLU ? BN / 2 : BN;
  constexpr int ROWCH = BK / 8;            // 16-byte chunks per tile row
  constexpr int RPB = 16 / ROWCH;          // tile rows per 256 bytes (all 64 LDS banks)
  constexpr int RI = 64 / ROWCH;           // tile rows filled by one DMA instruction
  constexpr int NSUB = MF == 32 ? BK / 16 : BK / 32;   // MFMA k-substeps per k-tile
  constexpr int NFR = NI + MI;             // fragment reads per wave per k-substep
  constexpr int NM = NI * MI;              // MFMAs per wave per k-substep
  constexpr int QWW = BN / RI / NW, QWX = BM / RI / NW;   // DMA instructions per wave and k-tile
  constexpr int STAGE = (BM + BN) * ROWCH;                // 16-byte chunks per stage
  static_assert(MI >= 1 && NI >= 1 && QWW * RI * NW == BN && QWX * RI * NW == BM, "tile shape");
  static_assert(!SWIGLU || (NI % 2 == 0), "SwiGLU pairs gate and up sub-tiles");
  static_assert(MF == 16 || MF == 32, "MFMA shape");
  static_assert((MF == 16) == (BK == 64), "16x16x32 runs 64-deep k-tiles, 32x32x16 32-deep");
  // 32x32x16: the last of the k-substeps runs after the barrier; 16x16x32:
  // two 32-deep MFMA k-steps per k-tile (see below).
  static_assert(MF == 16 ? NSUB == 2 : NSUB >= 2, "k-substeps per k-tile");

  // Epilogue staging geometry (see the epilogue): each wave stages 32-row
  // slabs of its output, PITCH bytes per row, in the ring stages after the
  // first; with a 2-stage ring the waves that do not fit in stage 1 stage in
  // a small extra region.
  constexpr int NJ = SWIGLU ? NI / 2 : NI;
  constexpr int WNOUT = NJ * MF;                       // output columns of a wave
  constexpr int ES = OUT32 ? 4 : 2;                     // output element bytes
  constexpr int PITCH = WNOUT * ES + (OUT32 ? 16 : 8);  // staging row pitch, bytes
  constexpr int STG = 32 * PITCH;                       // staging bytes per wave
  constexpr int WPA = STAGE * 16 / STG;                 // waves per ring stage
  constexpr int XTRA = (NSTAGE == 2 && WPA < NW) ? (NW - WPA) * STG : 0;
  static_assert(WPA * (NSTAGE - 1) >= NW || NSTAGE == 2, "staging must fit in stages 1 to 3");

  // The LDS ring as distinct arrays: the compiler sees that the DMA into one
  // stage never aliases the fragment reads of another.
  __shared__ u32x4 lds0[STAGE], lds1[STAGE], lds2[NSTAGE > 2 ? STAGE : (XTRA + 15) / 16 + 1],
      lds3[NSTAGE > 3 ? STAGE : 1];
  __shared__ int seg_tile[kMaxSegments + 1];
  __shared__ int seg_nrows[kMaxSegments], seg_row0[kMaxSegments];
  __shared__ int sh_seg[2];
  __shared__ int sh_range[2];   // WGRAD: the tile range of this block's XCD
  __shared__ uint32_t sh_bias[BIAS ? BN / 2 : 1];   // the tile's bias columns, bf16 pairs

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Wave w sits on SIMD w % 4 and takes token-row block wm = w / WGN: the
  // two waves sharing a SIMD take different row blocks (w and w + 4), so on
  // a tile whose valid rows end in its first half every SIMD has one wave's
  // MFMAs to do (the waves past the last valid row skip their main loop).
  const int wm = wave / WGN, wn = wave % WGN;
  const int nseg = a.E + a.S;
  const int NT = (a.Nout + NOUT_TILE - 1) / NOUT_TILE;
  const int off_E = a.offsets[a.E];

  // ---- tile schedule (wave 0, 2 segments per lane): each segment's row
  // count and first row, and two prefix sums over the segments.  A tile whose
  // rows fill at most half of BM (a segment's last, ragged m-tile) keeps only
  // the waves of its first half busy, about half the time of a full tile: such
  // "light" tiles form a list of their own (seg_lt: prefix of their count),
  // the others are "heavy" (seg_tile: prefix of heavy m-tiles; a segment's
  // light tile comes after its heavy ones).  Without the split seg_tile is
  // the prefix of all m-tiles and the light list is empty.  WGRAD: every segment has the
  // same M tiles; the prefix is that of the padded row counts (the segment's
  // k range), kept in seg_kpos.
  __shared__ int seg_kpos[WG ? kMaxSegments + 1 : 1];
  __shared__ int seg_lt[WG ? 1 : kMaxSegments + 1];
  const int nsplit = KSPLIT ? a.ksplit : 1;
  const int nslots = gridDim.x >> 3;   // blocks per XCD
  if (wave == 0) {
    int c0 = 0, c1 = 0, l0 = 0, l1 = 0, r, st;
    const int s0 = 2 * lane, s1 = 2 * lane + 1;
    auto classify = [&](int rr, int& c, int& l) {
      if (WG) {
        c = wgrad_pad(rr);
      } else {
        const int rag = rr % BM;
        c = rr / BM + (rag > BM / 2 ? 1 : 0);
        l = (rag > 0 && rag <= BM / 2) ? 1 : 0;
      }
    };
    if (s0 < nseg) {
      segment_rows(a, s0, off_E, r, st);
      classify(r, c0, l0);
      seg_nrows[s0] = r;
      seg_row0[s0] = st;
    }
    if (s1 < nseg) {
      segment_rows(a, s1, off_E, r, st);
      classify(r, c1, l1);
      seg_nrows[s1] = r;
      seg_row0[s1] = st;
    }
    int v = c0 + c1, incl = v, lv = l0 + l1, lincl = lv;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o), lu = __shfl_up(lincl, o);
      if (lane >= o) incl += u, lincl += lu;
    }
    const int excl = incl - v, lexcl = lincl - lv;
    if (WG) {
      const int mtw = (a.M + BM - 1) / BM;
      if (s0 < nseg) seg_kpos[s0] = excl;
      if (s1 < nseg) seg_kpos[s1] = excl + c0;
      if (lane == 63) seg_kpos[nseg] = incl;
      if (s0 < nseg) seg_tile[s0] = s0 * mtw;
      if (s1 < nseg) seg_tile[s1] = s1 * mtw;
      if (lane == 63) seg_tile[nseg] = nseg * mtw;
    } else {
      // The two lists are kept apart only when that lowers the number of
      // rounds of heavy tiles per block; otherwise every tile is "heavy":
      // one list in segment order, a segment's last tile after its others.
      const int nh = __shfl(incl, 63), nl = __shfl(lincl, 63);
      const int h = nh * NT * nsplit, all = (nh + nl) * NT * nsplit;
      const bool two = ((h + 7) / 8 + nslots - 1) / nslots < ((all + 7) / 8 + nslots - 1) / nslots;
      const int pe = two ? excl : excl + lexcl, pi = two ? incl : incl + lincl;
      if (s0 < nseg) seg_tile[s0] = pe, seg_lt[s0] = lexcl;
      if (s1 < nseg) seg_tile[s1] = pe + c0 + (two ? 0 : l0), seg_lt[s1] = lexcl + l0;
      if (lane == 63) seg_tile[nseg] = pi, seg_lt[nseg] = two ? lincl : 0;
    }
  }
  __syncthreads();
  // Heavy and light tiles per K slice; with several slices the slice is the
  // slowest index of each list.  Tile ids: the heavy list, then the light.
  const int tiles = seg_tile[nseg] * NT;
  const int ltiles = WG ? 0 : seg_lt[nseg] * NT;
  const int nheavy = tiles * nsplit, nlight = ltiles * nsplit;
  // Persistent blocks, one per compute unit: the blocks of XCD xcd (block b
  // runs on XCD b % 8) walk that XCD's sequence of tiles in steps of their
  // count: its contiguous eighth of the heavy list (so the tiles of one
  // expert weight stay within one L2), then its eighth of the light list.
  // Every XCD thus gets the same number of heavy tiles and of light tiles,
  // and light tiles come last, where they fill the last round unevenly.
  // WGRAD tiles differ in length (a segment's k range is its padded row
  // count: a shared expert's is every token), so there the XCD ranges split
  // the cumulative k-tiles instead of the tile count: XCD x takes the tiles
  // whose midpoints fall in its eighth of the k-tiles.
  const int xcd = blockIdx.x & 7;
  int it = blockIdx.x >> 3;
  int wg_first = 0, wg_end = 0;
  if (WG) {
    if (wave == 0) {
      const long long Ts = tiles / nseg;                          // tiles per segment
      const long long W = (long long)(seg_kpos[nseg] / 32) * Ts;  // k-tiles of all tiles
      const long long G = 8;
      // tiles j of segment s with midpoint below x W / 8, for x = this XCD
      // and the next: 8 w (2j + 1) < 2 x W - 16 C, where w is the segment's
      // k-tiles per tile and C the k-tiles of all tiles before it
      for (int e = 0; e < 2; ++e) {
        const long long X0 = 2 * (long long)(xcd + e) * W;
        long long cnt = 0;
        for (int sg = lane; sg < nseg; sg += 64) {
          const long long w = (seg_kpos[sg + 1] - seg_kpos[sg]) / 32;
          const long long X = X0 - 2 * G * ((long long)(seg_kpos[sg] / 32) * Ts);
          const long long c = X >= 1 ? ((X - 1) / (G * w) + 1) / 2 : 0;
          cnt += c < Ts ? c : Ts;
        }
        int ci = (int)cnt;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) ci += __shfl_xor(ci, o);
        if (lane == 0) sh_range[e] = ci;
      }
    }
    __syncthreads();
    wg_first = sh_range[0];
    wg_end = sh_range[1];
  }
  const int per = (nheavy + 7) >> 3, lper = (nlight + 7) >> 3;
  const int hlen = min(max(nheavy - xcd * per, 0), per);
  const int llen = min(max(nlight - xcd * lper, 0), lper);
  auto tile_at = [&](int i) {
    if (WG) return wg_first + i < wg_end ? wg_first + i : -1;
    if (i < hlen) return xcd * per + i;
    i -= hlen;
    return i < llen ? nheavy + xcd * lper + i : -1;
  };
  const int step = nslots;
  // The thread of the segment that holds tile LL records it in sh_seg[b].
  // A tile id decodes the same way in either list: the list's prefix of
  // m-tiles per segment (heavy: seg_tile; light: seg_lt, 0 or 1 per
  // segment), its tiles per K slice and its first id; a light tile's m-tile
  // index follows its segment's heavy ones.  The thread of the segment that
  // holds tile LL records the segment and the tile's K slice, n-tile and
  // m-tile in slot b.
  __shared__ int sh_coord[2][3];
  // Within a segment the m-tiles run fastest: the blocks working at once
  // share one n-tile of W, and X is read again for every n-tile, from the
  // L2 and the MALL while it fits there.  A weight gradient whose X (the
  // transposed gradient of the up projection's pre-activations, 2 d_ff or
  // d_ff rows per segment) is both the larger operand and larger than half
  // the 256 MB MALL runs the n-tiles fastest instead, so that X is read
  // once and the smaller W again (large_prefill dW1: 4.65 -> 3.85 ms).
  const bool nfast = WG && a.M > a.Nout && a.xbytes > (128LL << 20);
  auto locate = [&](int LL, int b) {
    const bool lt = !WG && LL >= nheavy;
    const int* P = lt ? seg_lt : seg_tile;
    const int i = LL - (lt ? nheavy : 0), tl = lt ? ltiles : tiles;
    const int ks = KSPLIT ? i / tl : 0;   // one K slice: i < tl
    const int L = i - ks * tl;
    if (tid < nseg && P[tid] * NT <= L && L < P[tid + 1] * NT) {
      const int hm = seg_tile[tid + 1] - seg_tile[tid];   // heavy m-tiles
      const int m = lt ? 1 : hm;                          // m-tiles in this list
      const int local = L - P[tid] * NT;
      sh_seg[b] = tid;
      sh_coord[b][0] = ks;
      sh_coord[b][1] = nfast ? local % NT : local / m;
      sh_coord[b][2] = nfast ? local / NT : local % m + (lt ? hm : 0);
    }
  };
  auto coords = [&](int b) {   // the tile located in slot b
    TileCoord c;
    c.seg = __builtin_amdgcn_readfirstlane(sh_seg[b]);
    c.ks = __builtin_amdgcn_readfirstlane(sh_coord[b][0]);
    c.nt = __builtin_amdgcn_readfirstlane(sh_coord[b][1]);
    c.mt = __builtin_amdgcn_readfirstlane(sh_coord[b][2]);
    if (WG) {   // output rows of this segment's gradient; no gather, no row offset
      c.rows = a.M;
      c.start = c.seg * a.M;
    } else {
      c.rows = seg_nrows[c.seg];
      c.start = seg_row0[c.seg];
    }
    return c;
  };

  // ---- LDS layout.  Row r of a tile (W rows first, then token rows) holds
  // its ROWCH chunks of 16 bytes at chunk positions kc ^ ((r / RPB) % ROWCH).
  // The LDS has 64 banks of 4 bytes (256 bytes, RPB rows) and serves 16 lanes
  // of a ds_read_b128 per cycle; the fragment reads of 16 consecutive rows
  // then use each (bank group, row % RPB) pair once: no bank conflicts.
  //
  // Tiles move from global memory straight into LDS (global_load_lds_dwordx4:
  // lane l of a wave instruction writes 16 bytes at the instruction's LDS
  // base + 16 l).  Instruction q of a k-tile fills rows RI*q .. RI*q+RI-1, so
  // lane l fetches row RI*q + l/ROWCH, logical chunk
  // (l % ROWCH) ^ ((4q + l/16) % ROWCH) (as RI = 4 RPB).
  // Wave w issues the W instructions q = w*QWW + j and the token-row
  // instructions q = BN/RI + w*QWX + j.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto kc_dma = [&](int q) { return (lane % ROWCH) ^ ((4 * q + lane / 16) % ROWCH); };
  // Source rows of this lane's token-row chunks: gathered tiles load their
  // sorted_assign entries (the token's assignment) ahead of the tile.
  int srow[QWX];
  // Rows past the tile's valid rows: -1 (no row), or with a 2 GiB+ X the
  // last valid row.
  const bool x_oob = a.xbytes < (1LL << 31);
  auto row_loads = [&](const TileCoord& c) {
#pragma unroll
    for (int j = 0; j < QWX; ++j) {
      const int q = BN / RI + wave * QWX + j;
      const int m = c.mt * BM + RI * q + lane / ROWCH - BN;
      if (m >= c.rows && x_oob) {
        srow[j] = -1;
      } else {
        const int mm = m < c.rows ? m : c.rows - 1;
        if (GATHER && c.seg < a.E) srow[j] = a.sorted_assign[c.start + mm];
        else srow[j] = mm;
      }
    }
  };
  // K elements of the tile's slice (WGRAD: the segment's padded row range),
  // source bases and this lane's byte offsets of its source chunks.
  int kslice;
  const char* xbase;
  const char* wbase;
  long long xext;   // bytes of X from xbase
  uint32_t woff[QWW], xoff[QWX];
  auto setup = [&](const TileCoord& c) {
    kslice = WG ? seg_kpos[c.seg + 1] - seg_kpos[c.seg] : a.K / nsplit;
    if (WG) {
      xbase = (const char*)(a.X + seg_kpos[c.seg]);
      wbase = (const char*)(a.W + seg_kpos[c.seg]);
    } else {
      if (GATHER) xbase = (const char*)a.X;
      else xbase = (const char*)(a.X + (long long)c.start * a.K + (long long)c.ks * kslice);
      wbase = (const char*)(a.W + (long long)c.seg * a.Wrows * a.K + (long long)c.ks * kslice);
    }
    xext = a.xbytes - (long long)(xbase - (const char*)a.X);
#pragma unroll
    for (int j = 0; j < QWW; ++j) {
      const int q = wave * QWW + j;
      const int rho = RI * q + lane / ROWCH;
      int wr;
      if (SWIGLU) {
        const int half = BN / 2;
        const int nn = c.nt * half + (rho < half ? rho : rho - half);
        const int nc = nn < a.f ? nn : a.f - 1;
        wr = rho < half ? nc : a.f + nc;
      } else {
        const int nn = c.nt * BN + rho;
        wr = nn < a.Wrows ? nn : a.Wrows - 1;
      }
      woff[j] = ((uint32_t)wr * (uint32_t)a.K + (uint32_t)kc_dma(q) * 8u) * 2u;
    }
#pragma unroll
    for (int j = 0; j < QWX; ++j) {
      const int q = BN / RI + wave * QWX + j;
      const int sr = srow[j];
      const uint32_t row = (GATHER && c.seg < a.E) ? (uint32_t)(sr / a.k) : (uint32_t)sr;
      xoff[j] = sr < 0 ? kNoRow : (row * (uint32_t)a.K + (uint32_t)kc_dma(q) * 8u) * 2u;
    }
  };
  // The bias columns of a tile (K slice 0 only), two per thread of the first
  // BN / 2, loaded a tile ahead and moved into sh_bias before the epilogue.
  uint32_t bias_reg = 0;
  auto bias_load = [&](const TileCoord& c) {
    if (BIAS && a.bias && c.ks == 0 && tid < BN / 2) {
      const int col = c.nt * BN + 2 * tid;
      bias_reg = col < a.Nout ? *(const uint32_t*)(a.bias + (long long)c.seg * a.Wrows + col) : 0u;
    }
  };
  // Fragment rows are MF-aligned bases plus lane % MF, so the swizzle term
  // depends on the lane only: one per-lane offset per k-substep.  32x32x16:
  // lane l reads row l & 31, chunk 2 s + (l >> 5) of k-substep s; 16x16x32:
  // row l & 15, chunk 4 s + (l >> 4) of 32-deep k-step s.
  int fro[NSUB];
#pragma unroll
  for (int s4 = 0; s4 < NSUB; ++s4) {
    if (MF == 32)
      fro[s4] = (lane & 31) * ROWCH + ((2 * s4 + (lane >> 5)) ^ (((lane & 31) / RPB) % ROWCH));
    else
      fro[s4] = (lane & 15) * ROWCH + ((4 * s4 + (lane >> 4)) ^ (((lane & 15) / RPB) % ROWCH));
  }
  int wrb[NI], xrb[MI];  // MF-row base of each fragment, in chunks
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    if (SWIGLU) {
      const int jj = j < NI / 2 ? j : j - NI / 2;
      wrb[j] = ((j < NI / 2 ? 0 : BN / 2) + wn * (BN / 2 / WGN) + jj * MF) * ROWCH;
    } else {
      wrb[j] = (wn * WN + j * MF) * ROWCH;
    }
  }
#pragma unroll
  for (int i = 0; i < MI; ++i) xrb[i] = (BN + wm * WM + i * MF) * ROWCH;

  typedef __attribute__((address_space(3))) void lds_void_t;
  // Token rows move through a buffer resource over X from the k-tile's
  // column on (with x_oob its extent bounds every valid offset and the
  // kNoRow offset of a missing row lies past it; otherwise it spans 4 GiB).
  auto dma = [&](u32x4* buf, int kt) {
    const char* wb = wbase + kt * (BK * 2);
    u32x4* wdst = buf + wv * QWW * 64;
    u32x4* xdst = buf + BN * ROWCH + wv * QWX * 64;
#pragma unroll
    for (int j = 0; j < QWW; ++j)
      __builtin_amdgcn_global_load_lds((const void*)(wb + woff[j]), (lds_void_t*)(wdst + j * 64),
                                       16, 0, 0);
#if __HIP_DEVICE_COMPILE__   // (with template-dependent operands the host pass drops the kernel)
    const long long xo = (long long)kt * (BK * 2);
    const int nrec = x_oob ? (int)(xext - xo) : -1;
    const __amdgpu_buffer_rsrc_t xres =
        __builtin_amdgcn_make_buffer_rsrc((void*)(xbase + xo), (short)0, nrec, 0x00020000);
#pragma unroll
    for (int j = 0; j < QWX; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (lds_void_t*)(xdst + j * 64), 16, xoff[j], 0,
                                               0, 0);
#endif
  };
  auto frag_load = [&](const u32x4* buf, u32x4(&wf)[NI], u32x4(&xf)[MI], int s4) {
#pragma unroll
    for (int j = 0; j < NI; ++j) wf[j] = buf[wrb[j] + fro[s4]];
#pragma unroll
    for (int i = 0; i < MI; ++i) xf[i] = buf[xrb[i] + fro[s4]];
  };

  constexpr int NDMA = QWW + QWX;
  constexpr int INFLIGHT = (NSTAGE - 2) * NDMA;   // DMAs that may stay in flight
  static_assert((NSTAGE - 1) * NDMA <= 63, "vmcnt range");
  // s_waitcnt immediate: vmcnt = INFLIGHT, expcnt and lgkmcnt = 0 (every
  // fragment read of this tile has completed before the barrier).
  constexpr int WAIT_IMM = (INFLIGHT & 15) | ((INFLIGHT >> 4) << 14);
  // the same with NSTAGE - 1 k-tiles' DMAs in flight (2-stage ring, tile start)
  constexpr int INFLIGHT3 = (NSTAGE - 1) * NDMA;
  constexpr int WAIT_IMM3 = (INFLIGHT3 & 15) | ((INFLIGHT3 >> 4) << 14);
  // A barrier after this wave's LDS operations have completed, with no wait
  // for its global loads and stores in flight (s_waitcnt lgkmcnt(0) only:
  // vmcnt 63, expcnt 7).
  auto lds_barrier = [&]() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
  };

  // ---- tile pipeline.  During a tile's epilogue (which stages its output in
  // the ring stages after the first), once its first 32-row slab is out, the block's next
  // tile issues the DMA of its first k-tile into stage 0 and loads its bias
  // columns, and the gathered source rows of the tile after that are
  // fetched.  Tile segments are located two tiles ahead (after a tile's main
  // loop, when no load is in flight), in sh_seg slots that alternate.  Loads
  // complete in order, so the wait for stage 0 at the top of a tile covers
  // the bias and row loads too.
  int LL = tile_at(it);
  if (LL < 0) return;   // uniform over the block
  int LL1 = tile_at(it + step);
  locate(LL, 0);
  if (LL1 >= 0) locate(LL1, 1);
  __syncthreads();
  TileCoord cur = coords(0);
  row_loads(cur);
  setup(cur);
  dma(lds0, 0);
  if (LL1 >= 0) row_loads(coords(1));
  bias_load(cur);
  lds_barrier();     // sh_seg has been read everywhere before it is rewritten
  int b = 0;         // sh_seg slot of this tile and of the tile two ahead
  for (;;) {
    const bool more = LL1 >= 0;   // uniform over the block
    const int LL2 = more ? tile_at(it + 2 * step) : -1;
    const int nk = kslice / BK;
    auto clampk = [&](int t) { return t < nk ? t : nk - 1; };
    // stage 0 has landed; the DMAs of the later stages may stay in flight
    if constexpr (BK == 64) {
      dma(lds1, clampk(1));
      __builtin_amdgcn_s_waitcnt(WAIT_IMM3);
    } else {
      dma(lds1, clampk(1));
      dma(lds2, clampk(2));
      __builtin_amdgcn_s_waitcnt(WAIT_IMM);
    }
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");

    u32x4 wf[2][NI], xf[2][MI];
    // this wave's token rows hold valid rows of the tile (uniform per wave)
    const bool wact = cur.mt * BM + wm * WM < cur.rows;
    accv acc[NI][MI];
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int i = 0; i < MI; ++i) acc[j][i] = accv{};
    auto mfmas = [&](const u32x4(&wf)[NI], const u32x4(&xf)[MI]) {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        // the down projection's W2 tile is bf16 in LDS: fp16 for the fp16 MFMA
        const u32x4 w = CVT16 ? bf16x8_to_f16x8(wf[j]) : wf[j];
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          if constexpr (MF == 32) {
            if (CVT16)
              acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                  __builtin_bit_cast(f16x8, w), __builtin_bit_cast(f16x8, xf[i]), acc[j][i], 0, 0,
                  0);
            else
              acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, w), __builtin_bit_cast(bf16x8, xf[i]), acc[j][i], 0,
                  0, 0);
          } else {
            if (CVT16)
              acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  __builtin_bit_cast(f16x8, w), __builtin_bit_cast(f16x8, xf[i]), acc[j][i], 0, 0,
                  0);
            else
              acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8, w), __builtin_bit_cast(bf16x8, xf[i]), acc[j][i], 0,
                  0, 0);
          }
        }
      }
    };

    // ---- main loop over k-tiles with an NSTAGE ring in LDS.  Iteration kt
    // issues the DMA of tile kt+3 into the stage of tile kt-1 (all its reads
    // finished before the previous barrier), computes tile kt, then waits
    // until tile kt+1 has landed (the DMAs of tiles kt+2 and kt+3 may stay in
    // flight: vmcnt(2 * DMAs per tile)) and crosses the barrier.  The last
    // k-substep's MFMAs run after the barrier, under the fragment reads of the
    // next tile, so the matrix pipe does not drain at tile boundaries.  The
    // loop body is straight-line: DMAs past the last tile are clamped to it
    // (into stages nobody reads again) and the tail iterations are peeled.
    auto iteration = [&](const u32x4* cur_st, const u32x4* next_st, u32x4* far, int kt) {
      dma(far, clampk(kt + NSTAGE - 1));
#pragma unroll
      for (int s4 = 0; s4 + 1 < NSUB; ++s4) {
        frag_load(cur_st, wf[(s4 + 1) & 1], xf[(s4 + 1) & 1], s4 + 1);
        mfmas(wf[s4 & 1], xf[s4 & 1]);
      }
      // substep 0: the DMA interleaved with its MFMAs and the next fragments
#if MOE_SCHED_FRONT
      sched_front<NM, SG_DS_READ, NFR, MOE_SCHED_PER, SG_VMEM_READ, NDMA>();
#else
      sched_interleave<NM, SG_VMEM_READ, NDMA, SG_DS_READ, NFR>();
#endif
#pragma unroll
      for (int s4 = 1; s4 + 1 < NSUB; ++s4)
        sched_interleave<NM, SG_DS_READ, NFR, SG_VMEM_READ, 0>();
      __builtin_amdgcn_s_waitcnt(WAIT_IMM);
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");   // no LDS read moves above the barrier
      frag_load(next_st, wf[0], xf[0], 0);
      mfmas(wf[(NSUB - 1) & 1], xf[(NSUB - 1) & 1]);
#if MOE_SCHED_FRONT
      sched_front<NM, SG_DS_READ, NFR, MOE_SCHED_PER, SG_VMEM_READ, 0>();
#else
      sched_interleave<NM, SG_DS_READ, NFR, SG_VMEM_READ, 0>();
#endif
    };
    // A wave without valid rows only issues its DMA share and keeps the
    // block's barriers.
    auto idle = [&](u32x4* far, int kt) {
      dma(far, clampk(kt + NSTAGE - 1));
      __builtin_amdgcn_s_waitcnt(WAIT_IMM);
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
    };
    // ---- 16x16x32 with 64-deep k-tiles in a 2-stage ring: two 32-deep MFMA
    // k-steps per k-tile, each in two phases.  The operand with more
    // fragments per wave (W for the up projection's 64 x 128 wave tiles, the
    // token rows for the down projection's 128 x 64) is read in two halves,
    // one per phase; the other operand is double-buffered across k-steps
    // (k-step s uses buffer s), so a wave holds 16 fragments instead of two
    // full sets of 12.  Each phase's MFMAs run under the fragment reads of
    // the next phase.  There is one barrier per k-tile, before its last
    // phase: it waits until tile kt+1 has landed, after which every wave's
    // reads of tile kt's stage are done, so the last phase also issues the
    // DMA of tile kt+2 into that stage, and the reads of tile kt+1's first
    // k-step.  The DMA thus runs one k-tile ahead.
    constexpr bool SPW = NI >= MI;   // W fragments split in halves (else token rows)
    u32x4 w16[SPW ? 1 : 2][NI], x16[SPW ? 2 : 1][MI];
    auto lw = [&](const u32x4* buf, u32x4(&d)[NI], int j0, int j1, int ks = 0) {
#pragma unroll
      for (int j = j0; j < j1; ++j) d[j] = buf[wrb[j] + fro[ks]];
    };
    auto lx = [&](const u32x4* buf, u32x4(&d)[MI], int i0, int i1, int ks = 0) {
#pragma unroll
      for (int i = i0; i < i1; ++i) d[i] = buf[xrb[i] + fro[ks]];
    };
    auto mm = [&](const u32x4(&wv)[NI], const u32x4(&xv)[MI], int j0, int j1, int i0, int i1) {
#pragma unroll
      for (int j = j0; j < j1; ++j) {
        const u32x4 w = CVT16 ? bf16x8_to_f16x8(wv[j]) : wv[j];
#pragma unroll
        for (int i = i0; i < i1; ++i) {
          if constexpr (MF == 16) {
            if (CVT16)
              acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  __builtin_bit_cast(f16x8, w), __builtin_bit_cast(f16x8, xv[i]), acc[j][i], 0, 0,
                  0);
            else
              acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8, w), __builtin_bit_cast(bf16x8, xv[i]), acc[j][i], 0,
                  0, 0);
          }
        }
      }
    };
    constexpr int NRA = SPW ? NI / 2 : MI / 2;        // phase A reads (second half, tile kt)
    constexpr int NRB = SPW ? MI + NI / 2 : NI + MI / 2;   // phase B reads (tile kt+1)
    auto iteration64 = [&](const u32x4* cur_st, const u32x4* next_st, u32x4* free_st, int kt) {
      if constexpr (SPW) {
        lw(cur_st, w16[0], NI / 2, NI, 0);
        mm(w16[0], x16[0], 0, NI / 2, 0, MI);
        sched_front<NM / 2, SG_DS_READ, NRA, MOE_SCHED_PER, SG_VMEM_READ, 0>();
        lx(cur_st, x16[1], 0, MI, 1);
        lw(cur_st, w16[0], 0, NI / 2, 1);
        mm(w16[0], x16[0], NI / 2, NI, 0, MI);
        sched_front<NM / 2, SG_DS_READ, NRB, MOE_SCHED_PER, SG_VMEM_READ, 0>();
        lw(cur_st, w16[0], NI / 2, NI, 1);
        mm(w16[0], x16[1], 0, NI / 2, 0, MI);
      } else {
        lx(cur_st, x16[0], MI / 2, MI, 0);
        mm(w16[0], x16[0], 0, NI, 0, MI / 2);
        sched_front<NM / 2, SG_DS_READ, NRA, MOE_SCHED_PER, SG_VMEM_READ, 0>();
        lw(cur_st, w16[1], 0, NI, 1);
        lx(cur_st, x16[0], 0, MI / 2, 1);
        mm(w16[0], x16[0], 0, NI, MI / 2, MI);
        sched_front<NM / 2, SG_DS_READ, NRB, MOE_SCHED_PER, SG_VMEM_READ, 0>();
        lx(cur_st, x16[0], MI / 2, MI, 1);
        mm(w16[1], x16[0], 0, NI, 0, MI / 2);
      }
      sched_front<NM / 2, SG_DS_READ, NRA, MOE_SCHED_PER, SG_VMEM_READ, 0>();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(WAIT_IMM);   // tile kt+1 has landed
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (SPW) {
        lx(next_st, x16[0], 0, MI, 0);
        lw(next_st, w16[0], 0, NI / 2, 0);
      } else {
        lw(next_st, w16[0], 0, NI, 0);
        lx(next_st, x16[0], 0, MI / 2, 0);
      }
      dma(free_st, clampk(kt + 2));
      if constexpr (SPW) mm(w16[0], x16[1], NI / 2, NI, 0, MI);
      else mm(w16[1], x16[0], 0, NI, MI / 2, MI);
      sched_front<NM / 2, SG_DS_READ, NRB, MOE_SCHED_PER, SG_VMEM_READ, NDMA>();
    };
    auto idle64 = [&](u32x4* free_st, int kt) {
      __builtin_amdgcn_s_waitcnt(WAIT_IMM);
      __builtin_amdgcn_s_barrier();
      __asm__ volatile("" ::: "memory");
      dma(free_st, clampk(kt + 2));
    };
    if constexpr (MF == 16) {
      if (wact) {
        if constexpr (SPW) {
          lx(lds0, x16[0], 0, MI, 0);
          lw(lds0, w16[0], 0, NI / 2, 0);
        } else {
          lw(lds0, w16[0], 0, NI, 0);
          lx(lds0, x16[0], 0, MI / 2, 0);
        }
        int kt = 0;
        for (; kt + 1 < nk; kt += 2) {
          iteration64(lds0, lds1, lds0, kt);
          iteration64(lds1, lds0, lds1, kt + 1);
        }
        if (kt < nk) iteration64(lds0, lds1, lds0, kt);
      } else {
        int kt = 0;
        for (; kt + 1 < nk; kt += 2) {
          idle64(lds0, kt);
          idle64(lds1, kt + 1);
        }
        if (kt < nk) idle64(lds0, kt);
      }
    } else if (wact) {
      frag_load(lds0, wf[0], xf[0], 0);
      int kt = 0;
      for (; kt + 3 < nk; kt += 4) {
        iteration(lds0, lds1, lds3, kt);
        iteration(lds1, lds2, lds0, kt + 1);
        iteration(lds2, lds3, lds1, kt + 2);
        iteration(lds3, lds0, lds2, kt + 3);
      }
      if (kt < nk) iteration(lds0, lds1, lds3, kt);
      if (kt + 1 < nk) iteration(lds1, lds2, lds0, kt + 1);
      if (kt + 2 < nk) iteration(lds2, lds3, lds1, kt + 2);
    } else {
      int kt = 0;
      for (; kt + 3 < nk; kt += 4) {
        idle(lds3, kt);
        idle(lds0, kt + 1);
        idle(lds1, kt + 2);
        idle(lds2, kt + 3);
      }
      if (kt < nk) idle(lds3, kt);
      if (kt + 1 < nk) idle(lds0, kt + 1);
      if (kt + 2 < nk) idle(lds1, kt + 2);
    }

    // Every DMA (including the clamped ones past the last tile) has landed and
    // every wave's last fragment reads are done before the ring is reused;
    // the tile's bias columns are in sh_bias, the segment of the tile two
    // ahead in sh_seg.
    if (BIAS && a.bias && cur.ks == 0 && tid < BN / 2) sh_bias[tid] = bias_reg;
    if (LL2 >= 0) locate(LL2, b);
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    // ---- epilogue.  32x32x16: lane holds token row (lane & 31) of each 32x32
    // tile and, in register group g, the four consecutive weight rows 8g +
    // 4*(lane>>5) + 0..3; 16x16x32: token row (lane & 15) of each 16x16 tile
    // and the weight rows 4*(lane>>4) + 0..3.  Stored directly, one
    // instruction would touch 16-32 rows with 16-32 bytes each; instead each
    // wave stages one 32-row slab of its output (one 32-row fragment, or two
    // 16-row ones; after bias and activation, in the output type) in a padded
    // LDS region of the ring stages after the first (with a 2-stage ring,
    // stage 1 and a small extra region) and writes it back as whole 16-byte
    // chunks of rows, CPR lanes per row, so a store instruction covers RPI
    // rows of contiguous bytes.  The padding keeps the staging writes and
    // reads free of bank conflicts.
    constexpr int CPR = WNOUT * ES / 16;                  // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;                         // rows per store instruction
    constexpr int SLAB = 32;                              // slab rows
    constexpr int FPS = SLAB / MF;                        // token fragments per slab
    static_assert(FPS >= 1 && MI % FPS == 0, "whole slabs");
    static_assert(CPR >= 1 && CPR <= 64 && 64 % CPR == 0 && SLAB % RPI == 0, "staging shape");
    // the next tile's first k-tile and bias, the row loads of the one after
    auto prefetch_next = [&]() {
      const TileCoord nx = coords(b ^ 1);
      setup(nx);
      dma(lds0, 0);
      bias_load(nx);
      if (LL2 >= 0) row_loads(coords(b));
    };
    // (a wave without valid rows stages zeros and stores nothing)
    char* stg;
    if constexpr (NSTAGE == 2) {
      stg = wv < WPA ? (char*)lds1 + wv * STG : (char*)lds2 + (wv - WPA) * STG;
    } else {
      const int wa = wv / WPA;
      stg = (char*)(wa == 0 ? lds1 : wa == 1 ? lds2 : lds3) + (wv % WPA) * STG;
    }
    const int colw = SWIGLU ? cur.nt * (BN / 2) + wn * (BN / 2 / WGN) : cur.nt * BN + wn * WN;
    char* obase =
        cur.ks == 0 ? (char*)a.out : (char*)(a.out2 + (long long)(cur.ks - 1) * a.part_elems);
#pragma unroll
    for (int sl = 0; sl < MI / FPS; ++sl) {
#pragma unroll
      for (int i2 = 0; i2 < FPS; ++i2) {
        const int i = sl * FPS + i2;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
#pragma unroll
          for (int g = 0; g < MF * MF / 256; ++g) {   // groups of 4 accumulators
            // four consecutive output columns nloc.. of slab row srow
            const int nloc = MF == 32 ? j * 32 + 8 * g + 4 * (lane >> 5) : j * 16 + 4 * (lane >> 4);
            const int srow = MF == 32 ? (lane & 31) : 16 * i2 + (lane & 15);
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = acc[j][i][4 * g + r];
            if (CVT16) {   // h was stored scaled by 2^-8
#pragma unroll
              for (int r = 0; r < 4; ++r) v[r] *= kHLoadScale;
            }
            if (SWIGLU) {
#pragma unroll
              for (int r = 0; r < 4; ++r) v[r] = silu_f(v[r]) * acc[j + NI / 2][i][4 * g + r];
            } else if (BIAS && a.bias && cur.ks == 0) {
              const u32x2 bb = *(const u32x2*)(sh_bias + (wn * WN + nloc) / 2);
              v[0] += __uint_as_float(bb[0] << 16);
              v[1] += __uint_as_float(bb[0] & 0xffff0000u);
              v[2] += __uint_as_float(bb[1] << 16);
              v[3] += __uint_as_float(bb[1] & 0xffff0000u);
            }
            char* dst = stg + srow * PITCH + nloc * ES;
            if (OUT32) {
              *(f32x4*)dst = f32x4{v[0], v[1], v[2], v[3]};
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                if (MODE == MODE_RELU) v[r] = fmaxf(v[r], 0.0f);
                if (MODE == MODE_GELU) v[r] = gelu_f(v[r]);
              }
              *(f16x4*)dst = f16x4{h_to_f16(v[0]), h_to_f16(v[1]), h_to_f16(v[2]), h_to_f16(v[3])};
            }
          }
        }
      }
      // LDS operations of one wave complete in order: the reads below see the
      // writes above, and the next slab's writes follow these reads.
#pragma unroll
      for (int q = 0; q < SLAB / RPI; ++q) {
        const int r = q * RPI + lane / CPR, c = lane % CPR;
        const u32x4 val = *(const u32x4*)(stg + r * PITCH + c * 16);
        const int m = cur.mt * BM + wm * WM + sl * SLAB + r;
        const int col = colw + c * (16 / ES);
        if (m < cur.rows && col < a.Nout)
          *(u32x4*)(obase + ((long long)(cur.start + m) * a.Nout + col) * ES) = val;
      }
      if (sl == 0 && more) prefetch_next();
    }
    if (!more) break;
    cur = coords(b ^ 1);
    it += step;
    LL1 = LL2;
    b ^= 1;
    lds_barrier();   // every wave's staging reads are done before stages 1 and 2 refill
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

// Block tiles per projection (token rows x weight rows).
#ifndef MOE_UP_BM
#define MOE_UP_BM 256
#endif
#ifndef MOE_UP_BN
#define MOE_UP_BN 256
#endif
#ifndef MOE_DN_BM
#define MOE_DN_BM 256
#endif
#ifndef MOE_DN_BN
#define MOE_DN_BN 256
#endif
#ifndef MOE_UP_WGM
#define MOE_UP_WGM 4
#endif
#ifndef MOE_UP_WGN
#define MOE_UP_WGN 2
#endif
#ifndef MOE_DN_WGM
#define MOE_DN_WGM 2
#endif
#ifndef MOE_DN_WGN
#define MOE_DN_WGN 4
#endif
#ifndef MOE_UP_OCC
#define MOE_UP_OCC 1
#endif
#ifndef MOE_DN_OCC
#define MOE_DN_OCC 1
#endif
constexpr int UP_BM = MOE_UP_BM, UP_BN = MOE_UP_BN, UP_WGM = MOE_UP_WGM, UP_WGN = MOE_UP_WGN;
constexpr int DN_BM = MOE_DN_BM, DN_BN = MOE_DN_BN, DN_WGM = MOE_DN_WGM, DN_WGN = MOE_DN_WGN;
constexpr int UP_OCC = MOE_UP_OCC, DN_OCC = MOE_DN_OCC;

int grid_blocks(const Shape& s, int BM, int NT, int ksplit = 1, int occ = 1) {
  const long long mt = (s.routed_rows() + BM - 1) / BM + s.E +
                       (long long)s.S * ((s.T + BM - 1) / BM);
  long long g = NT * mt * ksplit;
  // persistent: `occ` resident blocks per CU, each looping over tiles
  if (g > (long long)kNumCUs * occ) g = (long long)kNumCUs * occ;
  return (int)((g + 7) / 8 * 8);
}

// y_exp[r] += the K-slice partials of row r, in slice order.
__global__ __launch_bounds__(256) void part_fold_kernel(float* __restrict__ y_exp,
                                                        const float* __restrict__ y_part,
                                                        const int32_t* offsets, int T, int E,
                                                        int S, int d, int nparts,
                                                        long long part_elems) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int d4 = d / 4;
  const long long r = gid / d4;
  const int c = (int)(gid % d4) * 4;
  if (r >= (long long)offsets[E] + (long long)S * T) return;
  f32x4 v = *(const f32x4*)(y_exp + r * d + c);
  for (int p = 0; p < nparts; ++p) v += *(const f32x4*)(y_part + p * part_elems + r * d + c);
  *(f32x4*)(y_exp + r * d + c) = v;
}

}  // namespace

// K slices of a down-style grouped GEMM (K = reduction length, N = output
// columns) over the routed and shared row segments.
static int gemm_ksplit(const Shape& s, int K, int N) {
  // expected tiles with evenly routed experts (capacity-limited)
  long long per = (s.routed_rows() + s.E - 1) / s.E;
  if (s.cap > 0 && per > s.cap) per = s.cap;
  const long long mt = (long long)s.E * ((per + DN_BM - 1) / DN_BM) +
                       (long long)s.S * ((s.T + DN_BM - 1) / DN_BM);
  const long long tiles = mt * ((N + DN_BN - 1) / DN_BN);
  const int nkt = K / 32;     // k-tiles of the whole reduction
  int ks = 1;
  // split while the slices still fit in three quarters of the CUs and each
  // slice keeps at least 8 k-tiles
  while (ks < 4 && tiles * ks * 2 * 4 <= 3LL * kNumCUs && nkt % (ks * 2) == 0 &&
         nkt / (ks * 2) >= 8)
    ks *= 2;
  return ks;
}

int down_ksplit(const Shape& s) {
  if (s.dtype != MOE_BF16 || s.decode() || s.generic()) return 1;
  return gemm_ksplit(s, s.f, s.d);
}

int bwd_dx_ksplit(const Shape& s) { return gemm_ksplit(s, s.up_rows(), s.d); }

int down_parts(const Shape& s) { return s.decode() ? decode_nsplit(s) - 1 : down_ksplit(s) - 1; }

hipError_t launch_decode_up(const Shape& s, const void* x, const void* w_up, const void* b_up,
                            const float* s_up, const int32_t* offsets,
                            const int32_t* sorted_assign, void* h, hipStream_t st);
hipError_t launch_decode_down(const Shape& s, const void* h, const void* w_down,
                              const void* b_down, const float* s_down, const int32_t* offsets,
                              float* y_exp, float* y_part, bool complete, hipStream_t st);

// MFMA shape: the up projection always runs 16x16x32 with 64-deep k-tiles
// (faster at every measured size: at the same matrix-pipe occupancy it holds
// a higher clock); the down-style projections do so when long, at least 256
// GFLOP (about 0.2 ms; 2 x rows x depth x width at the upper bound of the
// rows), and otherwise keep 32x32x16 with 32-deep k-tiles, which is 2-6%
// faster on short launches (a few hundred tiles, K often split), where tile
// start-up dominates.
static std::atomic<int> g_gemm_policy{MOE_GEMM_AUTO};

void set_gemm_policy(int policy) { g_gemm_policy.store(policy, std::memory_order_relaxed); }

static bool long_flops(double flops) {
  const int policy = g_gemm_policy.load(std::memory_order_relaxed);
  if (policy == MOE_GEMM_MF32) return false;
  if (policy == MOE_GEMM_MF16) return true;
  return flops >= 256e9;
}

static bool long_launch(const Shape& s, long long depth, long long width) {
  return long_flops(2.0 * (double)s.max_rows() * (double)depth * (double)width);
}

// The up projection reduces over d_model, a multiple of 64 on the tiled path:
// the 16x16x32 loop always takes 64-deep k-tiles.
template <int MODE, int MF>
static void up_gemm(const Shape& s, const GemmArgs& a, int NT, hipStream_t st) {
  grouped_gemm_kernel<UP_BM, UP_BN, UP_WGM, UP_WGN, MODE, UP_OCC, MF, MF == 16 ? 64 : 32>
      <<<grid_blocks(s, UP_BM, NT, 1, UP_OCC), 64 * UP_WGM * UP_WGN, 0, st>>>(a);
}

// A down-style launch (MODE_DOWN, _LIN, _DXB) over the grid: 16x16x32 with
// 64-deep k-tiles for long launches whose K slices are whole 64-deep tiles,
// otherwise 32x32x16 with 32-deep k-tiles.
template <int MODE>
static void dn_gemm(bool long_run, int kslice, const GemmArgs& a, dim3 grid, hipStream_t st) {
  const dim3 block(64 * DN_WGM * DN_WGN);
  if (long_run && kslice % 64 == 0)
    grouped_gemm_kernel<DN_BM, DN_BN, DN_WGM, DN_WGN, MODE, DN_OCC, 16, 64><<<grid, block, 0, st>>>(a);
  else
    grouped_gemm_kernel<DN_BM, DN_BN, DN_WGM, DN_WGN, MODE, DN_OCC, 32, 32><<<grid, block, 0, st>>>(a);
}

hipError_t launch_up(const Shape& s, const void* x, const void* w_up, const void* b_up,
                     const float* s_up, const int32_t* offsets, const int32_t* sorted_assign,
                     void* h, hipStream_t st) {
  if (s.w_fp8() && !s.decode()) return hipErrorNotSupported;   // rejected by validation
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
                                                        s.tok_div(), s.E, s.S, s.d, s.f, s.up_rows(), s.f);
    else if (s.act == MOE_GELU)
      gemm_f32_kernel<MODE_GELU><<<blocks, 256, 0, st>>>(X, W, B, O, offsets, sorted_assign, s.T,
                                                        s.tok_div(), s.E, s.S, s.d, s.f, s.up_rows(), s.f);
    else
      gemm_f32_kernel<MODE_SWIGLU><<<blocks, 256, 0, st>>>(X, W, B, O, offsets, sorted_assign,
                                                          s.T, s.tok_div(), s.E, s.S, s.d, s.f,
                                                          s.up_rows(), s.f);
    return hipGetLastError();
  }
  if (s.generic()) return launch_up_generic(s, x, w_up, b_up, offsets, sorted_assign, h, st);
  if (s.decode()) return launch_decode_up(s, x, w_up, b_up, s_up, offsets, sorted_assign, h, st);
  GemmArgs a{(const uint16_t*)x, (const uint16_t*)w_up, (const uint16_t*)bias, h, offsets,
             sorted_assign, s.T, s.tok_div(), s.E, s.S, s.d, s.f, s.up_rows(), s.f, 1, nullptr, 0, 0,
             (long long)s.T * s.d * 2};
  const bool mf16 = g_gemm_policy.load(std::memory_order_relaxed) != MOE_GEMM_MF32;
  if (s.act == MOE_SWIGLU) {
    const int NT = (s.f + UP_BN / 2 - 1) / (UP_BN / 2);
    if (mf16) up_gemm<MODE_SWIGLU, 16>(s, a, NT, st);
    else up_gemm<MODE_SWIGLU, 32>(s, a, NT, st);
  } else {
    const int NT = (s.f + UP_BN - 1) / UP_BN;
    if (s.act == MOE_RELU) {
      if (mf16) up_gemm<MODE_RELU, 16>(s, a, NT, st);
      else up_gemm<MODE_RELU, 32>(s, a, NT, st);
    } else {
      if (mf16) up_gemm<MODE_GELU, 16>(s, a, NT, st);
      else up_gemm<MODE_GELU, 32>(s, a, NT, st);
    }
  }
  return hipGetLastError();
}

hipError_t launch_down(const Shape& s, const void* h, const void* w_down, const void* b_down,
                       const float* s_down, const int32_t* offsets, float* y_exp, float* y_part,
                       bool complete, hipStream_t st) {
  if (s.w_fp8() && !s.decode()) return hipErrorNotSupported;   // rejected by validation
  const void* bias = s.expert_bias() ? b_down : nullptr;
  if (s.dtype == MOE_F32) {
    const long long n = s.max_rows() * s.d;
    const int blocks = (int)((n + 255) / 256);
    gemm_f32_kernel<MODE_DOWN><<<blocks, 256, 0, st>>>(
        (const float*)h, (const float*)w_down, (const float*)bias, y_exp, offsets, nullptr, s.T,
        s.tok_div(), s.E, s.S, s.f, s.d, s.d, s.f);
    return hipGetLastError();
  }
  if (s.generic()) return launch_down_generic(s, h, w_down, b_down, offsets, y_exp, st);
  if (s.decode())
    return launch_decode_down(s, h, w_down, b_down, s_down, offsets, y_exp, y_part, complete, st);
  const int ks = down_ksplit(s);
  const long long part_elems = s.max_rows() * s.d;
  GemmArgs a{(const uint16_t*)h, (const uint16_t*)w_down, (const uint16_t*)bias, y_exp, offsets,
             nullptr, s.T, s.tok_div(), s.E, s.S, s.f, s.d, s.d, s.f, ks, y_part, part_elems, 0,
             s.max_rows() * s.f * 2};
  const int NT = (s.d + DN_BN - 1) / DN_BN;
  dn_gemm<MODE_DOWN>(long_launch(s, s.f, s.d), s.f / ks, a,
                     dim3(grid_blocks(s, DN_BM, NT, ks, DN_OCC)), st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ks == 1 || !complete) return e;
  const long long n = s.max_rows() * (s.d / 4);
  part_fold_kernel<<<(int)((n + 255) / 256), 256, 0, st>>>(y_exp, y_part, offsets, s.T, s.E, s.S,
                                                           s.d, ks - 1, part_elems);
  return hipGetLastError();
}

// ---------------------------------------------------------------- backward GEMMs
// out[r, n] = sum_j X[token of r, j] W_seg[n, j] (+ bias_seg[n]) for n < Wrows,
// over the routed and shared row segments; fp32 out [rows, Wrows].
hipError_t launch_bwd_lin(const Shape& s, const void* X, const void* W, const void* bias,
                          int Wrows, int K, float* out, const int32_t* offsets,
                          const int32_t* sorted_assign, hipStream_t st) {
  GemmArgs a{(const uint16_t*)X, (const uint16_t*)W, (const uint16_t*)bias, out, offsets,
             sorted_assign, s.T, s.tok_div(), s.E, s.S, K, Wrows, Wrows, s.f, 1, nullptr, 0, 0,
             (long long)s.T * K * 2};
  const int NT = (Wrows + DN_BN - 1) / DN_BN;
  dn_gemm<MODE_LIN>(long_launch(s, K, Wrows), K, a, dim3(grid_blocks(s, DN_BM, NT)), st);
  return hipGetLastError();
}

// out[r, n] = sum_j X[r, j] W_seg[n, j] for the rows X [rows, K] (bf16) and
// W [segments][N][K]; K slices as in the down projection (slice i > 0 into
// out2 + (i - 1) * part_elems).
hipError_t launch_bwd_dx(const Shape& s, const void* X, const void* W, int K, int N, float* out,
                         float* out2, long long part_elems, int ksplit, const int32_t* offsets,
                         hipStream_t st) {
  GemmArgs a{(const uint16_t*)X, (const uint16_t*)W, nullptr, out, offsets, nullptr, s.T,
             s.tok_div(), s.E, s.S, K, N, N, s.f, ksplit, out2, part_elems, 0,
             s.max_rows() * K * 2};
  const int NT = (N + DN_BN - 1) / DN_BN;
  dn_gemm<MODE_DXB>(long_launch(s, K, N), K / ksplit, a,
                    dim3(grid_blocks(s, DN_BM, NT, ksplit)), st);
  return hipGetLastError();
}

// out[seg] = A_seg B_seg^T: A [M, ldk] and B [N, ldk] bf16, segment seg
// reducing over its padded row range; fp32 out [segments][M][N].
hipError_t launch_bwd_wgrad(const Shape& s, const void* A, const void* B, int M, int N, int ldk,
                            float* out, const int32_t* offsets, hipStream_t st) {
  GemmArgs a{(const uint16_t*)A, (const uint16_t*)B, nullptr, out, offsets, nullptr, s.T,
             s.tok_div(), s.E, s.S, ldk, N, N, s.f, 1, nullptr, 0, M, (long long)M * ldk * 2};
  const long long tiles = (long long)(s.E + s.S) * ((M + DN_BM - 1) / DN_BM) *
                          ((N + DN_BN - 1) / DN_BN);
  long long g = tiles > kNumCUs ? kNumCUs : tiles;
  g = (g + 7) / 8 * 8;
  // the reduction runs over every segment's padded rows (multiples of 64);
  // long launches take the 16x16x32 loop with 64-deep k-tiles
  if (long_flops(2.0 * (double)M * (double)N * (double)ldk))
    grouped_gemm_kernel<DN_BM, DN_BN, DN_WGM, DN_WGN, MODE_WGRAD, DN_OCC, 16, 64>
        <<<(int)g, 64 * DN_WGM * DN_WGN, 0, st>>>(a);
  else
    grouped_gemm_kernel<DN_BM, DN_BN, DN_WGM, DN_WGN, MODE_WGRAD, DN_OCC, 32>
        <<<(int)g, 64 * DN_WGM * DN_WGN, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace moe
