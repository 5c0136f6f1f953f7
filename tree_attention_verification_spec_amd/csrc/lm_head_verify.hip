// The target model's LM head fused with the row statistics that verification reads.
//
// "EAGLE-3とMedusaで実装するSpeculative Decoding実践ガイド", section "並列検証：ターゲットモデルの
// 1回のforward passで一括確認する": one target pass gives the distribution T_p = softmax(W h_p) at
// every tree node ("多トークン予測（Medusa・EAGLE）", section "ツリー検証：候補を「木」に束ねて1回で
// 確かめる"); the guide's section "ドラフトヘッドの構成と学習手順" gives the Llama-3.1-8B-class
// shapes (hidden 4096, vocabulary 128256).  Verification reads only a few numbers per row -
// max, lowest argmax, S = sum exp(l - max), A = sum exp(l - max)(l - max) - and each child's
// logit in its parent's row, so the logits are reduced where they are produced and the
// B x N x V logits array is never written.
//
// lmhead_stats_kernel (M <= 64 hidden states): grid ceil(V / 64); a workgroup multiplies 64
// rows of W (four 16-row blocks, A operand of v_mfma_f32_16x16x32_bf16, 16-byte loads streamed
// from HBM) with all M hidden states (up to four 16-column blocks, B operand, L2-resident), K
// split over the four waves and summed in LDS.  The 64 x M logits tile then stays in LDS: per
// column, four threads reduce (max, lowest argmax) and then fp64 sums of fp32 exp(l - max), and
// the candidates whose token falls in the tile pick their parent's logit.  Partials go to the
// workspace, one per (row, 64 W rows).
// lmhead_stats_wide_kernel (65-128) and lmhead_stats_gemm_kernel (129-4096): every W tile must
// meet all hidden states, so these cover 256 W rows x 64 columns, or 256 W rows x 128 columns
// with W staged through LDS; the column blocks of one W tile get workgroup ids with the same
// residue mod 8, so they run on one XCD and read the tile through its L2.  Same partials and
// gathers.
// lmhead_merge_kernel: one workgroup per row; block max first, then the partials' sums rescaled
// by exp(m_j - max) in fp64 (no sequential rescaling), validation of the sequence's tree, and
// the outputs.
//
// At small M this is weight-streaming: W (1.05 GB at V = 128256, Dm = 4096) is read from HBM
// once; the hidden states (512 KB at 63 rows) are re-read from L2 by every workgroup, from a copy
// in fragment order (lmhead_xperm_kernel) so that each B-fragment load is four 256-byte runs.
#include <climits>

#include "common.h"

namespace spectree {
namespace {

constexpr int kLThreads = 256;
constexpr int kLKWaves = 4;                 // K slices per workgroup
constexpr int kLRB = 4;                     // 16-row blocks of W per workgroup
constexpr int kLRows = 16 * kLRB;           // vocabulary rows per workgroup
static_assert(kLRows == kWave && kLThreads == 4 * kLRows, "one token per lane, four threads per token");
constexpr int kLMaxCols = 64;               // hidden states (columns) per workgroup
constexpr int kLMaxRows = 4096;             // B * N limit
constexpr int kMergePer = 8;                // partials per merging thread held in registers
constexpr int kScanPer = 8;                 // tiles per thread in the typical bonus's scan

struct LmPart {       // one 64-token tile of one row
  double S;           // sum exp(l - m)
  double A;           // sum exp(l - m) (l - m)
  float m;            // tile max
  int argmax;         // lowest token id of the tile max (INT_MAX: none)
};

__device__ __forceinline__ bf16x8 ld8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Column stride of the fragment-ordered hidden states: M rounded up to 8 columns, so that every
// 16-lane run of a B fragment load starts on a 128-byte line (with a stride of M = 63 columns
// three of the four runs straddled lines; 243 -> 235 us at 63 rows).  The pad columns are never
// written or read.
__host__ __device__ constexpr int xp_stride(int M) { return (M + 7) & ~7; }

// Raw buffer loads (bounds-checked against the descriptor's byte count; the kernels keep every
// offset inside it): the descriptor is wave-uniform and lives in scalar registers.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
__device__ __forceinline__ BufRsrc buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ bf16x8 buf_ld8(BufRsrc r, uint32_t lane_off, uint32_t wave_off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, wave_off, 0));
}

// Optional output of the stats kernels (REJECT's residual draw needs the row it stops at): the
// fp32 logits of a 64-token x 64-column tile held in LDS as [token][column] are written to
// rows[column][token] (rows of V), lane = token so each store is one 256-byte run; the calling
// wave takes columns c_begin, c_begin + c_step, ...
__device__ __forceinline__ void store_tile_rows(const float (*tw)[kLMaxCols + 1], int vrow0, int ccol0,
                                                int c_begin, int c_step, int M, int V, float* __restrict__ rows) {
  const int lane = threadIdx.x & 63, v = vrow0 + lane;
  if (v >= V) return;
  for (int cc = c_begin; cc < kLMaxCols && ccol0 + cc < M; cc += c_step)
    rows[(size_t)(ccol0 + cc) * V + v] = tw[lane][cc];
}

template <int CBN>
__global__ __launch_bounds__(kLThreads) void lmhead_stats_kernel(
    const __bf16* __restrict__ W, const __bf16* __restrict__ Xp, int M, int Dm, int V, int N,
    int nblk, int ncb, const int32_t* __restrict__ parents, const int32_t* __restrict__ tokens,
    LmPart* __restrict__ parts, float* __restrict__ gath, float* __restrict__ rows) {
  // the K-slice partials and, once they are summed, the logits tile share one LDS block, so
  // two workgroups fit a CU
  constexpr size_t kRedBytes = sizeof(f32x4) * kLKWaves * kLRB * CBN * kWave;
  constexpr size_t kTileBytes = sizeof(float) * kLRows * (kLMaxCols + 1);
  __shared__ __attribute__((aligned(16))) unsigned char lds[kRedBytes > kTileBytes ? kRedBytes : kTileBytes];
  auto red = reinterpret_cast<f32x4 (*)[kLRB * CBN][kWave]>(lds);
  auto tile = reinterpret_cast<float (*)[kLMaxCols + 1]>(lds);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  // Workgroup id -> (W tile, column block): the ncb column blocks of a tile share id % 8, so
  // they run on one XCD (dispatch is round-robin over the 8) and read the tile through its L2.
  const int grp = blockIdx.x / (8 * ncb), rem = blockIdx.x - grp * 8 * ncb;
  const int tidx = grp * 8 + (rem & 7), cblk = rem >> 3;
  if (tidx >= nblk) return;
  const int row0 = tidx * kLRows, col0 = cblk * kLMaxCols;
  const int kslice = Dm / kLKWaves;
  const int kbeg = wave * kslice;
  // branch-free loads: rows past V and columns past M read the last valid one (never stored)
  const __bf16* arow[kLRB];
#pragma unroll
  for (int rb = 0; rb < kLRB; ++rb)
    arow[rb] = W + (size_t)min(row0 + rb * 16 + l16, V - 1) * Dm + kbeg + 8 * lg;
  // Xp is the hidden states in fragment order, element (col, k) at ((k / 8) Mp + col) 8 + k % 8
  // with Mp = xp_stride(M): a B fragment (lane l: column l % 16, k = 8 (l / 16) + [0, 8)) is four
  // 256-byte runs
  const int Mp = xp_stride(M);
  const __bf16* bptr[CBN];
#pragma unroll
  for (int cb = 0; cb < CBN; ++cb)
    bptr[cb] = Xp + ((size_t)(kbeg / 8 + lg) * Mp + min(col0 + cb * 16 + l16, M - 1)) * 8;
  f32x4 acc[kLRB][CBN];
#pragma unroll
  for (int rb = 0; rb < kLRB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CBN; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Two K steps per fetch, so both 64-byte halves of each 128-byte weight line are requested
  // back to back (one step per fetch left the second half to a later request, and a quarter of
  // the weight lines had left L2 by then: 1.36 GB read per launch for 1.05 GB of weights); two
  // slots, one pair of steps in flight while the other's products run.  Step indices are
  // clamped, so the loads past the last step re-read it inside the slice.
  const int steps = kslice / 32;
  struct Frags {
    bf16x8 a[kLRB][2];
    bf16x8 b[CBN][2];
  };
  auto fetch = [&](Frags& g, int s) {
#pragma unroll
    for (int rb = 0; rb < kLRB; ++rb)
#pragma unroll
      for (int h = 0; h < 2; ++h) g.a[rb][h] = ld8(arow[rb] + min(s + h, steps - 1) * 32);
#pragma unroll
    for (int cb = 0; cb < CBN; ++cb)
#pragma unroll
      for (int h = 0; h < 2; ++h) g.b[cb][h] = ld8(bptr[cb] + (size_t)min(s + h, steps - 1) * 32 * Mp);
  };
  auto products = [&](const Frags& g, int s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (s + h >= steps) break;
#pragma unroll
      for (int cb = 0; cb < CBN; ++cb)
#pragma unroll
        for (int rb = 0; rb < kLRB; ++rb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g.a[rb][h], g.b[cb][h], acc[rb][cb], 0, 0, 0);
    }
  };
  Frags g[2];
  fetch(g[0], 0);
  for (int s = 0; s < steps; s += 4) {
    fetch(g[1], s + 2);
    __builtin_amdgcn_sched_barrier(0);
    products(g[0], s);
    fetch(g[0], s + 4);
    __builtin_amdgcn_sched_barrier(0);
    products(g[1], s + 2);
  }
#pragma unroll
  for (int rb = 0; rb < kLRB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CBN; ++cb) red[wave][rb * CBN + cb][lane] = acc[rb][cb];
  __syncthreads();
  // the K slices summed (wave w takes the 16 x 16 blocks w, w + 4, ...), then written over the
  // partials as the logits tile (lane: column l16 of the block, rows 4 lg + e)
  constexpr int kPerWave = (kLRB * CBN + kLKWaves - 1) / kLKWaves;
  f32x4 sums[kPerWave];
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int t = wave + j * kLKWaves;
    if (t < kLRB * CBN) sums[j] = red[0][t][lane] + red[1][t][lane] + red[2][t][lane] + red[3][t][lane];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int t = wave + j * kLKWaves;
    if (t < kLRB * CBN) {
      const int rb = t / CBN, cb = t % CBN;
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[rb * 16 + 4 * lg + e][cb * 16 + l16] = sums[j][e];
    }
  }
  __syncthreads();
  if (rows) store_tile_rows(tile, row0, col0, wave, kLKWaves, M, V, rows);

  // per column: four consecutive threads share the tile's 64 rows, 16 each
  const int col = threadIdx.x >> 2, q = threadIdx.x & 3;
  float m = -INFINITY;
  int am = INT_MAX;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int vr = q * 16 + j;
    const float x = tile[vr][col];
    if (row0 + vr < V && x > m) {          // ascending ids: strict > keeps the lowest
      m = x;
      am = row0 + vr;
    }
  }
#pragma unroll
  for (int o = 1; o < 4; o <<= 1) {
    const float m2 = __shfl_xor(m, o);
    const int a2 = __shfl_xor(am, o);
    if (m2 > m || (m2 == m && a2 < am)) {
      m = m2;
      am = a2;
    }
  }
  double S = 0.0, A = 0.0;
  if (m != -INFINITY) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int vr = q * 16 + j;
      if (row0 + vr < V) {
        const float d = tile[vr][col] - m;
        const double e = (double)expf(d);
        S += e;
        A += e * (double)d;
      }
    }
  }
#pragma unroll
  for (int o = 1; o < 4; o <<= 1) {
    S += __shfl_xor(S, o);
    A += __shfl_xor(A, o);
  }
  if (q == 0 && col0 + col < M) parts[(size_t)(col0 + col) * nblk + tidx] = LmPart{S, A, m, am};

  // the candidates whose parent's column is in this block and whose token lies in this tile take
  // their parent's logit (only the sequences overlapping the block are scanned)
  const int c_lo = (col0 / N) * N, c_hi = min(M, (min(col0 + kLMaxCols, M) - 1) / N * N + N);
  for (int c = c_lo + threadIdx.x; c < c_hi; c += kLThreads) {
    const int i = c % N;
    if (i == 0) continue;
    const int p = parents[c], x = tokens[c];
    const int pc = c - i + p;
    if (p >= 0 && p < i && pc >= col0 && pc < col0 + kLMaxCols && x >= row0 && x < row0 + kLRows && x < V)
      gath[c] = tile[x - row0][pc - col0];
  }
}

// More than 64 hidden states: every 64-row W tile meets all of them, so what bounds the kernel
// above is re-reading the hidden states (16 MB at 2032 rows) once per 64 W rows.  Here a
// workgroup covers 256 W rows x 64 columns: each wave owns 64 W rows over the whole K (no K
// split, no LDS reduction) and the four waves read the same B fragments, so the column block is
// fetched into the CU once per 256 W rows.  The tiles are then written to LDS (one 64 x 64 tile
// per wave) and reduced per column by the wave's 64 lanes, with the same partials and gathers
// as above.
constexpr int kWRowsPerWave = 64;
constexpr int kWRows = kWRowsPerWave * kLKWaves;   // W rows per workgroup

__global__ __launch_bounds__(kLThreads) void lmhead_stats_wide_kernel(
    const __bf16* __restrict__ W, const __bf16* __restrict__ Xp, int M, int Dm, int V, int N,
    int nblk, int ntile, int ncb, const int32_t* __restrict__ parents,
    const int32_t* __restrict__ tokens, LmPart* __restrict__ parts, float* __restrict__ gath,
    float* __restrict__ rows) {
  __shared__ float tile[kLKWaves][kWRowsPerWave][kLMaxCols + 1];
  constexpr int RB = kWRowsPerWave / 16, CBN = kLMaxCols / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int grp = blockIdx.x / (8 * ncb), rem = blockIdx.x - grp * 8 * ncb;
  const int tidx = grp * 8 + (rem & 7), cblk = rem >> 3;
  if (tidx >= ntile) return;
  const int wrow0 = tidx * kWRows + wave * kWRowsPerWave, col0 = cblk * kLMaxCols;
  const __bf16* arow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    arow[rb] = W + (size_t)min(wrow0 + rb * 16 + l16, V - 1) * Dm + 8 * lg;
  const int Mp = xp_stride(M);
  const __bf16* bptr[CBN];
#pragma unroll
  for (int cb = 0; cb < CBN; ++cb) bptr[cb] = Xp + ((size_t)lg * Mp + min(col0 + cb * 16 + l16, M - 1)) * 8;
  f32x4 acc[RB][CBN];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CBN; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // two K steps per fetch (both halves of each 128-byte weight line back to back), two slots,
  // as in lmhead_stats_kernel
  const int steps = Dm / 32;
  struct Frags {
    bf16x8 a[RB][2];
    bf16x8 b[CBN][2];
  };
  auto fetch = [&](Frags& g, int s) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int h = 0; h < 2; ++h) g.a[rb][h] = ld8(arow[rb] + min(s + h, steps - 1) * 32);
#pragma unroll
    for (int cb = 0; cb < CBN; ++cb)
#pragma unroll
      for (int h = 0; h < 2; ++h) g.b[cb][h] = ld8(bptr[cb] + (size_t)min(s + h, steps - 1) * 32 * Mp);
  };
  auto products = [&](const Frags& g, int s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (s + h >= steps) break;
#pragma unroll
      for (int cb = 0; cb < CBN; ++cb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g.a[rb][h], g.b[cb][h], acc[rb][cb], 0, 0, 0);
    }
  };
  Frags g[2];
  fetch(g[0], 0);
  for (int s = 0; s < steps; s += 4) {
    fetch(g[1], s + 2);
    __builtin_amdgcn_sched_barrier(0);
    products(g[0], s);
    fetch(g[0], s + 4);
    __builtin_amdgcn_sched_barrier(0);
    products(g[1], s + 2);
  }
  float (*tw)[kLMaxCols + 1] = tile[wave];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CBN; ++cb)
#pragma unroll
      for (int e = 0; e < 4; ++e) tw[rb * 16 + 4 * lg + e][cb * 16 + l16] = acc[rb][cb][e];
  __syncthreads();
  if (rows) store_tile_rows(tw, wrow0, col0, 0, 1, M, V, rows);
  // lane = column: max and lowest argmax over the wave's 64 rows, then fp64 sums
  const int col = lane;
  float m = -INFINITY;
  int am = INT_MAX;
  for (int vr = 0; vr < kWRowsPerWave; ++vr) {
    const float x = tw[vr][col];
    if (wrow0 + vr < V && x > m) {
      m = x;
      am = wrow0 + vr;
    }
  }
  double S = 0.0, A = 0.0;
  if (m != -INFINITY) {
    for (int vr = 0; vr < kWRowsPerWave && wrow0 + vr < V; ++vr) {
      const float d = tw[vr][col] - m;
      const double e = (double)expf(d);
      S += e;
      A += e * (double)d;
    }
  }
  const int wt = tidx * kLKWaves + wave;          // this wave's 64-row tile among the nblk
  if (col0 + col < M && wt < nblk) parts[(size_t)(col0 + col) * nblk + wt] = LmPart{S, A, m, am};
  const int c_lo = (col0 / N) * N, c_hi = min(M, (min(col0 + kLMaxCols, M) - 1) / N * N + N);
  for (int c = c_lo + lane; c < c_hi; c += kWave) {
    const int i = c % N;
    if (i == 0) continue;
    const int p = parents[c], x = tokens[c];
    const int pc = c - i + p;
    if (p >= 0 && p < i && pc >= col0 && pc < col0 + kLMaxCols && x >= wrow0 && x < wrow0 + kWRowsPerWave && x < V)
      gath[c] = tw[x - wrow0][pc - col0];
  }
}

// Per-column reduction of one wave's 64 x 64 logits tile in LDS (lane = column): the (row,
// 64-row tile) partial and the gathers of the candidates whose parent's column and token fall in
// the tile.
__device__ __forceinline__ void wave_tile_epilogue(float (*tw)[kLMaxCols + 1], int wrow0, int wcol0, int M,
                                                   int V, int N, int nblk, const int32_t* __restrict__ parents,
                                                   const int32_t* __restrict__ tokens, LmPart* __restrict__ parts,
                                                   float* __restrict__ gath, float* __restrict__ rows) {
  if (rows) store_tile_rows(tw, wrow0, wcol0, 0, 1, M, V, rows);
  const int lane = threadIdx.x & 63;
  const int col = lane;
  float m = -INFINITY;
  int am = INT_MAX;
  for (int vr = 0; vr < 64; ++vr) {
    const float x = tw[vr][col];
    if (wrow0 + vr < V && x > m) {
      m = x;
      am = wrow0 + vr;
    }
  }
  double S = 0.0, A = 0.0;
  if (m != -INFINITY) {
    for (int vr = 0; vr < 64 && wrow0 + vr < V; ++vr) {
      const float d = tw[vr][col] - m;
      const double e = (double)expf(d);
      S += e;
      A += e * (double)d;
    }
  }
  const int wt = wrow0 / 64;
  if (wcol0 + col < M && wt < nblk) parts[(size_t)(wcol0 + col) * nblk + wt] = LmPart{S, A, m, am};
  if (wcol0 < M) {
    const int c_lo = (wcol0 / N) * N, c_hi = min(M, (min(wcol0 + kLMaxCols, M) - 1) / N * N + N);
    for (int c = c_lo + lane; c < c_hi; c += kWave) {
      const int i = c % N;
      if (i == 0) continue;
      const int p = parents[c], x = tokens[c];
      const int pc = c - i + p;
      if (p >= 0 && p < i && pc >= wcol0 && pc < wcol0 + kLMaxCols && x >= wrow0 && x < wrow0 + 64 && x < V)
        gath[c] = tw[x - wrow0][pc - wcol0];
    }
  }
}

// More than 128 hidden states: 256 W rows x 128 columns per workgroup, waves in 2 x 2, each 128
// W rows x 64 columns (per 32-wide K step a wave reads 12 fragments for 32 products), two
// workgroups per CU.  W goes through LDS, the hidden states straight to registers: a fragment
// load of W puts 16 different rows in each 16 lanes, so each group of four lanes would meet four
// cache lines and take the load unit four times as long, while the staging loads give each group
// of four lanes one row's 64 bytes, and the permuted hidden states are already in fragment
// order.  The staged W tile is stored unpadded, each row's four 16-byte chunks permuted by
// w_swz(row) = (row / 2) % 4, with which a fragment read (16 rows, one chunk each) takes the
// LDS's minimum of four clocks per instruction (measured with the bank-conflict counter; rows
// 80 bytes apart, unpermuted 64-byte rows and the other XOR permutations of the chunk index by
// two row bits take eight).  Three LDS buffers: the fragments of
// step s + 1 are read while step s's products run, and one barrier per step separates every
// write from the reads of the same buffer.
constexpr int kGT = 128;                 // columns per workgroup
constexpr int kG2Rows = 256;             // W rows per workgroup
__device__ __forceinline__ int w_swz(int r) { return (r >> 1) & 3; }

__global__ __launch_bounds__(kLThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void lmhead_stats_gemm_kernel(
    const __bf16* __restrict__ W, const __bf16* __restrict__ Xp, int M, int Dm, int V, int N,
    int nblk, int ntile, int ncb, const int32_t* __restrict__ parents,
    const int32_t* __restrict__ tokens, LmPart* __restrict__ parts, float* __restrict__ gath,
    float* __restrict__ rows) {
  constexpr int kBufs = 3;
  constexpr int kStageBytes1 = kG2Rows * 64;                                        // one step's W tile
  constexpr size_t kTileBytes = sizeof(float) * kLKWaves * 64 * (kLMaxCols + 1);  // a tile per wave
  constexpr size_t kLds = (size_t)kBufs * kStageBytes1 > kTileBytes ? (size_t)kBufs * kStageBytes1 : kTileBytes;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLds];
  auto tiles = reinterpret_cast<float (*)[64][kLMaxCols + 1]>(lds);
  constexpr int RB = 8, CBN = 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int wr = wave >> 1, wc = wave & 1;
  const int grp = blockIdx.x / (8 * ncb), rem = blockIdx.x - grp * 8 * ncb;
  const int tidx = grp * 8 + (rem & 7), cblk = rem >> 3;
  if (tidx >= ntile) return;
  const int row0 = tidx * kG2Rows, col0 = cblk * kGT;
  const uint32_t row_bytes = (uint32_t)Dm * sizeof(__bf16);
  const int arow0 = min(row0, V - 1);
  const BufRsrc wrs = buf_rsrc(W + (size_t)arow0 * Dm, (uint32_t)min(kG2Rows, V - arow0) * row_bytes);
  const int Mp = xp_stride(M);
  const BufRsrc xr = buf_rsrc(Xp, (uint32_t)Mp * row_bytes);
  // staging: thread t moves 16-byte slots q = t + 256 j (row q / 4, slot q % 4, which holds the
  // row's chunk (q % 4) ^ w_swz(row)); LDS address of slot q: 16 q
  uint32_t aoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = threadIdx.x + j * kLThreads, r = q >> 2;
    aoff[j] = (uint32_t)(min(row0 + r, V - 1) - arow0) * row_bytes + 16 * ((q & 3) ^ w_swz(r));
  }
  // B fragments of this wave's column block cb: 16 bytes at Xp[(4 s + lg) Mp + column]
  uint32_t boff[CBN];
#pragma unroll
  for (int cb = 0; cb < CBN; ++cb) boff[cb] = (uint32_t)(lg * Mp + min(col0 + wc * 64 + cb * 16 + l16, M - 1)) * 16;
  const int steps = Dm / 32;
  bf16x8 rav[4];
  auto load_a = [&](int s) {
    const uint32_t so = (uint32_t)min(s, steps - 1) * 64;
#pragma unroll
    for (int j = 0; j < 4; ++j) rav[j] = buf_ld8(wrs, aoff[j], so);
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<bf16x8*>(lds + buf * kStageBytes1 + (threadIdx.x + j * kLThreads) * 16) = rav[j];
  };
  bf16x8 fa[RB], fb[2][CBN];
  auto fetch_b = [&](int slot, int s) {
    const uint32_t so = (uint32_t)min(s, steps - 1) * 64 * (uint32_t)Mp;
#pragma unroll
    for (int cb = 0; cb < CBN; ++cb) fb[slot][cb] = buf_ld8(xr, boff[cb], so);
  };
  auto read_a = [&](int rb, int buf) {
    const int r = wr * 128 + rb * 16 + l16;
    fa[rb] = *reinterpret_cast<const bf16x8*>(lds + buf * kStageBytes1 + r * 64 + 16 * (lg ^ w_swz(r)));
  };
  f32x4 acc[RB][CBN];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CBN; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Step s (LDS buffer of step t: t % 3): W of step s + 2 (in registers since step s - 1) to its
  // buffer, W of step s + 3 and the B fragments of step s + 1 requested, then step s's products,
  // row block by row block, each followed by the read of that block's fragment for step s + 1
  // into the register it frees.  The buffer written at step s was last read during step s - 2,
  // before the barrier that ends step s - 1; the one read at step s was written at step s - 1,
  // before that same barrier.  Past the last step the loads and LDS traffic repeat in-bounds data
  // that is never used.
  auto step = [&](int s, int slot) __attribute__((always_inline)) {
    store_a((s + 2) % kBufs);
    load_a(s + 3);
    fetch_b(slot ^ 1, s + 1);
    __builtin_amdgcn_sched_barrier(0);
    const int nb = (s + 1) % kBufs;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int cb = 0; cb < CBN; ++cb)
        acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[rb], fb[slot][cb], acc[rb][cb], 0, 0, 0);
      read_a(rb, nb);
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);    // four products
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // one LDS read
    }
    __syncthreads();
  };
  load_a(0);
  store_a(0);
  load_a(1);
  store_a(1);
  load_a(2);
  fetch_b(0, 0);
  __syncthreads();
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) read_a(rb, 0);
  for (int s = 0; s < steps; s += 2) {
    step(s, 0);
    step(s + 1, 1);
  }
  // the wave's 128 x 64 tile to LDS (over the staging buffers) and reduced 64 rows at a time
  float (*tw)[kLMaxCols + 1] = tiles[wave];
#pragma unroll
  for (int hr = 0; hr < 2; ++hr) {
#pragma unroll
    for (int rb = 0; rb < RB / 2; ++rb)
#pragma unroll
      for (int cb = 0; cb < CBN; ++cb)
#pragma unroll
        for (int e = 0; e < 4; ++e) tw[rb * 16 + 4 * lg + e][cb * 16 + l16] = acc[hr * RB / 2 + rb][cb][e];
    __syncthreads();
    wave_tile_epilogue(tw, row0 + wr * 128 + hr * 64, col0 + wc * 64, M, V, N, nblk, parents, tokens, parts,
                       gath, rows);
    __syncthreads();
  }
}

// The hidden states [M, Dm] into fragment order (see lmhead_stats_kernel; column stride
// xp_stride(M)), 16 bytes per thread.
__global__ __launch_bounds__(kLThreads) void lmhead_xperm_kernel(const __bf16* __restrict__ X, int M, int Dm,
                                                                 __bf16* __restrict__ Xp) {
  const int id = blockIdx.x * kLThreads + threadIdx.x;     // (k / 8) * M + col
  const int K8 = Dm / 8;
  if (id >= K8 * M) return;
  const int k8 = id / M, col = id - k8 * M;
  *reinterpret_cast<bf16x8*>(Xp + ((size_t)k8 * xp_stride(M) + col) * 8) = ld8(X + (size_t)col * Dm + (size_t)k8 * 8);
}

__global__ __launch_bounds__(kLThreads) void lmhead_merge_kernel(
    const LmPart* __restrict__ parts, const float* __restrict__ gath, int nblk, int N, int V,
    const int32_t* __restrict__ parents, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ n_nodes, float* __restrict__ row_max, int32_t* __restrict__ row_argmax,
    double* __restrict__ row_sum, double* __restrict__ row_ent, float* __restrict__ cand_logit,
    int32_t* __restrict__ err) {
  __shared__ float s_m[kLThreads / kWave];
  __shared__ int s_a[kLThreads / kWave];
  __shared__ double s_S[kLThreads / kWave], s_A[kLThreads / kWave];
  __shared__ int s_err;
  const int col = blockIdx.x;
  const int b = col / N, i = col - b * N;
  const int t = threadIdx.x, lane = t & (kWave - 1), wv = t >> 6;
  if (t == 0) s_err = INT_MAX;
  __syncthreads();
  // the sequence's tree, validated by every column of the sequence (N <= 64)
  const int n = n_nodes ? n_nodes[b] : N;
  const bool bad_n = n < 0 || n > N;
  if (!bad_n && t < n) {
    const int p = parents[(size_t)b * N + t], x = tokens[(size_t)b * N + t];
    int code = 0;
    if (t == 0) {
      if (p != -1) code = SPEC_ERR_ROOT;
    } else if (p < 0 || p >= t) {
      code = SPEC_ERR_PARENT;
    } else if (x < 0 || x >= V) {
      code = SPEC_ERR_TOKEN;
    }
    if (code) atomicMin(&s_err, err_word(t, code));
  }
  // block max, lowest argmax among the tiles holding it; up to kMergePer partials per thread
  // are requested at once and kept for the sums (more than that: a strided loop)
  const LmPart* pp = parts + (size_t)col * nblk;
  const bool held = nblk <= kLThreads * kMergePer;
  LmPart mine[kMergePer];
  float m = -INFINITY;
  int am = INT_MAX;
  if (held) {
#pragma unroll
    for (int u = 0; u < kMergePer; ++u) {
      const int j = t + u * kLThreads;
      mine[u] = j < nblk ? pp[j] : LmPart{0.0, 0.0, -INFINITY, INT_MAX};
    }
#pragma unroll
    for (int u = 0; u < kMergePer; ++u) {
      if (mine[u].m > m || (mine[u].m == m && mine[u].argmax < am)) {
        m = mine[u].m;
        am = mine[u].argmax;
      }
    }
  } else {
    for (int j = t; j < nblk; j += kLThreads) {
      const float mj = pp[j].m;
      const int aj = pp[j].argmax;
      if (mj > m || (mj == m && aj < am)) {
        m = mj;
        am = aj;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o);
    const int a2 = __shfl_xor(am, o);
    if (m2 > m || (m2 == m && a2 < am)) {
      m = m2;
      am = a2;
    }
  }
  if (lane == 0) {
    s_m[wv] = m;
    s_a[wv] = am;
  }
  __syncthreads();
  m = s_m[0];
  am = s_a[0];
#pragma unroll
  for (int w = 1; w < kLThreads / kWave; ++w) {
    if (s_m[w] > m || (s_m[w] == m && s_a[w] < am)) {
      m = s_m[w];
      am = s_a[w];
    }
  }
  // sums rescaled to the row max: A_j is relative to m_j, so A += e (A_j + (m_j - M) S_j)
  double S = 0.0, A = 0.0;
  auto add = [&](const LmPart& pj) {
    if (pj.m != -INFINITY) {
      const double d = (double)pj.m - (double)m;
      const double e = exp(d);
      S += e * pj.S;
      A += e * (pj.A + d * pj.S);
    }
  };
  if (held) {
#pragma unroll
    for (int u = 0; u < kMergePer; ++u) add(mine[u]);
  } else {
    for (int j = t; j < nblk; j += kLThreads) add(pp[j]);
  }
  S = wave_sum(S);
  A = wave_sum(A);
  if (lane == 0) {
    s_S[wv] = S;
    s_A[wv] = A;
  }
  __syncthreads();
  if (t == 0) {
    S = 0.0;
    A = 0.0;
    for (int w = 0; w < kLThreads / kWave; ++w) {
      S += s_S[w];
      A += s_A[w];
    }
    const int e = bad_n ? err_word(0, SPEC_ERR_NNODES) : (s_err == INT_MAX ? 0 : s_err);
    const bool ok = e == 0 && i < n;
    row_max[col] = ok ? m : NAN;
    row_argmax[col] = ok ? am : -1;
    row_sum[col] = ok ? S : NAN;
    row_ent[col] = ok ? A : NAN;
    cand_logit[col] = (ok && i > 0) ? gath[col] : NAN;
    if (i == 0) err[b] = e;
  }
}


// Rejection-sampling arguments of verify_lm_kernel and the plan it leaves for the residual draw:
// plan[3b] = 1 when sequence b's bonus is a residual draw (else 0), plan[3b + 1] its draft row,
// plan[3b + 2] the kept node m.
struct LmDraft {
  const float* draft;       // [B, R, Vd]
  const int32_t* draft_row; // [B, N]
  const int32_t* t2d;       // [V] or NULL
  int R, Vd;
  int32_t* plan;            // [B, 3]
};

// Weight of token v in a residual draw from row m (logit l, statistics M and 1/S): the residual
// relu(T[v] - D[v]) with T[v] = exp(l - M) / S, or T[v] itself when the residual has no mass.
// Draft ids come through t2d when the draft vocabulary differs; an id outside it has D = 0.
__device__ __forceinline__ double draw_weight(float l, float M, double invS, const float* __restrict__ drow,
                                              const LmDraft& dr, int v, bool resid) {
  const double e = (double)expf(l - M) * invS;
  if (!resid) return e;
  const int dx = dr.t2d ? dr.t2d[v] : v;
  const double d = (dx >= 0 && dx < dr.Vd) ? (double)drow[dx] : 0.0;
  return fmax(e - d, 0.0);
}

// Tile sums of row m for a sequence whose bonus is a residual draw: grid (four 64-token tiles,
// sequence), one wave per tile, lane = token; row m's logits were stored by the stats kernel.
// Each tile leaves its fp64 (residual, target) weight sums for the draw's scan.
__global__ __launch_bounds__(kLThreads) void lm_tilesum_kernel(
    const float* __restrict__ rows, int N, int V, int nblk, const float* __restrict__ row_max,
    const double* __restrict__ row_sum, LmDraft dr, double2* __restrict__ tsum) {
  const int b = blockIdx.y, lane = threadIdx.x & (kWave - 1);
  const int tile = blockIdx.x * (kLThreads / kWave) + (threadIdx.x >> 6);
  if (dr.plan[3 * b] != 1 || tile >= nblk) return;
  const int r = dr.plan[3 * b + 1], m = dr.plan[3 * b + 2];
  const int v = tile * kLRows + lane;
  double wr = 0.0, wt = 0.0;
  if (v < V) {
    const float l = rows[((size_t)b * N + m) * V + v];
    const float M = row_max[(size_t)b * N + m];
    const double invS = 1.0 / row_sum[(size_t)b * N + m];
    const float* drow = dr.draft + ((size_t)b * dr.R + r) * dr.Vd;
    wr = draw_weight(l, M, invS, drow, dr, v, true);
    wt = draw_weight(l, M, invS, drow, dr, v, false);
  }
  wr = wave_sum(wr);
  wt = wave_sum(wt);
  if (lane == 0) tsum[(size_t)b * nblk + tile] = make_double2(wr, wt);
}

// The residual draw: q_v = relu(T[v] - D[v]) over row m, u Q placed by inverse CDF
// (Q the sum of the tiles' residual sums; a residual of zero mass draws from T_m instead).  One
// workgroup per sequence: a block scan over the tile sums finds the tile holding u Q, then one
// wave scans that tile's 64 weights, the remainder scaled to the wave's own total of the tile
// (equal to the stored sum up to the order of the fp64 additions).
__global__ __launch_bounds__(kLThreads) void lm_residual_kernel(
    const float* __restrict__ rows, const double2* __restrict__ tsum, int nblk,
    const float* __restrict__ row_max, const double* __restrict__ row_sum,
    const float* __restrict__ uniforms, int N, int V, LmDraft dr, int32_t* __restrict__ bonus) {
  __shared__ double s_w[kLThreads / kWave];
  __shared__ int s_tile;
  __shared__ double s_pre;
  const int b = blockIdx.x, t = threadIdx.x, lane = t & (kWave - 1), wv = t >> 6;
  if (dr.plan[3 * b] != 1) return;
  const int r = dr.plan[3 * b + 1], m = dr.plan[3 * b + 2];
  const double2* ts = tsum + (size_t)b * nblk;
  // total residual mass (fixed order: per-thread strided sums, then the waves in order)
  double part = 0.0;
  for (int j = t; j < nblk; j += kLThreads) part += ts[j].x;
  part = wave_sum(part);
  if (lane == 0) s_w[wv] = part;
  if (t == 0) {
    s_tile = -1;
    s_pre = -1.0;
  }
  __syncthreads();
  double Q = 0.0;
  for (int q = 0; q < kLThreads / kWave; ++q) Q += s_w[q];
  const bool resid = Q > 0.0;
  if (!resid) {
    __syncthreads();
    part = 0.0;
    for (int j = t; j < nblk; j += kLThreads) part += ts[j].y;
    part = wave_sum(part);
    if (lane == 0) s_w[wv] = part;
    __syncthreads();
    Q = 0.0;
    for (int q = 0; q < kLThreads / kWave; ++q) Q += s_w[q];
  }
  __syncthreads();
  const double target = (double)uniforms[(size_t)b * N] * Q;
  // chunks of kLThreads tiles: each thread's tile weight, a block scan, the first crossing
  double carry = 0.0;
  for (int j0 = 0; j0 < nblk; j0 += kLThreads) {
    const int j = j0 + t;
    const double wj = j < nblk ? (resid ? ts[j].x : ts[j].y) : 0.0;
    double incl = wj;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const double y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == kWave - 1) s_w[wv] = incl;
    __syncthreads();
    double off = carry;
    for (int q = 0; q < wv; ++q) off += s_w[q];
    const double before = off + incl - wj;
    if (wj > 0.0 && before <= target && target < before + wj) {
      s_tile = j;                            // one thread at most: the ranges are disjoint
      s_pre = before;
    }
    double tot = 0.0;
    for (int q = 0; q < kLThreads / kWave; ++q) tot += s_w[q];
    carry += tot;
    __syncthreads();
    if (s_tile >= 0) break;                  // uniform: read after the barrier
  }
  if (wv != 0) return;
  int tile = s_tile;
  const bool last = tile < 0;                // u Q at or past the rounded total: the last token
  if (last) {                                // with weight of the last tile with weight
    tile = nblk - 1;
    while (tile > 0 && !((resid ? ts[tile].x : ts[tile].y) > 0.0)) --tile;
  }
  const float M = row_max[(size_t)b * N + m];
  const double invS = 1.0 / row_sum[(size_t)b * N + m];
  const float* drow = dr.draft + ((size_t)b * dr.R + r) * dr.Vd;
  const int v = tile * kLRows + lane;
  const double w = v < V ? draw_weight(rows[((size_t)b * N + m) * V + v], M, invS, drow, dr, v, resid) : 0.0;
  double incl = w;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  const double tot = __shfl(incl, kWave - 1);
  const double stored = resid ? ts[tile].x : ts[tile].y;
  const double rem = last ? tot : (target - s_pre) / stored * tot;
  const unsigned long long cross = __ballot(w > 0.0 && incl > rem);
  const unsigned long long pos = __ballot(w > 0.0);
  int pick;
  if (cross) pick = __ffsll((long long)cross) - 1;
  else pick = pos ? 63 - __clzll((long long)pos) : 0;
  if (lane == 0) bonus[b] = tile * kLRows + pick;
}

// Greedy or typical verification straight from the LM head's statistics, with the bonus token.
// One workgroup per sequence.  Node c (parent p, token x): GREEDY accepts iff x is p's lowest
// argmax; TYPICAL iff T_p[x] = exp(l_p[x] - max_p) / S_p >= min(eps, delta exp(-H_p)), with
// H_p = ln S_p - A_p / S_p (fp64, T from the same fp32 exponential the sums were built from).
// Survival, the deepest survivor m and the path as spec_verify.  The bonus: GREEDY the argmax of
// row m; TYPICAL a draw from T_m by inverse CDF with u = uniforms[b, 0]: the 64-token tile
// holding u Z is found from the per-tile sums the LM head left in the workspace (Z = sum_j
// S_j e^(m_j - M)), the tile's 64 logits are recomputed (fp32 dot products), and the token is
// the first whose running weight exceeds the remainder (scaled to the recomputed tile's total,
// which differs from the stored sum only by fp32 rounding).
__global__ __launch_bounds__(SPEC_MAX_NODES) void verify_lm_kernel(
    const float* __restrict__ row_max, const int32_t* __restrict__ row_argmax,
    const double* __restrict__ row_sum, const double* __restrict__ row_ent,
    const float* __restrict__ cand, const LmPart* __restrict__ parts, int nblk,
    const __bf16* __restrict__ X, const __bf16* __restrict__ W, int Dm,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ parents,
    const int32_t* __restrict__ n_nodes, const float* __restrict__ uniforms, int N, int V,
    int max_depth, int mode, float eps, float delta, LmDraft dr, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ path, int32_t* __restrict__ bonus, uint8_t* __restrict__ node_accept,
    int32_t* __restrict__ err) {
  __shared__ int s_par[SPEC_MAX_NODES];
  __shared__ unsigned char s_acc[SPEC_MAX_NODES];
  __shared__ int s_err, s_best, s_kid;
  __shared__ double s_wsum[SPEC_MAX_NODES / kWave];
  __shared__ int s_tile;
  __shared__ double s_pre, s_scale;
  __shared__ float s_logit[kLRows];
  const int b = blockIdx.x, c = threadIdx.x;
  const int lane = c & (kWave - 1), wv = c >> 6;
  const size_t base = (size_t)b * N;
  const int n_raw = n_nodes ? n_nodes[b] : N;
  const bool bad_n = n_raw < 0 || n_raw > N;
  const int n = bad_n ? 0 : n_raw;
  if (c == 0) {
    s_err = INT_MAX;
    s_best = -1;
    s_kid = INT_MAX;
  }
  if (c < N) s_par[c] = parents[base + c];
  __syncthreads();
  int depth = 0;
  bool acc = false;
  if (c < n) {
    const int p = s_par[c];
    int code = 0;
    if (c == 0) {
      if (p != -1) code = SPEC_ERR_ROOT;
      acc = true;
    } else if (p < 0 || p >= c) {
      code = SPEC_ERR_PARENT;
    } else {
      int j = c;
      while (j > 0 && s_par[j] >= 0 && s_par[j] < j) {
        j = s_par[j];
        ++depth;
      }
      const int x = tokens[base + c];
      if (depth > max_depth) code = SPEC_ERR_DEPTH;
      else if (x < 0 || x >= V) code = SPEC_ERR_TOKEN;
      else if (mode == SPEC_VERIFY_GREEDY) acc = x == row_argmax[base + p];
      else {
        const double S = row_sum[base + p];
        const double T = (double)expf(cand[base + c] - row_max[base + p]) / S;
        if (mode == SPEC_VERIFY_TYPICAL) {
          const double H = log(S) - row_ent[base + p] / S;
          acc = T >= fmin((double)eps, (double)delta * exp(-H));
        } else {                              // REJECT: u D[x] < T[x]
          const int r = dr.draft_row[base + c];
          const int dx = dr.t2d ? dr.t2d[x] : x;
          if (r < 0 || r >= dr.R) code = SPEC_ERR_DRAFTROW;
          else if (dx < -1 || dx >= dr.Vd) code = SPEC_ERR_MAP;
          else {
            const double D = dx >= 0 ? (double)dr.draft[((size_t)b * dr.R + r) * dr.Vd + dx] : 0.0;
            acc = (double)uniforms[base + c] * D < T;
          }
        }
      }
    }
    if (code) atomicMin(&s_err, err_word(c, code));
    s_acc[c] = acc ? 1 : 0;
  }
  __syncthreads();
  const int e = bad_n ? err_word(0, SPEC_ERR_NNODES) : (s_err == INT_MAX ? 0 : s_err);
  if (e == 0 && c < n) {
    bool live = true;
    for (int j = c; j > 0; j = s_par[j]) live = live && s_acc[j];
    if (live) atomicMax(&s_best, (depth << 9) | (511 - c));
  }
  __syncthreads();
  if (c < N && node_accept) node_accept[base + c] = (e == 0 && c < n) ? s_acc[c] : 0;
  const bool ok = e == 0 && n > 0;
  const int m = ok ? 511 - (s_best & 511) : 0;
  if (c == 0) {
    int32_t* pr = path + (size_t)b * (max_depth + 1);
    for (int k = 0; k <= max_depth; ++k) pr[k] = -1;
    int len = 0;
    if (ok) {
      len = s_best >> 9;
      for (int j = m, k = len; k >= 0; --k, j = s_par[j]) pr[k] = j;
    }
    accept_len[b] = len;
    err[b] = e;
    if (!ok) bonus[b] = -1;
    else if (mode == SPEC_VERIFY_GREEDY) bonus[b] = row_argmax[base + m];
  }
  if (mode == SPEC_VERIFY_REJECT && c == 0) dr.plan[3 * b] = 0;
  if (!ok || mode == SPEC_VERIFY_GREEDY) return;            // uniform across the workgroup
  if (mode == SPEC_VERIFY_REJECT) {
    // m with children: a residual draw over the whole row (lm_tilesum_kernel, lm_residual_kernel)
    if (c < n && c > 0 && s_par[c] == m) atomicMin(&s_kid, c);
    __syncthreads();
    if (s_kid != INT_MAX) {
      if (c == 0) {
        dr.plan[3 * b] = 1;
        dr.plan[3 * b + 1] = dr.draft_row[base + s_kid];
        dr.plan[3 * b + 2] = m;
      }
      return;                                // uniform: s_kid read after the barrier
    }
  }

  // ---- TYPICAL bonus: the tile of row m holding u Z, from the per-tile partials
  const LmPart* pp = parts + (base + m) * nblk;
  const float M = row_max[base + m];
  const double Z = row_sum[base + m];
  const double target = (double)uniforms[base] * Z;
  if (c == 0) {
    s_tile = -1;
    s_pre = 0.0;
  }
  __syncthreads();
  if (nblk <= SPEC_MAX_NODES * kScanPer) {
    // thread c owns tiles 8c .. 8c + 7 (all requested at once): its weight, a block scan of the
    // threads' totals, and the owner of the crossing scans its own tiles
    double wj[kScanPer];
    double mine = 0.0;
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      const int j = c * kScanPer + k;
      const LmPart q = pp[j < nblk ? j : 0];
      wj[k] = (j < nblk && q.m != -INFINITY) ? q.S * exp((double)q.m - (double)M) : 0.0;
      mine += wj[k];
    }
    double incl = mine;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const double y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == kWave - 1) s_wsum[wv] = incl;
    __syncthreads();
    double run = incl - mine;
    for (int q = 0; q < wv; ++q) run += s_wsum[q];
    if (mine > 0.0 && run <= target && target < run + mine) {
#pragma unroll
      for (int k = 0; k < kScanPer; ++k) {
        if (wj[k] > 0.0 && run <= target && target < run + wj[k] && s_tile < 0) {
          s_tile = c * kScanPer + k;         // one thread: the ranges are disjoint
          s_pre = run;
        }
        run += wj[k];
      }
    }
    __syncthreads();
  } else {
  // more tiles: chunks of 256, each thread's weight, a block scan, the first crossing
  double carry = 0.0;
  for (int j0 = 0; j0 < nblk; j0 += SPEC_MAX_NODES) {
    const int j = j0 + c;
    double wj = 0.0;
    if (j < nblk) {
      const LmPart q = pp[j];
      if (q.m != -INFINITY) wj = q.S * exp((double)q.m - (double)M);
    }
    double incl = wj;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const double y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == kWave - 1) s_wsum[wv] = incl;
    __syncthreads();
    double off = carry;
    for (int q = 0; q < wv; ++q) off += s_wsum[q];
    const double before = off + incl - wj, after = off + incl;
    if (j < nblk && wj > 0.0 && before <= target && target < after) {
      s_tile = j;                            // one thread at most: the ranges are disjoint
      s_pre = before;
    }
    double tot = 0.0;
    for (int q = 0; q < SPEC_MAX_NODES / kWave; ++q) tot += s_wsum[q];
    carry += tot;
    __syncthreads();
    if (s_tile >= 0) break;                  // uniform: read after the barrier
  }
  }
  int tile = s_tile;
  if (tile < 0) {                            // u Z at or past the rounded total: the last tile
    if (c == 0) {                            // with weight
      int last = nblk - 1;
      while (last > 0 && !(pp[last].m != -INFINITY && pp[last].S > 0.0)) --last;
      s_tile = last;
      s_pre = -1.0;                          // take its last token
    }
    __syncthreads();
    tile = s_tile;
  }
  // the tile's 64 logits of row m: four threads per token, Dm / 4 products each
  {
    const int v_local = c >> 2, part = c & 3;
    const int v = tile * kLRows + v_local;
    float acc32 = 0.f;
    if (v < V) {
      const __bf16* wr = W + (size_t)v * Dm + part * 8;
      const __bf16* hr = X + (base + m) * (size_t)Dm + part * 8;
      const int nk = Dm / 32;
      for (int k0 = 0; k0 < nk; k0 += 8) {   // eight 16-byte pairs requested at once
        bf16x8 a8[8], h8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int k = (k0 + i < nk ? k0 + i : 0) * 32;
          a8[i] = ld8(wr + k);
          h8[i] = ld8(hr + k);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (k0 + i < nk)
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) acc32 = fmaf((float)a8[i][e2], (float)h8[i][e2], acc32);
      }
    }
    acc32 += __shfl_xor(acc32, 1);
    acc32 += __shfl_xor(acc32, 2);
    if (part == 0) s_logit[v_local] = v < V ? acc32 : -INFINITY;
  }
  __syncthreads();
  if (c == 0) {
    const double mj = (double)pp[tile].m;
    const double sc = exp(mj - (double)M);
    double tw = 0.0;
    for (int i = 0; i < kLRows; ++i)
      if (s_logit[i] != -INFINITY) tw += (double)expf(s_logit[i] - (float)mj) * sc;
    const double stored = pp[tile].S * sc;
    // the remainder inside the tile, scaled to the recomputed total
    double r = s_pre < 0.0 ? tw : (target - s_pre) * (stored > 0.0 ? tw / stored : 1.0);
    int tok = -1;
    double run = 0.0;
    for (int i = 0; i < kLRows; ++i) {
      if (s_logit[i] == -INFINITY) continue;
      const double wi = (double)expf(s_logit[i] - (float)mj) * sc;
      run += wi;
      if (wi > 0.0) tok = tile * kLRows + i;  // the last token with weight, if r is never passed
      if (run > r && wi > 0.0) break;
    }
    bonus[b] = tok;
  }
}

// Greedy verification from the fused statistics: node c (parent p, token x) is accepted iff
// x == row_argmax[p]; a node survives iff every node on its path below the root was accepted;
// m = the deepest survivor (lowest index on ties); bonus = row_argmax[m].  One workgroup per
// sequence, one thread per node; validation as spec_verify's (node count, root, parent, depth,
// token), smallest error word first.
__global__ __launch_bounds__(SPEC_MAX_NODES) void verify_greedy_stats_kernel(
    const int32_t* __restrict__ row_argmax, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ parents, const int32_t* __restrict__ n_nodes, int N, int V,
    int max_depth, int32_t* __restrict__ accept_len, int32_t* __restrict__ path,
    int32_t* __restrict__ bonus, uint8_t* __restrict__ node_accept, int32_t* __restrict__ err) {
  __shared__ int s_par[SPEC_MAX_NODES];
  __shared__ unsigned char s_acc[SPEC_MAX_NODES];
  __shared__ int s_err, s_best;
  const int b = blockIdx.x, c = threadIdx.x;
  const size_t base = (size_t)b * N;
  const int n_raw = n_nodes ? n_nodes[b] : N;
  const bool bad_n = n_raw < 0 || n_raw > N;
  const int n = bad_n ? 0 : n_raw;
  if (c == 0) {
    s_err = INT_MAX;
    s_best = -1;
  }
  if (c < N) s_par[c] = parents[base + c];
  __syncthreads();
  int depth = 0;
  bool acc = false;
  if (c < n) {
    const int p = s_par[c];
    int code = 0;
    if (c == 0) {
      if (p != -1) code = SPEC_ERR_ROOT;
      acc = true;
    } else if (p < 0 || p >= c) {
      code = SPEC_ERR_PARENT;
    } else {
      int j = c;
      while (j > 0 && s_par[j] >= 0 && s_par[j] < j) {   // parents strictly decrease: ends
        j = s_par[j];
        ++depth;
      }
      const int x = tokens[base + c];
      if (depth > max_depth) code = SPEC_ERR_DEPTH;
      else if (x < 0 || x >= V) code = SPEC_ERR_TOKEN;
      else acc = x == row_argmax[base + p];
    }
    if (code) atomicMin(&s_err, err_word(c, code));
    s_acc[c] = acc ? 1 : 0;
  }
  __syncthreads();
  const int e = bad_n ? err_word(0, SPEC_ERR_NNODES) : (s_err == INT_MAX ? 0 : s_err);
  if (e == 0 && c < n) {
    bool live = true;
    for (int j = c; j > 0; j = s_par[j]) live = live && s_acc[j];
    if (live) atomicMax(&s_best, (depth << 9) | (511 - c));
  }
  __syncthreads();
  if (c < N && node_accept) node_accept[base + c] = (e == 0 && c < n) ? s_acc[c] : 0;
  if (c == 0) {
    int32_t* pr = path + (size_t)b * (max_depth + 1);
    for (int k = 0; k <= max_depth; ++k) pr[k] = -1;
    int len = 0, tok = -1;
    if (e == 0 && n > 0) {
      const int m = 511 - (s_best & 511);
      len = s_best >> 9;
      for (int j = m, k = len; k >= 0; --k, j = s_par[j]) pr[k] = j;
      tok = row_argmax[base + m];
    }
    accept_len[b] = len;
    bonus[b] = tok;
    err[b] = e;
  }
}

}  // namespace
}  // namespace spectree

using namespace spectree;

namespace {
struct LmLayout {
  int nblk;
  size_t parts, gath, xperm, total;
};
LmLayout lm_layout(int B, int N, int V, int Dm) {
  LmLayout L{};
  L.nblk = (V + kLRows - 1) / kLRows;
  const size_t M = (size_t)B * N;
  L.parts = 0;
  L.gath = align_up(M * L.nblk * sizeof(LmPart), 256);
  L.xperm = L.gath + align_up(M * sizeof(float), 256);
  L.total = L.xperm + align_up((size_t)xp_stride((int)M) * Dm * 2, 256);
  return L;
}
}  // namespace

namespace {
constexpr int kLMaxVocab = 1 << 24;

// Sizes the statistics pass supports (shared by the workspace queries and the calls).
spec_status check_lm_shape(int B, int N, int Dm, int V) {
  if (B < 1 || N < 1 || Dm < 1 || V < 1) return SPEC_EINVAL;
  if (N > SPEC_MAX_NODES || (size_t)B * N > (size_t)kLMaxRows) return SPEC_EUNSUPPORTED;
  if (Dm % 128 != 0 || V > kLMaxVocab) return SPEC_EUNSUPPORTED;
  return SPEC_OK;
}
}  // namespace

extern "C" size_t spec_lm_head_stats_workspace(int B, int N, int Dm, int V) {
  if (check_lm_shape(B, N, Dm, V) != SPEC_OK) return 0;
  return lm_layout(B, N, V, Dm).total;
}

namespace {
spec_status check_lm(const void* hidden, const void* W, int B, int N, int Dm, int V) {
  const spec_status shape = check_lm_shape(B, N, Dm, V);
  if (shape != SPEC_OK) return shape;
  if (!hidden || !W) return SPEC_EINVAL;
  if ((reinterpret_cast<uintptr_t>(hidden) & 15) || (reinterpret_cast<uintptr_t>(W) & 15))
    return SPEC_EUNSUPPORTED;
  return SPEC_OK;
}

// permutation, tile kernel for the size, merge: the statistics into the given arrays
void launch_lm(const __bf16* X, const __bf16* Wb, const int32_t* parents, const int32_t* tokens,
               const int32_t* n_nodes, int B, int N, int Dm, int V, const LmLayout& L, char* w,
               float* row_max, int32_t* row_argmax, double* row_sum, double* row_ent, float* cand_logit,
               int32_t* err, float* rows, hipStream_t s) {
  const int M = B * N;
  LmPart* parts = reinterpret_cast<LmPart*>(w + L.parts);
  float* gath = reinterpret_cast<float*>(w + L.gath);
  __bf16* Xp = reinterpret_cast<__bf16*>(w + L.xperm);
  const int ncb = (M + kLMaxCols - 1) / kLMaxCols;
  const dim3 g1((unsigned)((L.nblk + 7) / 8 * 8 * ncb)), blk(kLThreads);
  const int nchunk = M * (Dm / 8);
  launch("lm_head_xperm", lmhead_xperm_kernel, dim3((unsigned)((nchunk + kLThreads - 1) / kLThreads)), blk, s, X,
         M, Dm, Xp);
  const char* nm = "lm_head_stats";
  const int nb = L.nblk;
  if (M > 2 * kLMaxCols) {
    const int ntile = (V + kG2Rows - 1) / kG2Rows, ncb2 = (M + kGT - 1) / kGT;
    const dim3 gg((unsigned)((ntile + 7) / 8 * 8 * ncb2));
    launch(nm, lmhead_stats_gemm_kernel, gg, blk, s, Wb, Xp, M, Dm, V, N, nb, ntile, ncb2, parents, tokens, parts, gath, rows);
  } else if (M > kLMaxCols) {
    const int ntile = (V + kWRows - 1) / kWRows;
    const dim3 gw((unsigned)((ntile + 7) / 8 * 8 * ncb));
    launch(nm, lmhead_stats_wide_kernel, gw, blk, s, Wb, Xp, M, Dm, V, N, nb, ntile, ncb, parents, tokens, parts, gath, rows);
  } else if (M <= 16) launch(nm, lmhead_stats_kernel<1>, g1, blk, s, Wb, Xp, M, Dm, V, N, nb, ncb, parents, tokens, parts, gath, rows);
  else if (M <= 32) launch(nm, lmhead_stats_kernel<2>, g1, blk, s, Wb, Xp, M, Dm, V, N, nb, ncb, parents, tokens, parts, gath, rows);
  else if (M <= 48) launch(nm, lmhead_stats_kernel<3>, g1, blk, s, Wb, Xp, M, Dm, V, N, nb, ncb, parents, tokens, parts, gath, rows);
  else launch(nm, lmhead_stats_kernel<4>, g1, blk, s, Wb, Xp, M, Dm, V, N, nb, ncb, parents, tokens, parts, gath, rows);
  launch("lm_head_merge", lmhead_merge_kernel, dim3((unsigned)M), blk, s, parts, gath, L.nblk, N, V,
         parents, tokens, n_nodes, row_max, row_argmax, row_sum, row_ent, cand_logit, err);
}

// spec_verify_lm_head's own part of the workspace, after the LM head's: the statistics
struct VlLayout {
  size_t mx, am, sum, ent, cand, err, plan, rows, tsum, sub, total;
};
VlLayout vl_layout(const LmLayout& L, int B, int N, int V, int mode) {
  const bool reject = mode == SPEC_VERIFY_REJECT, walk = mode == SPEC_VERIFY_WALK;
  const size_t M = (size_t)B * N;
  VlLayout v{};
  v.mx = L.total;
  v.am = v.mx + align_up(M * sizeof(float), 256);
  v.sum = v.am + align_up(M * sizeof(int32_t), 256);
  v.ent = v.sum + align_up(M * sizeof(double), 256);
  v.cand = v.ent + align_up(M * sizeof(double), 256);
  v.err = v.cand + align_up(M * sizeof(float), 256);
  v.plan = v.err + align_up((size_t)B * sizeof(int32_t), 256);
  v.rows = v.plan + align_up((size_t)B * 3 * sizeof(int32_t), 256);
  // REJECT and WALK: every row's logits (REJECT's residual draw reads row m; WALK runs
  // spec_verify on them); REJECT: row m's tile sums; WALK: spec_verify's own workspace
  v.tsum = v.rows + (reject || walk ? align_up(M * V * sizeof(float), 256) : 0);
  v.sub = v.tsum + (reject ? align_up((size_t)B * L.nblk * sizeof(double2), 256) : 0);
  v.total = v.sub + (walk ? align_up(spec_verify_workspace(B, N, V), 256) : 0);
  return v;
}
}  // namespace

extern "C" spec_status spec_lm_head_stats(const void* hidden, const void* W, const int32_t* parents,
                                          const int32_t* tokens, const int32_t* n_nodes, int B, int N,
                                          int Dm, int V, float* row_max, int32_t* row_argmax,
                                          double* row_sum, double* row_ent, float* cand_logit,
                                          int32_t* err, void* workspace, size_t ws_bytes, void* stream) {
  const spec_status st = check_lm(hidden, W, B, N, Dm, V);
  if (st != SPEC_OK) return st;
  if (!parents || !tokens || !row_max || !row_argmax || !row_sum || !row_ent || !cand_logit || !err)
    return SPEC_EINVAL;
  const LmLayout L = lm_layout(B, N, V, Dm);
  if (!workspace || ws_bytes < L.total) return SPEC_EWORKSPACE;
  launch_lm(static_cast<const __bf16*>(hidden), static_cast<const __bf16*>(W), parents, tokens, n_nodes, B, N, Dm,
            V, L, static_cast<char*>(workspace), row_max, row_argmax, row_sum, row_ent, cand_logit, err,
            nullptr, static_cast<hipStream_t>(stream));
  return launch_status();
}

extern "C" size_t spec_verify_lm_head_workspace(int B, int N, int Dm, int V, int mode) {
  if (check_lm_shape(B, N, Dm, V) != SPEC_OK) return 0;
  return vl_layout(lm_layout(B, N, V, Dm), B, N, V, mode).total;
}

extern "C" spec_status spec_verify_lm_head(const void* hidden, const void* W, const int32_t* tokens,
                                           const int32_t* parents, const int32_t* n_nodes,
                                           const float* uniforms, const float* draft_probs,
                                           const int32_t* draft_row, const int32_t* t2d, int B, int N,
                                           int Dm, int V, int R, int Vd, int max_depth, int mode,
                                           float eps, float delta, int32_t* accept_len, int32_t* path,
                                           int32_t* bonus_token, uint8_t* node_accept, int32_t* err,
                                           void* workspace, size_t ws_bytes, void* stream) {
  const spec_status st = check_lm(hidden, W, B, N, Dm, V);
  if (st != SPEC_OK) return st;
  if (!tokens || !parents || !uniforms || !accept_len || !path || !bonus_token || !err || max_depth < 0)
    return SPEC_EINVAL;
  if (mode != SPEC_VERIFY_GREEDY && mode != SPEC_VERIFY_TYPICAL && mode != SPEC_VERIFY_REJECT &&
      mode != SPEC_VERIFY_WALK)
    return SPEC_EUNSUPPORTED;
  if (mode == SPEC_VERIFY_TYPICAL && (!(eps == eps) || !(delta == delta))) return SPEC_EINVAL;
  if (mode == SPEC_VERIFY_REJECT || mode == SPEC_VERIFY_WALK) {
    if (!draft_probs || !draft_row || R < 1 || Vd < 1) return SPEC_EINVAL;
    if (!t2d && Vd != V) return SPEC_EINVAL;
  }
  const LmLayout L = lm_layout(B, N, V, Dm);
  const VlLayout VL = vl_layout(L, B, N, V, mode);
  if (!workspace || ws_bytes < VL.total) return SPEC_EWORKSPACE;
  char* w = static_cast<char*>(workspace);
  float* mx = reinterpret_cast<float*>(w + VL.mx);
  int32_t* am = reinterpret_cast<int32_t*>(w + VL.am);
  double* sum = reinterpret_cast<double*>(w + VL.sum);
  double* ent = reinterpret_cast<double*>(w + VL.ent);
  float* cand = reinterpret_cast<float*>(w + VL.cand);
  int32_t* lerr = reinterpret_cast<int32_t*>(w + VL.err);
  LmDraft dr{};
  dr.draft = draft_probs; dr.draft_row = draft_row; dr.t2d = t2d; dr.R = R; dr.Vd = Vd;
  dr.plan = reinterpret_cast<int32_t*>(w + VL.plan);
  const bool keep_rows = mode == SPEC_VERIFY_REJECT || mode == SPEC_VERIFY_WALK;
  float* rows = keep_rows ? reinterpret_cast<float*>(w + VL.rows) : nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const __bf16* X = static_cast<const __bf16*>(hidden);
  const __bf16* Wb = static_cast<const __bf16*>(W);
  launch_lm(X, Wb, parents, tokens, n_nodes, B, N, Dm, V, L, w, mx, am, sum, ent, cand, lerr, rows, s);
  if (mode == SPEC_VERIFY_WALK) {
    // the sibling-residual walk visits every sibling's residual over whole rows: it runs as
    // spec_verify's WALK on the logits rows the statistics pass just stored
    if (launch_status() != SPEC_OK) return SPEC_EHIP;
    return spec_verify(rows, draft_probs, draft_row, t2d, tokens, parents, n_nodes, uniforms, B, N, V, R, Vd,
                       max_depth, SPEC_VERIFY_WALK, eps, delta, accept_len, path, bonus_token, node_accept, err,
                       w + VL.sub, VL.total - VL.sub, stream);
  }
  launch("verify_lm", verify_lm_kernel, dim3(B), dim3(SPEC_MAX_NODES), s, (const float*)mx, (const int32_t*)am,
         (const double*)sum, (const double*)ent, (const float*)cand,
         (const LmPart*)reinterpret_cast<LmPart*>(w + L.parts), L.nblk, X, Wb, Dm, tokens, parents, n_nodes,
         uniforms, N, V, max_depth, (int)mode, eps, delta, dr, accept_len, path, bonus_token, node_accept, err);
  if (mode == SPEC_VERIFY_REJECT) {
    double2* tsum = reinterpret_cast<double2*>(w + VL.tsum);
    launch("verify_lm_tilesum", lm_tilesum_kernel, dim3((unsigned)((L.nblk + 3) / 4), (unsigned)B), dim3(kLThreads),
           s, (const float*)rows, N, V, L.nblk, (const float*)mx, (const double*)sum, dr, tsum);
    launch("verify_lm_residual", lm_residual_kernel, dim3(B), dim3(kLThreads), s, (const float*)rows,
           (const double2*)tsum, L.nblk, (const float*)mx, (const double*)sum, uniforms, N, V, dr, bonus_token);
  }
  return launch_status();
}

extern "C" spec_status spec_verify_greedy_stats(const int32_t* row_argmax, const int32_t* tokens,
                                                const int32_t* parents, const int32_t* n_nodes, int B,
                                                int N, int V, int max_depth, int32_t* accept_len,
                                                int32_t* path, int32_t* bonus_token,
                                                uint8_t* node_accept, int32_t* err, void* stream) {
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES || V < 1 || max_depth < 0) return SPEC_EINVAL;
  if (!row_argmax || !tokens || !parents || !accept_len || !path || !bonus_token || !err) return SPEC_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch("verify_greedy_stats", verify_greedy_stats_kernel, dim3(B), dim3(SPEC_MAX_NODES), s, row_argmax, tokens,
         parents, n_nodes, N, V, max_depth, accept_len, path, bonus_token, node_accept, err);
  return launch_status();
}
