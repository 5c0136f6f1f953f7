// Medusa heads: z_j = h + SiLU(W_res[j] h), logits_j = W_lm z_j (shared LM head),
// D_j = softmax(logits_j), per-head top-k.
//
// "多トークン予測（Medusa・EAGLE）", section "Medusa：本体に複数の予測ヘッドを足す" (light heads on
// the same final hidden state, all in one pass); "EAGLE-3とMedusaで実装するSpeculative Decoding
// 実践ガイド", section "アーキテクチャ：複数ヘッドによる並列トークン予測" (one feed-forward layer
// plus a residual per head); "Medusa（マルチヘッド投機的デコーディング）", sections
// "Medusaの基本アーキテクチャ" and "ツリー構造の候補構築" (the heads' top candidates build the
// tree).
//
// Both products have a handful of columns (the batch, or batch x heads) against megabytes of
// weights, so they are weight-streaming: each weight element is read from HBM once.  They run
// on v_mfma_f32_16x16x32_bf16 with the weight rows as the M dimension (A operand, 16-byte loads
// straight from HBM) and the few activation columns as N (B operand, L2-resident).  The K
// dimension is split over the four waves of a workgroup and the partial tiles are summed in
// LDS, so a workgroup keeps four independent load streams in flight.
//
// z stays fp32 (no rounding back to bf16 before the LM head).  The LM head consumes it as an
// exact three-term bf16 split z = hi + mid + lo; each W_lm fragment is multiplied with the
// three parts into one fp32 accumulator, which costs MFMA issue slots but no extra HBM bytes.
#include <climits>
#include <cstdlib>

#include "common.h"

namespace spectree {
namespace {

constexpr int kThreads = 256;
constexpr int kKWaves = 4;       // K slices per workgroup
constexpr int kMaxCols = 64;     // B * H limit of the LM head

__device__ __forceinline__ bf16x8 load8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// grid: H * Dm / (16 RB) workgroups; workgroup = RB blocks of 16 output rows of one head, K
// split over 4 waves (each wave all RB blocks of its K slice, so one h fragment serves RB
// products and h is re-read from L2 once per workgroup).
// Layout of each part of the z split in the workspace: [Dm / 8][NC][8], i.e. element (col, k)
// at ((k / 8) * NC + col) * 8 + k % 8.  The LM head's B fragment (lane l: column l % 16,
// k = 8 (l / 16) + [0, 8)) is then four 256-byte runs with consecutive lanes on consecutive 16
// bytes, instead of 16 columns x 64 bytes scattered over the part (measured 18 us of the LM
// head's 84 on the Medusa workload went to those fragment loads).
__device__ __forceinline__ size_t zsplit_index(int NC, int Dm, int col, int k) {
  (void)Dm;
  return ((size_t)(k >> 3) * NC + col) * 8 + (k & 7);
}

template <int RB>
__global__ __launch_bounds__(kThreads) void resblock_kernel(const __bf16* __restrict__ h,
                                                            const __bf16* __restrict__ W, int B, int H,
                                                            int Dm, __bf16* __restrict__ zsplit) {
  __shared__ f32x4 red[kKWaves][RB][kWave];
  const int blocks_per_head = Dm / (16 * RB);
  const int j = blockIdx.x / blocks_per_head;
  const int row0 = (blockIdx.x - j * blocks_per_head) * 16 * RB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int kslice = Dm / kKWaves;
  const int kbeg = wave * kslice;
  const __bf16* arow = W + ((size_t)j * Dm + row0 + l16) * Dm + kbeg + 8 * lg;
  const bool col_ok = l16 < B;
  const __bf16* bcol = h + (size_t)(col_ok ? l16 : 0) * Dm + kbeg + 8 * lg;
  // Loads are branch-free (a column past B reads column 0 and is never stored) and the next
  // steps' fragments are requested before this step's products, so loads stay in flight.
  // Buffers of four steps in a ring of NB, one buffer requested ahead of the products; the
  // ring index is static inside the unrolled body (a register copy would wait for the loads
  // it copies).  Step indices are clamped to the slice, so every load stays inside it; steps
  // past the slice are loaded (L2 hits) but not multiplied.
  constexpr int U = 4, NB = 2;
  f32x4 acc[RB];
#pragma unroll
  for (int r = 0; r < RB; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int steps = kslice / 32;             // >= 1 (Dm % 128 == 0, 4 K slices)
  bf16x8 a[NB][U][RB], bv[NB][U];
  auto fetch = [&](bf16x8 (&ar)[U][RB], bf16x8 (&br)[U], int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int st = min(s0 + u, steps - 1);
#pragma unroll
      for (int r = 0; r < RB; ++r) ar[u][r] = load8(arow + (size_t)r * 16 * Dm + st * 32);
      br[u] = load8(bcol + st * 32);
    }
  };
  auto products = [&](const bf16x8 (&ar)[U][RB], const bf16x8 (&br)[U], int valid) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (u < valid) {
#pragma unroll
        for (int r = 0; r < RB; ++r) acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar[u][r], br[u], acc[r], 0, 0, 0);
      }
  };
#pragma unroll
  for (int q = 0; q < NB - 1; ++q) fetch(a[q], bv[q], q * U);
  for (int s = 0; s < steps; s += NB * U) {
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      fetch(a[(q + NB - 1) % NB], bv[(q + NB - 1) % NB], s + (q + NB - 1) * U);
      __builtin_amdgcn_sched_barrier(0);    // keep the prefetch ahead of the products
      products(a[q], bv[q], steps - (s + q * U));
    }
  }
#pragma unroll
  for (int r = 0; r < RB; ++r) red[wave][r][lane] = acc[r];
  __syncthreads();
  if (!col_ok) return;
  const int b = l16;
  const int NC = B * H;
  // Every wave finishes a share of the row blocks: z = h + SiLU(W h), as an exact bf16 split.
  for (int r = wave; r < RB; r += kKWaves) {
    const f32x4 sum = red[0][r][lane] + red[1][r][lane] + red[2][r][lane] + red[3][r][lane];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = row0 + r * 16 + 4 * lg + e;   // output feature
      const float av = sum[e];
      const float z = (float)h[(size_t)b * Dm + row] + av / (1.f + expf(-av));
      const __bf16 hi = (__bf16)z;
      const float r1 = z - (float)hi;
      const __bf16 mid = (__bf16)r1;
      const __bf16 lo = (__bf16)(r1 - (float)mid);
      const size_t col = (size_t)b * H + j;
      const size_t at = zsplit_index(NC, Dm, col, row);
      zsplit[at] = hi;
      zsplit[(size_t)NC * Dm + at] = mid;
      zsplit[2 * (size_t)NC * Dm + at] = lo;
    }
  }
}

// grid: ceil(V / (16 RB)) workgroups; workgroup = 16 RB rows of W_lm (RB blocks of 16 per wave),
// K split over the 4 waves.  logits[col, v], col = b * H + j.
template <int CBN, int RB>
__global__ __launch_bounds__(kThreads) void lm_head_kernel(const __bf16* __restrict__ W_lm,
                                                           const __bf16* __restrict__ zsplit, int NC, int Dm,
                                                           int V, float* __restrict__ logits) {
  __shared__ f32x4 red[kKWaves][RB * CBN][kWave];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int row0 = blockIdx.x * 16 * RB;
  const int kslice = Dm / kKWaves;
  const int kbeg = wave * kslice;
  const __bf16* arow[RB];
  bool row_ok[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = row0 + rb * 16 + l16;
    row_ok[rb] = r < V;
    arow[rb] = W_lm + (size_t)(row_ok[rb] ? r : 0) * Dm + kbeg + 8 * lg;
  }
  const __bf16* bptr[3][CBN];
  bool col_ok[CBN];
#pragma unroll
  for (int cb = 0; cb < CBN; ++cb) {
    const int col = cb * 16 + l16;
    col_ok[cb] = col < NC;
#pragma unroll
    for (int sp = 0; sp < 3; ++sp)
      bptr[sp][cb] = zsplit + (size_t)sp * NC * Dm + zsplit_index(NC, Dm, col_ok[cb] ? col : 0, kbeg + 8 * lg);
  }
  f32x4 acc[RB][CBN];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CBN; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Loads are branch-free (rows past V and columns past NC read row / column 0 and are never
  // stored).  All fragments of the next step (W_lm from HBM, z from L2) are requested before
  // this step's products: the memory counter drains in issue order, so a load issued after
  // the prefetch could only be waited for together with it.
  // Two K steps per fetch, so both 64-byte halves of each 128-byte W_lm line are requested
  // back to back (one step per fetch left the second half to a later request that often
  // missed L2: 363 MB read per launch for 262 MB of weights, now 299 MB); two slots, one pair
  // of steps in flight while the other's products run.  Step indices are clamped, so the loads
  // past the last step re-read it (L2 hits) and stay inside the slice.
  const int steps = kslice / 32;
  struct Frags {
    bf16x8 a[RB][2];
    bf16x8 b[3][CBN][2];
  };
  auto fetch = [&](Frags& g, int s) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int h = 0; h < 2; ++h) g.a[rb][h] = load8(arow[rb] + min(s + h, steps - 1) * 32);
#pragma unroll
    for (int sp = 0; sp < 3; ++sp)
#pragma unroll
      for (int cb = 0; cb < CBN; ++cb)
#pragma unroll
        for (int h = 0; h < 2; ++h) g.b[sp][cb][h] = load8(bptr[sp][cb] + (size_t)min(s + h, steps - 1) * 32 * NC);
  };
  auto products = [&](const Frags& g, int s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (s + h >= steps) break;
#pragma unroll
      for (int cb = 0; cb < CBN; ++cb)
#pragma unroll
        for (int sp = 0; sp < 3; ++sp)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g.a[rb][h], g.b[sp][cb][h], acc[rb][cb], 0, 0, 0);
    }
  };
  Frags g[2];
  fetch(g[0], 0);
  for (int s = 0; s < steps; s += 4) {
    fetch(g[1], s + 2);
    __builtin_amdgcn_sched_barrier(0);    // keep the prefetch ahead of the products
    products(g[0], s);
    fetch(g[0], s + 4);
    __builtin_amdgcn_sched_barrier(0);
    products(g[1], s + 2);
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CBN; ++cb) red[wave][rb * CBN + cb][lane] = acc[rb][cb];
  __syncthreads();
  // Every wave finishes a quarter of the tiles.
  for (int t = wave; t < RB * CBN; t += kKWaves) {
    const f32x4 sum = red[0][t][lane] + red[1][t][lane] + red[2][t][lane] + red[3][t][lane];
    const int rb = t / CBN, cb = t % CBN;
    const int col = cb * 16 + l16;
    if (col >= NC) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = row0 + rb * 16 + 4 * lg + e;
      if (r < V) logits[(size_t)col * V + r] = sum[e];
    }
  }
}

// ---------------------------------------------------------------- softmax and top-k
//
// One workgroup per column (b, j).  Top-k in (value desc, id asc) order without k selection
// rounds: the k-th largest of the 256 per-thread maxima is a lower bound tau of the row's k-th
// largest value (the k threads ranked above it each hold an element at least that large), so
// every top-k element is >= tau.  Those candidates (typically a few more than k) are gathered
// in LDS and each one's rank among them, which equals its rank in the row, is counted
// directly.  More than kCand candidates (heavy ties) falls back to k selection rounds.
// Weights are exp2(x log2 e - m log2 e) with the hardware exp2; the shared rounding of
// m log2 e cancels in the normalised probabilities.

constexpr int kCand = 512;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float weight(float x, float mL) {
  return __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -mL));
}

struct __attribute__((aligned(16))) TopkShared {   // tmax is read as float4
  float tmax[kThreads];
  float cv[kCand];
  int ci[kCand];
  float red[kThreads / kWave];
  int redi[kThreads / kWave];
  float tau, m;
  int n;
};

// Row max and tau from the per-thread maxima (written to sh.tmax by the caller).
__device__ __forceinline__ void row_max_and_tau(TopkShared& sh, float tm, int k) {
  const int t = threadIdx.x;
  if (t == 0) sh.n = 0;
  __syncthreads();
  int rank = 0;
  float m = -INFINITY;
  const float4* tm4 = reinterpret_cast<const float4*>(sh.tmax);
#pragma unroll 4
  for (int j4 = 0; j4 < kThreads / 4; ++j4) {
    const float4 o = tm4[j4];
    const int j = 4 * j4;
    rank += (o.x > tm || (o.x == tm && j < t)) + (o.y > tm || (o.y == tm && j + 1 < t)) +
            (o.z > tm || (o.z == tm && j + 2 < t)) + (o.w > tm || (o.w == tm && j + 3 < t));
    m = fmaxf(m, fmaxf(fmaxf(o.x, o.y), fmaxf(o.z, o.w)));
  }
  if (rank == k - 1) sh.tau = tm;     // the ranks are a permutation of 0..255 and k <= 64
  if (t == 0) sh.m = m;
  __syncthreads();
}

__device__ __forceinline__ void push_candidate(TopkShared& sh, float x, int v) {
  const int slot = atomicAdd(&sh.n, 1);
  if (slot < kCand) { sh.cv[slot] = x; sh.ci[slot] = v; }
}

__device__ __forceinline__ float block_sum_f(TopkShared& sh, float v) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh.red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < kThreads / kWave; ++q) s += sh.red[q];
  return s;
}

// Ranks of the gathered candidates; the k first go to the outputs.
__device__ __forceinline__ void rank_candidates(const TopkShared& sh, int nc, int k, float mL, float invS,
                                                int32_t* idx_out, float* prob_out) {
  for (int c = threadIdx.x; c < nc; c += kThreads) {
    const float cv = sh.cv[c];
    const int ci = sh.ci[c];
    int r = 0;
    for (int j = 0; j < nc; ++j) r += (sh.cv[j] > cv || (sh.cv[j] == cv && sh.ci[j] < ci)) ? 1 : 0;
    if (r < k) {
      idx_out[r] = ci;
      prob_out[r] = weight(cv, mL) * invS;
    }
  }
}

// k selection rounds over the row in memory, each the largest element below the previous pick
// in (value desc, id asc) order.  Branch-free selects; used when the candidates overflow.
__device__ void select_rounds(TopkShared& sh, const float* row, int V, int k, float mL, float invS,
                              int32_t* idx_out, float* prob_out) {
  float prev_v = INFINITY;
  int prev_i = -1;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int v = threadIdx.x; v < V; v += kThreads) {
      const float x = row[v];
      const bool below = (x < prev_v) | ((x == prev_v) & (v > prev_i));
      const bool better = (x > bv) | ((x == bv) & (v < bi));
      const bool take = below & better;
      bv = take ? x : bv;
      bi = take ? v : bi;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float v2 = __shfl_xor(bv, o);
      const int i2 = __shfl_xor(bi, o);
      const bool take = (v2 > bv) | ((v2 == bv) & (i2 < bi));
      bv = take ? v2 : bv;
      bi = take ? i2 : bi;
    }
    __syncthreads();
    if ((threadIdx.x & 63) == 0) { sh.red[threadIdx.x >> 6] = bv; sh.redi[threadIdx.x >> 6] = bi; }
    __syncthreads();
    bv = sh.red[0];
    bi = sh.redi[0];
#pragma unroll
    for (int q = 1; q < kThreads / kWave; ++q)
      if (sh.red[q] > bv || (sh.red[q] == bv && sh.redi[q] < bi)) { bv = sh.red[q]; bi = sh.redi[q]; }
    if (threadIdx.x == 0) {
      idx_out[r] = bi;
      prob_out[r] = weight(bv, mL) * invS;
    }
    prev_v = bv;
    prev_i = bi;
  }
}

// Rows of up to 256 * PER logits, held in registers: element (i / VEC) * 256 * VEC + t * VEC +
// i % VEC of the row in slot i of thread t (VEC = 4: 16-byte loads, V % 4 == 0).
template <int PER, int VEC>
__global__ __launch_bounds__(kThreads) void softmax_topk_kernel(const float* __restrict__ logits, int V, int k,
                                                                int32_t* __restrict__ topk_idx,
                                                                float* __restrict__ topk_prob,
                                                                float* __restrict__ probs) {
  __shared__ TopkShared sh;
  const int col = blockIdx.x;
  const int t = threadIdx.x;
  const float* row = logits + (size_t)col * V;
  auto index = [&](int i) { return ((i / VEC) * kThreads + t) * VEC + i % VEC; };
  float x[PER];
#pragma unroll
  for (int i = 0; i < PER; i += VEC) {
    const int v = index(i);
    const int at = v < V ? v : 0;
    if (VEC == 4) {
      const float4 q = *reinterpret_cast<const float4*>(row + at);
      x[i] = q.x;
      x[i + (VEC > 1 ? 1 : 0)] = q.y;
      x[i + (VEC > 2 ? 2 : 0)] = q.z;
      x[i + (VEC > 3 ? 3 : 0)] = q.w;
    } else {
      x[i] = row[at];
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) x[i] = index(i) < V ? x[i] : -INFINITY;
  float tm = -INFINITY;
#pragma unroll
  for (int i = 0; i < PER; ++i) tm = fmaxf(tm, x[i]);
  sh.tmax[t] = tm;
  row_max_and_tau(sh, tm, k);
  const float tau = sh.tau;
  const float mL = sh.m * kLog2e;
  // candidates, then the weights (x is overwritten by its weight)
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (x[i] >= tau && index(i) < V) push_candidate(sh, x[i], index(i));
    x[i] = weight(x[i], mL);                     // 0 past the row
    sum += x[i];
  }
  const float invS = 1.f / block_sum_f(sh, sum);  // barriers inside: the candidates are in
  const int nc = sh.n;
  int32_t* io = topk_idx + (size_t)col * k;
  float* po = topk_prob + (size_t)col * k;
  if (nc <= kCand) rank_candidates(sh, nc, k, mL, invS, io, po);
  else select_rounds(sh, row, V, k, mL, invS, io, po);
  if (probs) {
    float* pr = probs + (size_t)col * V;
#pragma unroll
    for (int i = 0; i < PER; i += VEC) {
      const int v = index(i);
      if (v < V) {
        if (VEC == 4) {
          *reinterpret_cast<float4*>(pr + v) =
              make_float4(x[i] * invS, x[i + (VEC > 1 ? 1 : 0)] * invS, x[i + (VEC > 2 ? 2 : 0)] * invS,
                          x[i + (VEC > 3 ? 3 : 0)] * invS);
        } else {
          pr[v] = x[i] * invS;
        }
      }
    }
  }
}

// Larger vocabularies: the same steps with the row re-read (from L2) in each pass.
__global__ __launch_bounds__(kThreads) void softmax_topk_big_kernel(const float* __restrict__ logits, int V,
                                                                    int k, int32_t* __restrict__ topk_idx,
                                                                    float* __restrict__ topk_prob,
                                                                    float* __restrict__ probs) {
  __shared__ TopkShared sh;
  const int col = blockIdx.x;
  const int t = threadIdx.x;
  const float* row = logits + (size_t)col * V;
  float tm = -INFINITY;
  for (int v = t; v < V; v += kThreads) tm = fmaxf(tm, row[v]);
  sh.tmax[t] = tm;
  row_max_and_tau(sh, tm, k);
  const float tau = sh.tau;
  const float mL = sh.m * kLog2e;
  float sum = 0.f;
  for (int v = t; v < V; v += kThreads) {
    const float x = row[v];
    if (x >= tau) push_candidate(sh, x, v);
    sum += weight(x, mL);
  }
  const float invS = 1.f / block_sum_f(sh, sum);
  const int nc = sh.n;
  int32_t* io = topk_idx + (size_t)col * k;
  float* po = topk_prob + (size_t)col * k;
  if (nc <= kCand) rank_candidates(sh, nc, k, mL, invS, io, po);
  else select_rounds(sh, row, V, k, mL, invS, io, po);
  if (probs)
    for (int v = t; v < V; v += kThreads) probs[(size_t)col * V + v] = weight(row[v], mL) * invS;
}

template <int RB>
void launch_lm_head(int cbn, const char* nm, dim3 grid, dim3 blk, hipStream_t s, const __bf16* wl, const __bf16* zs,
                    int NC, int Dm, int V, float* logits) {
  if (cbn == 1) launch(nm, lm_head_kernel<1, RB>, grid, blk, s, wl, zs, NC, Dm, V, logits);
  else if (cbn == 2) launch(nm, lm_head_kernel<2, RB>, grid, blk, s, wl, zs, NC, Dm, V, logits);
  else if (cbn == 3) launch(nm, lm_head_kernel<3, RB>, grid, blk, s, wl, zs, NC, Dm, V, logits);
  else launch(nm, lm_head_kernel<4, RB>, grid, blk, s, wl, zs, NC, Dm, V, logits);
}

struct HeadsLayout {
  size_t zsplit, logits, total;
};

HeadsLayout heads_layout(int B, int H, int Dm, int V) {
  HeadsLayout L{};
  const size_t NC = (size_t)B * H;
  size_t off = 0;
  L.zsplit = off; off += align_up(3 * NC * Dm * sizeof(__bf16), 256);
  L.logits = off; off += align_up(NC * V * sizeof(float), 256);
  L.total = off;
  return L;
}

}  // namespace
}  // namespace spectree

using namespace spectree;

extern "C" size_t spec_medusa_heads_workspace(int B, int H, int Dm, int V, int k) {
  if (B < 1 || H < 1 || Dm < 1 || V < 1 || k < 1) return 0;
  if (B > 16 || H > kMaxCols || B * H > kMaxCols || Dm % 128 != 0 || k > 64 || k > V) return 0;
  return heads_layout(B, H, Dm, V).total;
}

extern "C" spec_status spec_medusa_heads(const void* h, const void* W_res, const void* W_lm, int B, int H,
                                         int Dm, int V, int k, int32_t* topk_idx, float* topk_prob,
                                         float* draft_probs, void* workspace, size_t ws_bytes,
                                         void* stream) {
  if (B < 1 || H < 1 || Dm < 1 || V < 1 || k < 1) return SPEC_EINVAL;
  if (!h || !W_res || !W_lm || !topk_idx || !topk_prob) return SPEC_EINVAL;
  if (B > 16 || H > kMaxCols || B * H > kMaxCols || Dm % 128 != 0 || k > 64 || k > V) return SPEC_EUNSUPPORTED;
  const HeadsLayout L = heads_layout(B, H, Dm, V);
  if (!workspace || ws_bytes < L.total) return SPEC_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(workspace);
  __bf16* zsplit = reinterpret_cast<__bf16*>(w + L.zsplit);
  float* logits = reinterpret_cast<float*>(w + L.logits);
  const int NC = B * H;
  const dim3 blk(kThreads);
  // Row blocks per ResBlock workgroup: 2 (Dm % 32 == 0 always holds here), or as forced by the
  // tuning override res_rowblocks (1, 2 or 4).
  int rrb = tuning(kKnobResRowBlocks, 2);
  if (rrb != 1 && rrb != 2 && rrb != 4) rrb = 2;
  const __bf16* hb = static_cast<const __bf16*>(h);
  const __bf16* wr = static_cast<const __bf16*>(W_res);
  if (rrb == 4) launch("medusa_resblock", resblock_kernel<4>, dim3(H * (Dm / 64)), blk, s, hb, wr, B, H, Dm, zsplit);
  else if (rrb == 2) launch("medusa_resblock", resblock_kernel<2>, dim3(H * (Dm / 32)), blk, s, hb, wr, B, H, Dm, zsplit);
  else launch("medusa_resblock", resblock_kernel<1>, dim3(H * (Dm / 16)), blk, s, hb, wr, B, H, Dm, zsplit);
  // 16-row blocks of W_lm per wave (RB): 8 by default, 4 with the tuning override lm_rowblocks.
  const int RBv = tuning(kKnobLmRowBlocks, 8) == 4 ? 4 : 8;
  const dim3 grid_lm((V + 16 * RBv - 1) / (16 * RBv));
  const __bf16* wl = static_cast<const __bf16*>(W_lm);
  const __bf16* zs = zsplit;
  const char* nm = "medusa_lm_head";
  const int cbn = (NC + 15) / 16;
  if (RBv == 8) launch_lm_head<8>(cbn, nm, grid_lm, blk, s, wl, zs, NC, Dm, V, logits);
  else launch_lm_head<4>(cbn, nm, grid_lm, blk, s, wl, zs, NC, Dm, V, logits);
  const float* lg = logits;
  const char* nt = "medusa_softmax_topk";
  // logits rows start on 16-byte boundaries when V % 4 == 0 (the workspace is 256-byte aligned)
  if (V % 4 == 0) {
    if (V <= 16 * kThreads) launch(nt, softmax_topk_kernel<16, 4>, dim3(NC), blk, s, lg, V, k, topk_idx, topk_prob, draft_probs);
    else if (V <= 32 * kThreads) launch(nt, softmax_topk_kernel<32, 4>, dim3(NC), blk, s, lg, V, k, topk_idx, topk_prob, draft_probs);
    else if (V <= 64 * kThreads) launch(nt, softmax_topk_kernel<64, 4>, dim3(NC), blk, s, lg, V, k, topk_idx, topk_prob, draft_probs);
    else if (V <= 128 * kThreads) launch(nt, softmax_topk_kernel<128, 4>, dim3(NC), blk, s, lg, V, k, topk_idx, topk_prob, draft_probs);
    else launch(nt, softmax_topk_big_kernel, dim3(NC), blk, s, lg, V, k, topk_idx, topk_prob, draft_probs);
  } else {
    if (V <= 16 * kThreads) launch(nt, softmax_topk_kernel<16, 1>, dim3(NC), blk, s, lg, V, k, topk_idx, topk_prob, draft_probs);
    else if (V <= 64 * kThreads) launch(nt, softmax_topk_kernel<64, 1>, dim3(NC), blk, s, lg, V, k, topk_idx, topk_prob, draft_probs);
    else launch(nt, softmax_topk_big_kernel, dim3(NC), blk, s, lg, V, k, topk_idx, topk_prob, draft_probs);
  }
  return launch_status();
}
