// Verification: per-node acceptance, longest accepted path, bonus token.
//
// Rules: "EAGLE-3とMedusaで実装するSpeculative Decoding実践ガイド", section
// "棄却サンプリング：出力品質を保証する" (accept with probability min(1, T[x]/D[x]); on a reject
// draw from norm(relu(T - D)); drop every candidate after a reject); "Medusa（マルチヘッド
// 投機的デコーディング）", section "Medusa-1とMedusa-2の違い" (typical acceptance against an
// entropy-based threshold); "多トークン予測（Medusa・EAGLE）", section
// "ツリー検証：候補を「木」に束ねて1回で確かめる" (keep the path that passes the longest).
//
// Three kernels in stream order (four with the row listing of large problems); no kernel
// synchronises workgroups (the kernel boundaries order their results), and every global load is
// issued before it is needed.
//   rows    rows of nodes with children are split into chunks of 8K logits; each workgroup
//           streams one chunk once (float4 loads held in registers) into (max, lowest argmax,
//           sum exp(x - max) and, for typical acceptance, sum exp(x - max)(x - max)), fp32 exp
//           with fp64 sums.  Small problems: grid (seq, node, chunk), workgroups of leaf rows
//           leave after a 1 KB look at the parents.  Large ones: one workgroup first lists the
//           rows with children and workgroup i takes the i-th listed (row, chunk) item.
//   decide_bonus  grid (seq, chunk).  First the decision, derived by every workgroup of the
//           sequence (outputs written by chunk 0's): merge of the row chunks (1-4 lanes per
//           node), validation, node tests in fp64, survival = AND over the parent chain, the
//           deepest survivor (LDS max on depth, -index), the path, and the plan of the bonus
//           draw.  Then this chunk (2K or 4K logits) of the kept row m: chunk max / argmax, and
//           fp64 chunk sums of exp(x - max) and, for a residual draw, of relu(T - D) with T
//           normalised by the row statistics of the first kernel; small batches also keep
//           each token's weight.
//   select  per sequence: the chunk holding u * Z (scan of the chunk sums), then an in-order
//           fp64 scan inside it (of the kept weights, or recomputed ones) for the smallest
//           token whose running sum exceeds u * Z.  With kept weights and at most 64 chunks,
//           one wave does all of it with shuffles; otherwise a 256-thread workgroup.
#include <algorithm>
#include <cfloat>
#include <atomic>
#include <climits>
#include <mutex>

#include "common.h"

namespace spectree {
namespace {

constexpr int kThreads = 256;
// Logits per workgroup in the bonus pass: 2048 for batches up to kSmallChunkMaxB whose rows fit
// in one wave's worth of chunks (the decision is derived per workgroup, so more, shorter chunks
// pay off while they are few), 4096 otherwise.
constexpr int kChunkSmall = 2048;
constexpr int kChunkLarge = 4096;
constexpr int kSmallChunkMaxB = 8;
constexpr int kStoreWeightsMaxB = 8;          // batches that keep the bonus pass's weights when
                                              // the row has more chunks than a wave has lanes
constexpr int kPartsPerLane = 8;             // row-chunk partials per merging lane and batch

struct RowPart {      // one chunk of one logits row
  double S;           // sum exp(x - m)
  double A;           // sum exp(x - m) * (x - m)
  float m;            // chunk max
  int argmax;         // lowest index of the chunk max
  int nonfinite;
  int pad;
};

struct BonusPlan {
  int m;              // kept node
  int kind;           // 0 done, 1 argmax of row m, 2 draw from T_m, 3 draw from relu(T_m - D)
  int r;              // draft row of the residual
  float M;            // row max of m (residual draws)
  double S;           // sum exp(x - M) over row m (residual draws)
  double cs;          // the residual is relu(T_m - cs * D): 1, or after the walk's rejections
};

struct BonusPart {
  double S;           // sum exp(x - m) over the chunk (fp64; m = chunk max, or the row max for
                      // residual draws)
  double Q;           // chunk sum of relu(T - D) (residual draws)
  float m;
  int argmax;
  int nonfinite;
  int pad;
};

struct VerifyArgs {
  const float* logits;
  const float* draft;
  const int32_t* draft_row;
  const int32_t* t2d;
  const int32_t* tokens;
  const int32_t* parents;
  const int32_t* n_nodes;
  const float* uniforms;
  int B, N, V, R, Vd, max_depth, mode;
  float eps, delta;
  int32_t* accept_len;
  int32_t* path;
  int32_t* bonus;
  uint8_t* node_accept;
  int32_t* err;
  int CR;               // row-pass chunks per row
  int RC;               // logits per row-pass chunk
  int CS, C;            // bonus-pass chunk size (kChunkSmall or kChunkLarge) and chunks per row
  RowPart* rowparts;    // [B, N, CR]
  int32_t* row_list;    // [B * N]: b * N + p of each row with children (large problems)
  int32_t* row_count;   // [1]: entries of row_list
  BonusPlan* plans;     // [B]
  BonusPart* bparts;    // [B, C]
  double* weights;      // [B, C * CS]: the bonus pass's per-token weights (kinds 2 and 3),
                        // kept only for small batches (NULL otherwise)
  double* gsum;         // [B, C, CS / 64, 2]: per 64-token group, the sums of the bonus pass's
                        // weights (kind 2: exp(x - chunk max); kind 3: relu(T - cs D)) and, for
                        // kind 3, of exp(x - M); when the weights are not kept and one wave
                        // holds the chunks (NULL otherwise)
  double* wc;           // [B, N] walk: child c is tested against relu(T_p - wc D) / wf
  double* wf;           // [B, N]
  double* wend;         // [B, N] walk: residual scale after every child of node p is rejected
  int wk;               // walk: workgroups per node (1: one workgroup does the whole chain)
  int wspin;            // walk, wk > 1: polls of a node's counter before a workgroup stops waiting
  int32_t* wsync;       // [B, N] walk, wk > 1: arrivals per node (zeroed by the row pass)
  double* wpart;        // [B, N, wk, 2, 2] walk, wk > 1: each workgroup's partial sums of a pass
                        // (fp, z), in the slot of the pass's parity
};

// ------------------------------------------------------------------ reductions
//
// Every sum of exponentials is formed against a maximum that is known first, so no reduction
// step needs an exponential: block max (lowest index among equal maxima) in fp32, then fp32
// exp(x - max) summed in fp64.

constexpr int kWavesPB = kThreads / kWave;

// Max with the lowest index among equal maxima, and OR of the nonfinite flags, over the block;
// the result is returned to every thread.  NaN never compares greater, so it never wins (the
// nonfinite flag reports it).
__device__ void block_argmax(float& m, int& am, int& nf) {
  __shared__ float sm[kWavesPB];
  __shared__ int sam[kWavesPB], snf[kWavesPB];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o);
    const int am2 = __shfl_xor(am, o), nf2 = __shfl_xor(nf, o);
    if (m2 > m || (m2 == m && am2 < am)) { m = m2; am = am2; }
    nf |= nf2;
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { sm[w] = m; sam[w] = am; snf[w] = nf; }
  __syncthreads();
  m = sm[0]; am = sam[0]; nf = snf[0];
#pragma unroll
  for (int k = 1; k < kWavesPB; ++k) {
    if (sm[k] > m || (sm[k] == m && sam[k] < am)) { m = sm[k]; am = sam[k]; }
    nf |= snf[k];
  }
}

// Block sums of two fp64 values, returned to every thread.
__device__ void block_sum2(double& x, double& y) {
  __shared__ double sx[kWavesPB], sy[kWavesPB];
  x = wave_sum(x);
  y = wave_sum(y);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { sx[w] = x; sy[w] = y; }
  __syncthreads();
  x = sx[0]; y = sy[0];
#pragma unroll
  for (int k = 1; k < kWavesPB; ++k) { x += sx[k]; y += sy[k]; }
}

__device__ double block_sum(double v) {
  double dummy = 0.0;
  block_sum2(v, dummy);
  return v;
}

// Inclusive prefix sum in thread order (fp64); `total` receives the block sum.
__device__ double block_scan(double v, double& total) {
  __shared__ double sw[kWavesPB];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  __syncthreads();
  if (lane == kWave - 1) sw[w] = v;
  __syncthreads();
  double off = 0.0;
  total = 0.0;
#pragma unroll
  for (int k = 0; k < kWavesPB; ++k) {
    if (k < w) off += sw[k];
    total += sw[k];
  }
  return v + off;
}

// ------------------------------------------------------------------ chunk loads

// Loads one chunk of a row into registers: thread t holds elements lo + (k * 256 + t) * VEC + e.
// Branch-free (addresses past the chunk are clamped to its first element and the value replaced
// by -inf), so all loads are issued back to back.  VEC = 4 needs V % 4 == 0.
template <int VEC, int PER>
__device__ __forceinline__ void load_chunk(const float* row, int lo, int hi, float (&x)[PER]) {
#pragma unroll
  for (int k = 0; k < PER / VEC; ++k) {
    const int base = lo + (k * kThreads + (int)threadIdx.x) * VEC;
    const bool in = base < hi;
    const int at = in ? base : lo;
    if (VEC == 4) {
      const float4 v4 = *reinterpret_cast<const float4*>(row + at);
      x[k * VEC] = in ? v4.x : -INFINITY;
      x[k * VEC + (VEC > 1 ? 1 : 0)] = in ? v4.y : -INFINITY;
      x[k * VEC + (VEC > 2 ? 2 : 0)] = in ? v4.z : -INFINITY;
      x[k * VEC + (VEC > 3 ? 3 : 0)] = in ? v4.w : -INFINITY;
    } else {
      const float v = row[at];
      x[k] = in ? v : -INFINITY;
    }
  }
}

// Token index of register slot k (see load_chunk).
template <int VEC>
__device__ __forceinline__ int chunk_index(int lo, int k) {
  return lo + ((k / VEC) * kThreads + (int)threadIdx.x) * VEC + k % VEC;
}

// ------------------------------------------------------------------ kernel 1: row chunks

// Chunk c of row p of sequence b: (max, lowest argmax, sum exp(x - max) and, in typical mode,
// sum exp(x - max)(x - max)) into rowparts.  row_load requests the chunk (all loads at once),
// row_reduce reduces it.
template <int VEC, int PER>
__device__ __forceinline__ void row_load(const VerifyArgs& a, int b, int p, int c, float (&x)[PER]) {
  const float* row = a.logits + ((size_t)b * a.N + p) * a.V;
  const int lo = c * a.RC;                 // a.RC == PER * kThreads
  load_chunk<VEC>(row, lo, min(a.V, lo + a.RC), x);
}

// Reduction of a chunk loaded by row_load.
template <int VEC, int PER>
__device__ void row_reduce(const VerifyArgs& a, int b, int p, int c, const float (&x)[PER]) {
  const int t = threadIdx.x;
  const int lo = c * a.RC;
  const int hi = min(a.V, lo + a.RC);
  // chunk max (lowest index: a thread's slots run in increasing token order), nonfinite flag
  float m = -INFINITY;
  int am = INT_MAX, nf = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int idx = chunk_index<VEC>(lo, k);
    if (idx < hi) {
      nf |= !isfinite(x[k]);
      if (x[k] > m) { m = x[k]; am = idx; }
    }
  }
  block_argmax(m, am, nf);
  // sum exp(x - max); the entropy term sum exp(x - max)(x - max) only in typical mode (the
  // other modes never read it)
  double S = 0.0, A = 0.0;
  if (m != -INFINITY && !nf) {
    if (a.mode == SPEC_VERIFY_TYPICAL) {
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const float d = x[k] - m;          // -inf past the chunk -> exp 0
        const float ex = __expf(d);
        S += (double)ex;
        A += (ex > 0.f) ? (double)ex * (double)d : 0.0;
      }
    } else {
#pragma unroll
      for (int k = 0; k < PER; ++k) S += (double)__expf(x[k] - m);
    }
  }
  block_sum2(S, A);
  if (am == INT_MAX) m = -INFINITY;
  if (t == 0) a.rowparts[((size_t)b * a.N + p) * a.CR + c] = RowPart{S, A, m, am, nf, 0};
}

template <int VEC, int PER>
__global__ __launch_bounds__(kThreads) void rows_kernel(VerifyArgs a) {
  // 1-D grid over (seq, node, chunk): grid y/z are limited to 65536.
  const int c = blockIdx.x % a.CR;
  const int p = (blockIdx.x / a.CR) % a.N;
  const int b = blockIdx.x / (a.CR * a.N);
  const int t = threadIdx.x;
  // n_nodes and the parent entries are requested together (the parent load does not wait for
  // n; its index is clamped into the row, and entries past n are ignored below)
  const int n = a.n_nodes ? a.n_nodes[b] : a.N;
  const int par = a.parents[(size_t)b * a.N + min(max(t, 1), a.N - 1)];
  if (n < 0 || n > a.N || p >= n) return;
  // only rows of nodes that some node names as its parent are read
  const int named = (t >= 1 && t < n && par == p) ? 1 : 0;
  if (!__syncthreads_or(named)) return;
  if (a.wsync && c == 0 && t == 0) a.wsync[(size_t)b * a.N + p] = 0;
  float x[PER];
  row_load<VEC>(a, b, p, c, x);
  row_reduce<VEC>(a, b, p, c, x);
}

// Large problems: most (sequence, node, chunk) workgroups of rows_kernel only look at the
// parents and leave, and on large grids those empty workgroups, interleaved with the ones that
// stream, cost about a fifth of the pass.  So one workgroup first lists the rows with children,
// in (sequence, node) order, and the row pass then maps workgroup i to the i-th (listed row,
// chunk) item.  Used for B * N <= kListMax.
constexpr int kListMax = 4096;
constexpr int kListPer = kListMax / kThreads;

// Thread t owns the contiguous entries [t * per, t * per + per) of the B x N (sequence, node)
// table in both passes; its parent and n_nodes loads are all requested at once.
__global__ __launch_bounds__(kThreads) void rows_list_kernel(VerifyArgs a) {
  __shared__ unsigned char s_named[kListMax];
  const int t = threadIdx.x;
  const int total = a.B * a.N;
  const int per = (total + kThreads - 1) / kThreads;   // <= kListPer
  const int i0 = t * per;
  int par[kListPer], nn[kListPer];
#pragma unroll
  for (int k = 0; k < kListPer; ++k) {
    const int i = min(i0 + k, total - 1);
    par[k] = a.parents[i];
    nn[k] = a.n_nodes ? a.n_nodes[i / a.N] : a.N;
  }
#pragma unroll
  for (int k = 0; k < kListPer; ++k)
    if (k < per && i0 + k < total) s_named[i0 + k] = 0;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kListPer; ++k) {
    const int i = i0 + k;
    if (k < per && i < total) {
      // a valid child's parent: entries of sequences with an invalid n_nodes, and invalid
      // parent entries, list nothing (the decision reports those errors)
      const int b = i / a.N, c = i - b * a.N, n = nn[k], p = par[k];
      if (n >= 1 && n <= a.N && c >= 1 && c < n && p >= 0 && p < c) s_named[b * a.N + p] = 1;
    }
  }
  __syncthreads();
  // ordered compaction over the same runs
  int cnt = 0;
#pragma unroll
  for (int k = 0; k < kListPer; ++k)
    if (k < per && i0 + k < total) cnt += s_named[i0 + k];
  double all;
  int at = (int)(block_scan((double)cnt, all) - cnt);   // counts are exact in fp64
#pragma unroll
  for (int k = 0; k < kListPer; ++k)
    if (k < per && i0 + k < total && s_named[i0 + k]) a.row_list[at++] = i0 + k;
  if (t == 0) *a.row_count = (int)all;
}

// Workgroup i takes the i-th (listed row, chunk) item, so the workgroups with work come first
// and back to back; the rest leave after one look at the count.  The count and the list entry
// are requested together (the entry's index is clamped into the list).
template <int VEC, int PER>
__global__ __launch_bounds__(kThreads) void rows_listed_kernel(VerifyArgs a) {
  const int it = blockIdx.x;
  const int count = *a.row_count;
  const int idx = a.row_list[min(it / a.CR, a.B * a.N - 1)];
  if (it >= count * a.CR) return;
  const int b = idx / a.N;
  const int p = idx - b * a.N;
  const int c = it - (it / a.CR) * a.CR;
  if (a.wsync && c == 0 && threadIdx.x == 0) a.wsync[idx] = 0;
  float x[PER];
  row_load<VEC>(a, b, p, c, x);
  row_reduce<VEC>(a, b, p, c, x);
}

// ------------------------------------------------------------------ kernel 2: decision

__device__ void write_neutral(const VerifyArgs& a, int b, int e) {
  const int t = threadIdx.x;
  if (t < a.N && a.node_accept) a.node_accept[(size_t)b * a.N + t] = 0;
  for (int j = t; j <= a.max_depth; j += kThreads) a.path[(size_t)b * (a.max_depth + 1) + j] = -1;
  if (t == 0) {
    a.accept_len[b] = 0;
    a.bonus[b] = -1;
    a.err[b] = e;
  }
}

// The decision for sequence b, in every thread of the workgroup.  Each workgroup of the bonus
// pass derives it for itself (a few KB of chunk partials and one gather per node, read from
// L2 by all chunks of the sequence) instead of waiting for a kernel of its own; only the
// workgroup with `out` set writes the outputs and the plan for the draw.
__device__ BonusPlan decide(const VerifyArgs& a, int b, bool out) {
  __shared__ int s_par[SPEC_MAX_NODES];
  __shared__ int s_dep[SPEC_MAX_NODES];
  __shared__ int s_acc[SPEC_MAX_NODES];
  __shared__ int s_has[SPEC_MAX_NODES];
  __shared__ float s_mx[SPEC_MAX_NODES];
  __shared__ int s_am[SPEC_MAX_NODES];
  __shared__ double s_S[SPEC_MAX_NODES];
  __shared__ double s_H[SPEC_MAX_NODES];
  __shared__ int s_drow[SPEC_MAX_NODES];
  __shared__ int s_first[SPEC_MAX_NODES];      // lowest-index child of each node
  __shared__ int s_fpass[SPEC_MAX_NODES];      // walk: lowest-index child that passes its test
  __shared__ double s_wend[SPEC_MAX_NODES];
  __shared__ int s_err, s_best, s_minchild;
  __shared__ BonusPlan s_plan;
  const int c = threadIdx.x;
  // Every load that does not depend on another is requested here, together: n_nodes, the
  // parent, token, uniform and draft row of this thread's node, and the chunk partials this
  // lane merges (L lanes per node: 4, 2 or 1 for up to 64, 128 or 256 nodes, each lane a
  // strided subset of the chunks).  Indices are clamped into their arrays; what a thread reads
  // for a node past n, or for a row without children (whose partials were never written), is
  // ignored.
  const int n = a.n_nodes ? a.n_nodes[b] : a.N;
  const size_t ci = (size_t)b * a.N + min(c, a.N - 1);
  const int par_c = a.parents[ci];
  const int tok_c = a.tokens[ci];
  const float u_c = a.uniforms[ci];
  const bool walk = a.mode == SPEC_VERIFY_WALK;
  const bool rej = a.mode == SPEC_VERIFY_REJECT || walk;
  const int drow_c = rej ? a.draft_row[ci] : -1;
  // walk: this node's test constants and its residual scale as a parent (a.wc, a.wf, a.wend
  // always point into the workspace; other modes read and ignore them)
  const size_t wi = walk ? ci : 0;
  const double wc_c = a.wc[wi], wf_c = a.wf[wi], wend_c = a.wend[wi];
  const int L = a.N <= 64 ? 4 : (a.N <= 128 ? 2 : 1);
  const int mn = c / L, sub = c % L;
  const RowPart* rp = a.rowparts + ((size_t)b * a.N + min(mn, a.N - 1)) * a.CR;
  RowPart q[kPartsPerLane];
#pragma unroll
  for (int k = 0; k < kPartsPerLane; ++k) {
    const int ck = sub + k * L;
    q[k] = rp[ck < a.CR ? ck : 0];
  }
  // Second round, in flight during the merge: the target logit of this node's token in its
  // parent's row and, for rejection sampling, either the draft probability of that token (one
  // vocabulary) or its draft-vocabulary index (the probability is then gathered after the
  // merge).  Both loads are unconditional, from a pointer chosen per launch, so that no branch
  // makes the merge wait for them; their values are used only once the node is validated.
  const int pc = min(max(par_c, 0), a.N - 1);
  const int tc = min(max(tok_c, 0), a.V - 1);
  const float lpx_c = a.logits[((size_t)b * a.N + pc) * a.V + tc];
  const size_t drow_off = rej ? ((size_t)b * a.R + min(max(drow_c, 0), a.R - 1)) * a.Vd : 0;
  const float dval_c = *((rej && !a.t2d) ? a.draft + drow_off + tc : a.logits);
  const int dx_c = *((rej && a.t2d) ? a.t2d + tc : a.parents);
  if (c == 0) { s_err = INT_MAX; s_best = -1; s_minchild = INT_MAX; }
  if (c < a.N) {
    s_par[c] = par_c; s_has[c] = 0; s_acc[c] = 0; s_drow[c] = drow_c;
    s_first[c] = INT_MAX; s_fpass[c] = INT_MAX; s_wend[c] = wend_c;
  }
  __syncthreads();
  BonusPlan* plan = a.plans + b;
  if (n < 0 || n > a.N || n == 0) {
    if (out) {
      write_neutral(a, b, n == 0 ? 0 : err_word(0, SPEC_ERR_NNODES));
      if (c == 0) *plan = BonusPlan{0, 0, 0, 0.f, 0.0};
    }
    return BonusPlan{0, 0, 0, 0.f, 0.0};
  }

  // rows read: nodes named as a parent by some valid child
  if (c >= 1 && c < n) {
    const int p = s_par[c];
    if (p >= 0 && p < c) {
      s_has[p] = 1;
      if (walk) atomicMin(&s_first[p], c);
    }
  }
  __syncthreads();
  const bool mhas = mn < n && s_has[mn];
  int code = 0, depth = 0, tok = -1, drow = -1, dx = -1;
  float u = 0.f;
  if (c < n) {
    const int p = s_par[c];
    if (c == 0) {
      if (p != -1) code = SPEC_ERR_ROOT;
    } else if (p < 0 || p >= c) {
      code = SPEC_ERR_PARENT;
    } else {
      tok = tok_c;
      u = u_c;
      drow = drow_c;
      int j = c;
      while (j > 0) {
        const int pj = s_par[j];
        if (pj < 0 || pj >= j) break;
        j = pj;
        ++depth;
      }
      if (depth > a.max_depth) code = SPEC_ERR_DEPTH;
      else if (tok < 0 || tok >= a.V) code = SPEC_ERR_TOKEN;
      if (code == 0 && rej) {
        // the walk needs the children of a node on one draft row (its first child's)
        const int r0 = walk ? s_drow[s_first[s_par[c]]] : drow;
        if (drow < 0 || drow >= a.R) code = SPEC_ERR_DRAFTROW;
        else if (r0 >= 0 && r0 < a.R && r0 != drow) code = SPEC_ERR_DRAFTROW;
        else dx = tok;                          // mapped (and checked) after the merge
      }
    }
    s_dep[c] = depth;
  }

  // ---- statistics of the rows that have children: merge their chunks.  Max first, then
  // S = sum_c S_c e^(m_c - M) and A = sum_c e^(m_c - M) (A_c + (m_c - M) S_c); the chunk
  // exponentials are independent of one another.  Chunks past the first kPartsPerLane per
  // lane are read in further batches.
  {
    float m = -INFINITY;
    int am = INT_MAX, nf = 0;
    auto upd = [&](const RowPart& r) {
      nf |= r.nonfinite;
      if (r.m > m || (r.m == m && r.argmax < am)) { m = r.m; am = r.argmax; }
    };
    const int per_lane = kPartsPerLane * L;
    if (mhas) {
#pragma unroll
      for (int k = 0; k < kPartsPerLane; ++k)
        if (sub + k * L < a.CR) upd(q[k]);
      for (int k0 = per_lane; k0 < a.CR; k0 += per_lane) {
        RowPart r[kPartsPerLane];
#pragma unroll
        for (int k = 0; k < kPartsPerLane; ++k) {
          const int ck = k0 + sub + k * L;
          r[k] = rp[ck < a.CR ? ck : 0];
        }
#pragma unroll
        for (int k = 0; k < kPartsPerLane; ++k)
          if (k0 + sub + k * L < a.CR) upd(r[k]);
      }
    }
    for (int o = 1; o < L; o <<= 1) {            // the L lanes of a node are adjacent
      const float m2 = __shfl_xor(m, o);
      const int am2 = __shfl_xor(am, o), nf2 = __shfl_xor(nf, o);
      if (m2 > m || (m2 == m && am2 < am)) { m = m2; am = am2; }
      nf |= nf2;
    }
    double S = 0.0, A = 0.0;
    auto add = [&](const RowPart& r) {
      if (r.m == -INFINITY) return;
      const double d = (double)r.m - (double)m;
      const double sc = exp(d);
      S += sc * r.S;
      A += sc * (r.A + d * r.S);
    };
    if (mhas && m != -INFINITY && !nf) {
#pragma unroll
      for (int k = 0; k < kPartsPerLane; ++k)
        if (sub + k * L < a.CR) add(q[k]);
      for (int k0 = per_lane; k0 < a.CR; k0 += per_lane) {
        RowPart r[kPartsPerLane];
#pragma unroll
        for (int k = 0; k < kPartsPerLane; ++k) {
          const int ck = k0 + sub + k * L;
          r[k] = rp[ck < a.CR ? ck : 0];
        }
#pragma unroll
        for (int k = 0; k < kPartsPerLane; ++k)
          if (k0 + sub + k * L < a.CR) add(r[k]);
      }
    }
    for (int o = 1; o < L; o <<= 1) {
      S += __shfl_xor(S, o);
      A += __shfl_xor(A, o);
    }
    if (mhas && sub == 0) {
      if (nf) atomicMin(&s_err, err_word(mn, SPEC_ERR_NONFINITE));
      s_mx[mn] = m;
      s_am[mn] = am;
      s_S[mn] = S;
      s_H[mn] = log(S) - A / S;
    }
  }
  if (code == 0 && dx >= 0 && a.t2d) {
    dx = dx_c;
    if (dx < -1 || dx >= a.Vd) code = SPEC_ERR_MAP;
  }
  if (code) atomicMin(&s_err, err_word(c, code));
  __syncthreads();
  if (s_err != INT_MAX) {
    if (out) {
      write_neutral(a, b, s_err);
      if (c == 0) *plan = BonusPlan{0, 0, 0, 0.f, 0.0};
    }
    return BonusPlan{0, 0, 0, 0.f, 0.0};
  }

  // ---- per-node tests (fp64)
  if (c >= 1 && c < n) {
    const int p = s_par[c];
    const double T = exp((double)lpx_c - (double)s_mx[p]) / s_S[p];
    bool acc;
    if (a.mode == SPEC_VERIFY_GREEDY) {
      acc = tok == s_am[p];
    } else if (a.mode == SPEC_VERIFY_TYPICAL) {
      const double tau = fmin((double)a.eps, (double)a.delta * exp(-s_H[p]));
      acc = T >= tau;
    } else {
      double d = 0.0;
      if (dx >= 0) d = a.t2d ? (double)a.draft[drow_off + dx] : (double)dval_c;
      // walk: u D[x] < R[x] with R = relu(T - wc D) / wf, the running residual after the
      // earlier siblings' rejections (none left once it has summed to zero)
      acc = walk ? (wf_c > 0.0 && (double)u * d * wf_c < T - wc_c * d) : (double)u * d < T;
    }
    s_acc[c] = acc ? 1 : 0;
  }
  if (c == 0) s_acc[0] = 1;
  __syncthreads();
  if (walk) {
    // siblings are tried in index order: only the first child that passes is taken
    if (c >= 1 && c < n && s_acc[c]) atomicMin(&s_fpass[s_par[c]], c);
    __syncthreads();
    const int keep = (c >= 1 && c < n) ? (s_acc[c] && s_fpass[s_par[c]] == c) : 0;
    __syncthreads();
    if (c >= 1 && c < n) s_acc[c] = keep;
    __syncthreads();
  }

  // ---- survival and the deepest survivor (walk: the survivors are the walk's path)
  bool ok = true;
  if (c < n) {
    int j = c;
    while (j > 0) {
      ok = ok && s_acc[j];
      j = s_par[j];
    }
    if (ok) atomicMax(&s_best, (s_dep[c] << 9) | (511 - c));
  }
  if (out && c < a.N && a.node_accept)
    a.node_accept[(size_t)b * a.N + c] = (c < n) ? (uint8_t)(walk ? ok : s_acc[c]) : 0;
  __syncthreads();
  const int m = 511 - (s_best & 511);
  const int dm = s_best >> 9;
  if (c >= 1 && c < n && s_par[c] == m) atomicMin(&s_minchild, c);
  if (out)
    for (int j = c; j <= a.max_depth; j += kThreads)
      if (j > dm) a.path[(size_t)b * (a.max_depth + 1) + j] = -1;
  __syncthreads();
  if (c == 0) {
    if (out) {
      int j = m;
      for (int d = dm; d >= 0; --d) {
        a.path[(size_t)b * (a.max_depth + 1) + d] = j;
        j = s_par[j];
      }
      a.accept_len[b] = dm;
      a.err[b] = 0;
    }
    BonusPlan pl{m, 0, 0, 0.f, 0.0, 1.0};
    if (a.mode == SPEC_VERIFY_GREEDY) {
      if (s_has[m]) {
        if (out) a.bonus[b] = s_am[m];
      } else {
        pl.kind = 1;
      }
    } else if (a.mode == SPEC_VERIFY_TYPICAL) {
      pl.kind = 2;
    } else if (s_minchild != INT_MAX) {
      pl.kind = 3;
      pl.r = s_drow[s_minchild];
      pl.M = s_mx[m];
      pl.S = s_S[m];
      if (walk) pl.cs = s_wend[m];
    } else {
      pl.kind = 2;
    }
    if (out) *plan = pl;
    s_plan = pl;
  }
  __syncthreads();
  return s_plan;
}

// ------------------------------------------------------------------ kernels 3-4: bonus draw

__device__ __forceinline__ double draft_at(const VerifyArgs& a, int b, int r, int v) {
  if (a.t2d) {
    // Only candidates' entries are validated; any other entry outside [0, Vd) reads as
    // "not in the draft vocabulary".
    const int dx = a.t2d[v];
    return (dx >= 0 && dx < a.Vd) ? (double)a.draft[((size_t)b * a.R + r) * a.Vd + dx] : 0.0;
  }
  return (double)a.draft[((size_t)b * a.R + r) * a.Vd + v];
}

// ------------------------------------------------------------------ walk: residual chains
//
// The walk tries the children c_1 < c_2 < ... of a node p (one draft row D) against a running
// distribution: R_0 = T_p, and R_j = norm(relu(R_(j-1) - D)) after the j-th rejection.  Since
// relu(relu(y) - z) = relu(y - z) for z >= 0, R_j = relu(T_p - c_j D) / f(c_j) with
// f(c) = sum_x relu(T_p[x] - c D[x]), c_0 = 0, f(c_0) = 1 and c_(j+1) = c_j + f(c_j).  None of
// this depends on which children pass, so the chain of every node is computed ahead of the
// decision, all nodes at once: the workgroup of node p writes (c_(j-1), f(c_(j-1))) for its
// j-th child and c_k (k children) for a residual bonus draw at p.
//
// Each f is a pass over the row, one 1024-thread workgroup per node (the passes are sequential).
// The test is done in units of S: relu(T - c D) = relu(e - cS D) / S with e = fp32 exp(x - M) (as
// in the row pass) and cS = c S, one fp64 FMA per token.  Tokens with D = 0 add T at every c:
// their sum is taken in the first pass only.  A token with D > 0 that adds nothing at c adds
// nothing at any larger c, since e - cS D only falls as c grows; so each streaming pass also
// collects, in LDS, the tokens with D != 0 that still add something, and once they fit (the
// chain's c grows by f each step and the set shrinks), every later pass reads only that list.
// Every thread keeps two register sets of 8 tokens in flight (the next set's loads are issued
// before the current one is reduced), and the way the draft row is read (DM: 0 one value at a
// time, 1 16-byte loads, 2 through t2d) is fixed per launch.  Grid (seq, node); nodes with fewer
// than two children need no pass.
constexpr int kChainCap = 16384;              // LDS list: (exp(x - M), D) pairs, 128 KB

template <int THREADS, int PER, int VEC, int DM>
struct Chain {
  static constexpr int kWaves = THREADS / kWave;
  static constexpr int kStep = THREADS * PER;

  // token index of slot u of the set starting at v0 (VEC consecutive tokens per load)
  static __device__ __forceinline__ int index(int v0, int u) {
    return v0 + ((u / VEC) * THREADS + (int)threadIdx.x) * VEC + u % VEC;
  }

  static __device__ __forceinline__ double sum(double v, double* red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x >> 6;
    if (lane == 0) red[wv] = v;
    __syncthreads();
    double r = 0.0;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) r += red[q];
    __syncthreads();
    return r;
  }

  static __device__ __forceinline__ void load(const VerifyArgs& a, const float* row, const float* drow, int v0,
                                              float (&x)[PER], float (&d)[PER]) {
#pragma unroll
    for (int u = 0; u < PER / VEC; ++u) {
      const int vb = index(v0, u * VEC);
      const int at = vb < a.V ? vb : 0;
      if (VEC == 4) {
        const float4 x4 = *reinterpret_cast<const float4*>(row + at);
        x[u * VEC] = x4.x;
        x[u * VEC + (VEC > 1 ? 1 : 0)] = x4.y;
        x[u * VEC + (VEC > 2 ? 2 : 0)] = x4.z;
        x[u * VEC + (VEC > 3 ? 3 : 0)] = x4.w;
        if (DM == 1) {
          const float4 d4 = *reinterpret_cast<const float4*>(drow + at);
          d[u * VEC] = d4.x;
          d[u * VEC + (VEC > 1 ? 1 : 0)] = d4.y;
          d[u * VEC + (VEC > 2 ? 2 : 0)] = d4.z;
          d[u * VEC + (VEC > 3 ? 3 : 0)] = d4.w;
        }
      } else {
        x[u] = row[at];
      }
    }
    if (DM == 2) {
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int v = index(v0, u);
        const int dx = a.t2d[v < a.V ? v : 0];
        const bool mapped = dx >= 0 && dx < a.Vd;
        const float dv = drow[mapped ? dx : 0];
        d[u] = mapped ? dv : 0.f;
      }
    } else if (DM == 0) {
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int v = index(v0, u);
        d[u] = drow[v < a.V ? v : 0];
      }
    }
  }

  // fp += relu(e - cS D) over tokens with D != 0, z += e over tokens with D = 0 (FIRST), cnt =
  // tokens with D != 0 that add something; BUILD appends those to the LDS list as (e, D)
  template <bool FIRST, bool BUILD>
  static __device__ __forceinline__ void reduce(const VerifyArgs& a, int v0, const float (&x)[PER],
                                                const float (&d)[PER], float M, double cS, double& fp, double& z,
                                                int& cnt, float2* list, int* list_n) {
    const int lane = threadIdx.x & (kWave - 1);
    float e[PER], dk[PER];
    int mine = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const bool in = index(v0, u) < a.V;
      e[u] = __expf(x[u] - M);
      if (FIRST) z += (in && d[u] == 0.f) ? (double)e[u] : 0.0;
      const double q = __builtin_fma(-cS, (double)d[u], (double)e[u]);
      const bool keep = in && d[u] != 0.f && q > 0.0;
      fp += keep ? q : 0.0;
      mine += keep ? 1 : 0;
      dk[u] = keep ? d[u] : 0.f;               // 0 marks a token that is not appended
    }
    cnt += mine;
    if (BUILD) {
      int incl = mine;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      int at = 0;
      if (lane == kWave - 1 && incl) at = atomicAdd(list_n, incl);
      int pos = __shfl(at, kWave - 1) + incl - mine;
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        if (dk[u] != 0.f) {
          if (pos < kChainCap) list[pos] = make_float2(e[u], dk[u]);
          ++pos;
        }
      }
    }
  }

  // the steps s0, s0 + ds, s0 + 2 ds, ... of kStep tokens each
  template <bool FIRST, bool BUILD>
  static __device__ void stream(const VerifyArgs& a, const float* row, const float* drow, float M, double cS,
                                double& fp, double& z, int& cnt, float2* list, int* list_n, int s0, int ds) {
    float xa[PER], da[PER], xb[PER], db[PER];
    const int v1 = ds * kStep;
    load(a, row, drow, s0 * kStep, xa, da);
    for (int v0 = s0 * kStep; v0 < a.V; v0 += 2 * v1) {
      load(a, row, drow, v0 + v1, xb, db);   // in flight during the reduce
      reduce<FIRST, BUILD>(a, v0, xa, da, M, cS, fp, z, cnt, list, list_n);
      if (v0 + v1 >= a.V) break;
      load(a, row, drow, v0 + 2 * v1, xa, da);
      reduce<FIRST, BUILD>(a, v0 + v1, xb, db, M, cS, fp, z, cnt, list, list_n);
    }
  }
};

// Several workgroups per node (a.wk > 1, chosen on the host so that every workgroup that can
// have work is resident at once, one per CU): workgroup q of node p streams the steps q, q + wk,
// ... of each pass, keeps its own LDS list, and after every pass stores its partial sums in the
// node's slots of that pass's parity (a workgroup can be one pass ahead of a sibling still
// reading, never two) and, once the stores are complete, adds its arrival to the node's
// counter; each then waits for all wk arrivals and sums the partials in a fixed order, so every
// workgroup of the node derives the same c_(j+1).  The wait is bounded: a workgroup that runs out of it (a sibling
// that is not resident) leaves, except workgroup 0, which finishes the chain alone over the
// whole row; the results are the same up to the order of the fp64 sums.
constexpr int kWalkSpinMax = 1 << 14;   // polls of the counter (each followed by a short sleep);
                                        // the tuning override walk_spin sets another

template <int THREADS, int PER, int VEC, int DM>
__global__ __launch_bounds__(THREADS) void walk_chain_kernel(VerifyArgs a) {
  using CH = Chain<THREADS, PER, VEC, DM>;
  __shared__ float2 s_list[kChainCap];
  __shared__ int s_kids[SPEC_MAX_NODES];
  __shared__ int s_wcnt[CH::kWaves];
  __shared__ double s_red[CH::kWaves];
  __shared__ int s_n;
  __shared__ float s_M;
  __shared__ double s_S;
  __shared__ double s_fp, s_z;
  __shared__ int s_ok;
  const int K = a.wk;
  const int wg_node = blockIdx.x / K, part = blockIdx.x - wg_node * K;
  // node-major over the batch (every sequence's node 0 first, then node 1, ...): low-index
  // nodes, nearest the root, tend to have the most children and so the longest chains
  const int p = wg_node / a.B, b = wg_node - p * a.B;
  const size_t node = (size_t)b * a.N + p;       // (sequence, node) index of the counters and slots
  const int t = threadIdx.x, lane = t & (kWave - 1), wv = t >> 6;
  const int n = a.n_nodes ? a.n_nodes[b] : a.N;
  if (n < 1 || n > a.N || p >= n) return;
  const size_t base = (size_t)b * a.N;
  // the children of p in index order (one candidate node per thread; THREADS >= N)
  const int i = p + 1 + t;
  const bool kid = i < n && a.parents[base + i] == p;
  const unsigned long long bal = __ballot(kid);
  if (lane == 0) s_wcnt[wv] = __popcll(bal);
  __syncthreads();
  int off = 0, k = 0;
#pragma unroll
  for (int q = 0; q < CH::kWaves; ++q) {
    off += q < wv ? s_wcnt[q] : 0;
    k += s_wcnt[q];
  }
  if (kid) s_kids[off + __popcll(bal & ((1ull << lane) - 1))] = i;
  __syncthreads();
  if (k == 0) return;
  if (t == 0 && part == 0) {
    a.wc[base + s_kids[0]] = 0.0;
    a.wf[base + s_kids[0]] = 1.0;
    if (k == 1) a.wend[base + p] = 1.0;
  }
  if (k == 1) return;
  if (t == 0) {                            // row statistics of p from its row-pass chunks
    const RowPart* rp = a.rowparts + (base + p) * a.CR;
    float M = -INFINITY;
    for (int q = 0; q < a.CR; ++q) M = fmaxf(M, rp[q].m);
    double S = 0.0;
    for (int q = 0; q < a.CR; ++q)
      if (rp[q].m != -INFINITY) S += rp[q].S * exp((double)rp[q].m - (double)M);
    s_M = M;
    s_S = S;
  }
  __syncthreads();
  const float M = s_M;
  const double S = s_S, invS = 1.0 / S;
  const int r = min(max(a.draft_row[base + s_kids[0]], 0), a.R - 1);
  const float* row = a.logits + (base + p) * a.V;
  const float* drow = a.draft + ((size_t)b * a.R + r) * a.Vd;
  int parts = K;          // workgroups sharing the passes (1 once this one works alone)
  double cj = 1.0, zS = 0.0;               // zS: sum of e over tokens with D = 0
  int listed = -1;        // entries of s_list once it holds every token (of this workgroup's
                          // steps) that can still add
  // this workgroup's tokens with D != 0 that added in the previous pass; before the first, the
  // tokens of its steps, so the list is built at once when it can hold all of them
  const int row_steps = (a.V + CH::kStep - 1) / CH::kStep;
  const int my_steps = K > 1 ? (part < row_steps ? (row_steps - part + K - 1) / K : 0) : row_steps;
  int prev = (long long)my_steps * CH::kStep <= kChainCap ? my_steps * CH::kStep : INT_MAX;
  bool zdone = false;     // zS holds the whole row's sum
  for (int j = 1; j < k; ++j) {
    const double cS = cj * S;
    double fp = 0.0, z = 0.0;
    if (listed < 0) {
      const bool build = prev <= kChainCap;
      if (t == 0) s_n = 0;
      __syncthreads();
      int cnt = 0;
      const int s0 = parts > 1 ? part : 0;
      if (!zdone) {
        if (build) CH::template stream<true, true>(a, row, drow, M, cS, fp, z, cnt, s_list, &s_n, s0, parts);
        else CH::template stream<true, false>(a, row, drow, M, cS, fp, z, cnt, s_list, &s_n, s0, parts);
        z = CH::sum(z, s_red);
      } else {
        if (build) CH::template stream<false, true>(a, row, drow, M, cS, fp, z, cnt, s_list, &s_n, s0, parts);
        else CH::template stream<false, false>(a, row, drow, M, cS, fp, z, cnt, s_list, &s_n, s0, parts);
      }
      fp = CH::sum(fp, s_red);
      prev = (int)CH::sum((double)cnt, s_red);
      if (build) listed = prev;
    } else {
      for (int e = t; e < listed; e += THREADS) {
        const float2 ed = s_list[e];
        const double q = __builtin_fma(-cS, (double)ed.y, (double)ed.x);
        fp += q > 0.0 ? q : 0.0;
      }
      fp = CH::sum(fp, s_red);
    }
    if (parts > 1) {
      if (wv == 0) {
        int ok = 0;
        if (lane == 0) {
          // the slot of this pass's parity: a workgroup may run one pass ahead of a sibling
          // still reading this pass's partials, never two
          double* slot = a.wpart + ((node * K + part) * 2 + (j & 1)) * 2;
          // Everything exchanged here is an agent-scope atomic (performed coherently across the
          // XCDs' caches), so no cache write-back or invalidation is needed; the wait makes the
          // two stores complete before the arrival is counted.
          __hip_atomic_store(slot, fp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(slot + 1, z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          __builtin_amdgcn_s_waitcnt(0);
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          __hip_atomic_fetch_add(a.wsync + node, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const int target = j * K;
          int polls = 0;
          while (!(ok = __hip_atomic_load(a.wsync + node, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) &&
                 ++polls < a.wspin)
            __builtin_amdgcn_s_sleep(8);
        }
        ok = __shfl(ok, 0);
        // lane q loads workgroup q's partials (all at once), summed in a fixed lane order
        double sf = 0.0, sz = 0.0;
        if (ok) {
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          if (lane < K) {
            const double* o = a.wpart + ((node * K + lane) * 2 + (j & 1)) * 2;
            sf = __hip_atomic_load(o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            sz = __hip_atomic_load(o + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          sf = wave_sum(sf);
          sz = wave_sum(sz);
        }
        if (lane == 0) {
          s_fp = sf;
          s_z = sz;
          s_ok = ok;
        }
      }
      __syncthreads();
      if (!s_ok) {
        if (part != 0) return;
        parts = 1;            // workgroup 0 redoes this pass, and the rest, over the whole row
        listed = -1;
        prev = INT_MAX;
        --j;
        continue;
      }
      fp = s_fp;
      z = s_z;
    }
    if (!zdone) {
      zS = z;
      zdone = true;
    }
    const double f = (zS + fp) * invS;
    if (t == 0 && part == 0) {
      a.wc[base + s_kids[j]] = cj;
      a.wf[base + s_kids[j]] = f;
    }
    cj += f;
  }
  if (t == 0 && part == 0) a.wend[base + p] = cj;
}

template <int THREADS, int PER>
void launch_chain(const VerifyArgs& a, dim3 grid, bool vec4, bool dvec, hipStream_t s) {
  const char* nm = "verify_walk_chain";
  const dim3 blk(THREADS);
  if (a.t2d) {
    if (vec4) launch(nm, walk_chain_kernel<THREADS, PER, 4, 2>, grid, blk, s, a);
    else launch(nm, walk_chain_kernel<THREADS, PER, 1, 2>, grid, blk, s, a);
  } else if (vec4 && dvec) {
    launch(nm, walk_chain_kernel<THREADS, PER, 4, 1>, grid, blk, s, a);
  } else if (vec4) {
    launch(nm, walk_chain_kernel<THREADS, PER, 4, 0>, grid, blk, s, a);
  } else {
    launch(nm, walk_chain_kernel<THREADS, PER, 1, 0>, grid, blk, s, a);
  }
}

// Sum over aligned groups of LANES lanes (4, 8, 16, 32 or 64), in every lane of the group: DPP
// moves inside a row of 16 (swap neighbours, swap pairs, mirror each half, mirror the row),
// shuffles across rows.
template <int CTRL>
__device__ __forceinline__ double dpp_move(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xF, 0xF, false);
  return __hiloint2double(hi, lo);
}
template <int LANES>
__device__ __forceinline__ double lane_group_sum(double v) {
  v += dpp_move<0xB1>(v);                      // quad_perm [1, 0, 3, 2]
  v += dpp_move<0x4E>(v);                      // quad_perm [2, 3, 0, 1]
  if (LANES >= 8) v += dpp_move<0x141>(v);     // row_half_mirror
  if (LANES >= 16) v += dpp_move<0x140>(v);    // row_mirror
  if (LANES >= 32) v += __shfl_xor(v, 16);
  if (LANES >= 64) v += __shfl_xor(v, 32);
  return v;
}

template <int VEC, int CS>
__device__ void bonus_chunk(const VerifyArgs& a, int b, int c, const BonusPlan& pl) {
  constexpr int kPer = CS / kThreads;
  const float* row = a.logits + ((size_t)b * a.N + pl.m) * a.V;
  const int lo = c * a.CS, hi = min(a.V, lo + a.CS);
  float x[kPer];
  load_chunk<VEC>(row, lo, hi, x);
  double dr[kPer];
  if (pl.kind == 3) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int v = chunk_index<VEC>(lo, k);
      dr[k] = draft_at(a, b, pl.r, v < hi ? v : lo);
    }
  }
  float m = -INFINITY;
  int am = INT_MAX, nf = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int idx = chunk_index<VEC>(lo, k);
    if (idx < hi) {
      nf |= !isfinite(x[k]);
      if (x[k] > m) { m = x[k]; am = idx; }
    }
  }
  block_argmax(m, am, nf);                 // chunk max / argmax / nonfinite, in every thread
  // Each token's weight of the draw (kind 3: relu(T - D); kind 2: exp(x - chunk max)) is
  // either summed per 64-token group for the one-wave draw (rows of at most 64 chunks) or, for
  // small batches with longer rows, stored so that the workgroup draw scans exactly these
  // values instead of recomputing the chunk.
  double S = 0.0, Q = 0.0;
  double w[kPer], ex[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) w[k] = ex[k] = 0.0;
  if (!nf && pl.kind == 3) {
    // exp(x - M) with the row max, and relu(T - D) with T normalised by the row statistics
    const double inv = 1.0 / pl.S;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      if (chunk_index<VEC>(lo, k) < hi) {
        ex[k] = exp((double)x[k] - (double)pl.M);
        S += ex[k];
        w[k] = fmax(ex[k] * inv - pl.cs * dr[k], 0.0);
        Q += w[k];
      }
    }
  } else if (!nf && pl.kind == 2 && m != -INFINITY) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      w[k] = (x[k] == -INFINITY) ? 0.0 : exp((double)x[k] - (double)m);
      S += w[k];
    }
  }
  if (a.weights && pl.kind >= 2) {
    double* wrow = a.weights + (size_t)b * a.C * a.CS;
#pragma unroll
    for (int k = 0; k < kPer; k += 2) {       // chunk_index(k + 1) == chunk_index(k) + 1 for even k
      const int v = chunk_index<VEC>(lo, k);
      if (VEC >= 2) {
        *reinterpret_cast<double2*>(wrow + v) = make_double2(w[k], w[k + 1]);
      } else {
        wrow[v] = w[k];
        wrow[chunk_index<VEC>(lo, k + 1)] = w[k + 1];
      }
    }
  }
  if (a.gsum && pl.kind >= 2) {
    // Group sums for the one-wave draw: this thread's VEC consecutive tokens of register group
    // g lie in 64-token group (g * kThreads + t) * VEC / 64, shared by kWave / VEC aligned lanes
    // of one wave, which add their parts; the first of them stores the sums (the exp(x - M)
    // sums only for residual draws).
    constexpr int kLanes = kWave / VEC;
    double* gs = a.gsum + ((size_t)b * a.C + c) * (CS / 64) * 2;
    const bool resid = pl.kind == 3;
#pragma unroll
    for (int g = 0; g < kPer / VEC; ++g) {
      double pw = 0.0, pe = 0.0;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        pw += w[g * VEC + e];
        pe += ex[g * VEC + e];
      }
      pw = lane_group_sum<kLanes>(pw);
      if (resid) pe = lane_group_sum<kLanes>(pe);
      if ((threadIdx.x & (kLanes - 1)) == 0) {
        const int grp = (chunk_index<VEC>(lo, g * VEC) - lo) / 64;
        *reinterpret_cast<double2*>(gs + grp * 2) = make_double2(pw, pe);
      }
    }
  }
  block_sum2(S, Q);
  if (pl.kind == 3) m = pl.M;              // S is relative to the row max
  if (threadIdx.x == 0) a.bparts[(size_t)b * a.C + c] = BonusPart{S, Q, m, am, nf, 0};
}

// Grid (seq, chunk): the decision of the sequence (outputs written by chunk 0's workgroup),
// then this chunk of the kept row's bonus pass.
template <int VEC, int CS>
__global__ __launch_bounds__(kThreads) void decide_bonus_kernel(VerifyArgs a) {
  const int c = blockIdx.x % a.C, b = blockIdx.x / a.C;
  const BonusPlan pl = decide(a, b, c == 0);
  if (pl.kind == 0) return;
  bonus_chunk<VEC, CS>(a, b, c, pl);
}

// Weight of token v for draw `kind`: 2 -> exp(x - M) (T up to the common factor 1/S),
// 3 -> relu(exp(x - M) / S - cs D[v]).
__device__ __forceinline__ double draw_weight(const VerifyArgs& a, int b, int kind, int r, float x, int v,
                                              float M, double S, double cs) {
  const double e = exp((double)x - (double)M);
  if (kind == 2) return e;
  return fmax(e / S - cs * draft_at(a, b, r, v), 0.0);
}

// Smallest token of chunk [lo, hi) whose running sum (from `base`, fp64, ascending token order)
// exceeds thr; -1 if none.  Thread t owns a contiguous run of `per` tokens (a multiple of VEC,
// so the run is read with VEC-wide loads).
template <int VEC, int CS>
__device__ int scan_chunk(const VerifyArgs& a, int b, int kind, int r, const float* row, int lo, int hi,
                          float M, double S, double cs, double base, double thr) {
  constexpr int kPer = CS / kThreads;
  __shared__ int s_hit;
  const int per = (hi - lo + kThreads * VEC - 1) / (kThreads * VEC) * VEC;   // <= kPer
  const int my_lo = lo + (int)threadIdx.x * per;
  float xv[kPer];
#pragma unroll
  for (int k = 0; k < kPer; k += VEC) {
    const int v = my_lo + k;
    const bool in = k < per && v < hi;
    const int at = in ? v : lo;
    if (VEC == 4) {
      const float4 v4 = *reinterpret_cast<const float4*>(row + at);
      xv[k] = v4.x;
      xv[k + (VEC > 1 ? 1 : 0)] = v4.y;
      xv[k + (VEC > 2 ? 2 : 0)] = v4.z;
      xv[k + (VEC > 3 ? 3 : 0)] = v4.w;
    } else {
      xv[k] = row[at];
    }
  }
  double w[kPer];
  double mine = 0.0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int v = my_lo + k;
    w[k] = (k < per && v < hi) ? draw_weight(a, b, kind, r, xv[k], v, M, S, cs) : 0.0;
    mine += w[k];
  }
  if (threadIdx.x == 0) s_hit = INT_MAX;
  double total;
  const double before = base + (block_scan(mine, total) - mine);   // barriers inside
  if (before + mine > thr) {
    double run = before;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      run += w[k];
      if (k < per && my_lo + k < hi && run > thr) { atomicMin(&s_hit, my_lo + k); break; }
    }
  }
  __syncthreads();
  const int hit = s_hit;
  __syncthreads();
  return hit == INT_MAX ? -1 : hit;
}

// Inverse-CDF draw with u = uniforms[b, 0] over the weights of `kind` (rcs: the residual's
// scale of D); thread t < C holds the sum q of chunk t.  The chunk is the first whose inclusive
// prefix exceeds u * Z (if rounding puts u * Z past the end: the last chunk of positive mass),
// then the token inside it.
template <int VEC, int CS>
__device__ int draw(const VerifyArgs& a, int b, int kind, int r, const float* row, double q, float M,
                    double S, double rcs, float u) {
  __shared__ int s_pick, s_last, s_tok;
  __shared__ double s_base[2];
  const int t = threadIdx.x;
  if (t >= a.C) q = 0.0;
  if (t == 0) { s_pick = INT_MAX; s_last = -1; }
  double Z;
  const double incl = block_scan(q, Z);                           // barriers inside
  const double thr = (double)u * Z;
  if (t < a.C && incl > thr) atomicMin(&s_pick, t);
  if (t < a.C && q > 0.0) atomicMax(&s_last, t);
  __syncthreads();
  const int pick = s_pick, last = s_last;
  if (t == pick) s_base[0] = incl - q;
  if (t == last) s_base[1] = incl - q;
  __syncthreads();
  const int cs = pick != INT_MAX ? pick : (last >= 0 ? last : 0);
  const double base = pick != INT_MAX ? s_base[0] : (last >= 0 ? s_base[1] : 0.0);
  const int lo = cs * a.CS, hi = min(a.V, lo + a.CS);
  int tok = scan_chunk<VEC, CS>(a, b, kind, r, row, lo, hi, M, S, rcs, base, thr);
  if (tok < 0) {                            // rounding put thr at the chunk's end
    if (t == 0) {
      s_tok = -1;
      for (int v = hi - 1; v >= lo; --v)
        if (draw_weight(a, b, kind, r, row[v], v, M, S, rcs) > 0.0) { s_tok = v; break; }
    }
    __syncthreads();
    tok = s_tok;
  }
  return tok;
}

// Smallest token of chunk [lo, hi) whose running sum of the stored weights (times scale, from
// `base`, fp64, ascending token order) exceeds thr; -1 if none.  Thread t owns a contiguous run
// of `per` tokens (even, so the run is read with 16-byte loads).
template <int CS>
__device__ int scan_stored(const double* wrow, int lo, int hi, double scale, double base, double thr) {
  constexpr int kPer = CS / kThreads;
  __shared__ int s_hit;
  const int per = (hi - lo + kThreads * 2 - 1) / (kThreads * 2) * 2;   // <= kPer
  const int my_lo = lo + (int)threadIdx.x * per;
  double w[kPer];
#pragma unroll
  for (int k = 0; k < kPer; k += 2) {
    const int v = my_lo + k;
    const bool in = k < per && v < hi;
    const double2 p = *reinterpret_cast<const double2*>(wrow + (in ? v : lo));
    w[k] = in ? p.x * scale : 0.0;
    w[k + 1] = (in && v + 1 < hi) ? p.y * scale : 0.0;
  }
  double mine = 0.0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) mine += w[k];
  if (threadIdx.x == 0) s_hit = INT_MAX;
  double total;
  const double before = base + (block_scan(mine, total) - mine);   // barriers inside
  if (before + mine > thr) {
    double run = before;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      run += w[k];
      if (k < per && my_lo + k < hi && run > thr) { atomicMin(&s_hit, my_lo + k); break; }
    }
  }
  __syncthreads();
  const int hit = s_hit;
  __syncthreads();
  return hit == INT_MAX ? -1 : hit;
}

// Inverse-CDF draw over the weights stored by the bonus pass: thread t < C holds chunk t's sum
// q and the factor that scales its stored weights (1 for a residual draw; exp(chunk max - row
// max) for a draw from T).  Same chunk choice and rounding fallbacks as draw().
template <int CS>
__device__ int draw_stored(const VerifyArgs& a, int b, double q, double scale, float u) {
  __shared__ int s_pick, s_last, s_tok;
  __shared__ double s_base[2], s_scale[2];
  const int t = threadIdx.x;
  if (t >= a.C) q = 0.0;
  if (t == 0) { s_pick = INT_MAX; s_last = -1; }
  double Z;
  const double incl = block_scan(q, Z);                           // barriers inside
  const double thr = (double)u * Z;
  if (t < a.C && incl > thr) atomicMin(&s_pick, t);
  if (t < a.C && q > 0.0) atomicMax(&s_last, t);
  __syncthreads();
  const int pick = s_pick, last = s_last;
  if (t == pick) { s_base[0] = incl - q; s_scale[0] = scale; }
  if (t == last) { s_base[1] = incl - q; s_scale[1] = scale; }
  __syncthreads();
  const int k = pick != INT_MAX ? 0 : 1;
  const int cs = pick != INT_MAX ? pick : (last >= 0 ? last : 0);
  const double base = (pick != INT_MAX || last >= 0) ? s_base[k] : 0.0;
  const double sc = (pick != INT_MAX || last >= 0) ? s_scale[k] : 1.0;
  const int lo = cs * a.CS, hi = min(a.V, lo + a.CS);
  const double* wrow = a.weights + (size_t)b * a.C * a.CS;
  int tok = scan_stored<CS>(wrow, lo, hi, sc, base, thr);
  if (tok < 0) {                            // rounding put thr at the chunk's end
    if (t == 0) {
      s_tok = -1;
      for (int v = hi - 1; v >= lo; --v)
        if (wrow[v] * sc > 0.0) { s_tok = v; break; }
    }
    __syncthreads();
    tok = s_tok;
  }
  return tok;
}

template <int VEC, int CS>
__global__ __launch_bounds__(kThreads) void select_kernel(VerifyArgs a) {
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  // the plan, this thread's chunk part and the draw's uniform u = uniforms[b, 0] are requested
  // together (none of their indices depends on the plan; threads past C read part 0 and ignore
  // it)
  const BonusPlan pl = a.plans[b];
  const BonusPart bp = a.bparts[(size_t)b * a.C + (t < a.C ? t : 0)];
  const float u = a.uniforms[(size_t)b * a.N];
  if (pl.kind == 0) return;
  // merge the chunk parts (one per thread): row max / argmax / nonfinite
  double Sc = 0.0, Qc = 0.0;
  float mc = -INFINITY;
  int amc = INT_MAX, nf = 0;
  if (t < a.C) {
    Sc = bp.S; Qc = bp.Q; mc = bp.m; amc = bp.argmax; nf = bp.nonfinite;
  }
  float m = mc;
  int am = amc;
  block_argmax(m, am, nf);
  if (nf) {
    write_neutral(a, b, err_word(pl.m, SPEC_ERR_NONFINITE));
    return;
  }
  if (pl.kind == 1) {
    if (t == 0) a.bonus[b] = am;
    return;
  }
  const float* row = a.logits + ((size_t)b * a.N + pl.m) * a.V;
  int tok;
  if (pl.kind == 2) {
    const double sc = (mc == -INFINITY) ? 0.0 : exp((double)mc - (double)m);
    if (a.weights) tok = draw_stored<CS>(a, b, Sc * sc, sc, u);
    else tok = draw<VEC, CS>(a, b, 2, pl.r, row, Sc * sc, m, 0.0, 1.0, u);
  } else {
    const double Z = block_sum(t < a.C ? Qc : 0.0);
    if (Z > 0.0) tok = a.weights ? draw_stored<CS>(a, b, Qc, 1.0, u) : draw<VEC, CS>(a, b, 3, pl.r, row, Qc, pl.M, pl.S, pl.cs, u);
    else tok = draw<VEC, CS>(a, b, 2, pl.r, row, Sc, pl.M, pl.S, 1.0, u);   // residual of zero mass: T_m
  }
  if (t == 0) a.bonus[b] = tok;
}

// One-wave draw over stored weights (when the tuning override stores them for a row of at most
// 64 chunks): lane t holds chunk t's part, and inside the chosen chunk lane t owns a contiguous
// run of CS / 64 tokens, so every reduction and scan is a wave shuffle and the kernel has no
// barrier.  Same chunk choice, token choice and rounding fallbacks as select_kernel.

// Inclusive prefix sum over the wave in lane order (fp64).
__device__ __forceinline__ double wave_scan(double v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  return v;
}

__device__ void write_neutral_wave(const VerifyArgs& a, int b, int e) {
  const int t = threadIdx.x;
  if (a.node_accept)
    for (int i = t; i < a.N; i += kWave) a.node_accept[(size_t)b * a.N + i] = 0;
  for (int j = t; j <= a.max_depth; j += kWave) a.path[(size_t)b * (a.max_depth + 1) + j] = -1;
  if (t == 0) {
    a.accept_len[b] = 0;
    a.bonus[b] = -1;
    a.err[b] = e;
  }
}

template <int VEC, int CS>
__global__ __launch_bounds__(kWave) void select_wave_kernel(VerifyArgs a) {
  constexpr int kRun = CS / kWave;             // tokens per lane inside a chunk
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const BonusPlan pl = a.plans[b];
  const BonusPart bp = a.bparts[(size_t)b * a.C + (t < a.C ? t : 0)];
  const float u = a.uniforms[(size_t)b * a.N];
  if (pl.kind == 0) return;
  double Sc = 0.0, Qc = 0.0;
  float mc = -INFINITY;
  int amc = INT_MAX, nf = 0;
  if (t < a.C) {
    Sc = bp.S; Qc = bp.Q; mc = bp.m; amc = bp.argmax; nf = bp.nonfinite;
  }
  float m = mc;
  int am = amc;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {           // row max / lowest argmax / nonfinite
    const float m2 = __shfl_xor(m, o);
    const int am2 = __shfl_xor(am, o), nf2 = __shfl_xor(nf, o);
    if (m2 > m || (m2 == m && am2 < am)) { m = m2; am = am2; }
    nf |= nf2;
  }
  if (nf) {
    write_neutral_wave(a, b, err_word(pl.m, SPEC_ERR_NONFINITE));
    return;
  }
  if (pl.kind == 1) {
    if (t == 0) a.bonus[b] = am;
    return;
  }
  // chunk weights: q = this chunk's sum, scale = factor of its stored weights; a residual of
  // zero mass draws from T_m instead, recomputed from the logits (stored weights are zero)
  double q, scale = 1.0;
  bool stored = true;
  if (pl.kind == 2) {
    scale = (mc == -INFINITY) ? 0.0 : exp((double)mc - (double)m);
    q = Sc * scale;
  } else if (wave_sum(Qc) > 0.0) {
    q = Qc;
  } else {
    q = Sc;                                    // relative to the row max pl.M
    stored = false;
  }
  if (t >= a.C) q = 0.0;
  const double incl = wave_scan(q);
  const double Z = __shfl(incl, kWave - 1);
  const double thr = (double)u * Z;
  const unsigned long long over = __ballot(t < a.C && incl > thr);
  const unsigned long long mass = __ballot(t < a.C && q > 0.0);
  const int cs = over ? __ffsll(over) - 1 : (mass ? 63 - __clzll(mass) : 0);
  const double base = (over || mass) ? __shfl(incl - q, cs) : 0.0;
  const double sc = (over || mass) ? __shfl(scale, cs) : 1.0;
  const int lo = cs * a.CS, hi = min(a.V, lo + a.CS);
  const int my_lo = lo + t * kRun;
  double w[kRun];
  if (stored) {
    const double* wrow = a.weights + (size_t)b * a.C * a.CS;
#pragma unroll
    for (int k = 0; k < kRun; k += 2) {
      const int v = my_lo + k;
      const double2 p = *reinterpret_cast<const double2*>(wrow + (v < hi ? v : lo));
      w[k] = v < hi ? p.x * sc : 0.0;
      w[k + 1] = v + 1 < hi ? p.y * sc : 0.0;
    }
  } else {
    const float* row = a.logits + ((size_t)b * a.N + pl.m) * a.V;
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      const int v = my_lo + k;
      w[k] = v < hi ? exp((double)row[v] - (double)pl.M) : 0.0;
    }
  }
  double mine = 0.0;
#pragma unroll
  for (int k = 0; k < kRun; ++k) mine += w[k];
  const double before = base + (wave_scan(mine) - mine);
  // every lane whose run crosses thr finds its first token past thr; the smallest wins
  int mt = INT_MAX;
  if (before + mine > thr) {
    double run = before;
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      run += w[k];
      if (mt == INT_MAX && my_lo + k < hi && run > thr) mt = my_lo + k;
    }
  }
  int tok = wave_min(mt);
  if (tok == INT_MAX) tok = -1;
  if (tok < 0) {                               // rounding put thr at the chunk's end: the
    int lastpos = -1;                          // last token of positive weight
#pragma unroll
    for (int k = 0; k < kRun; ++k)
      if (my_lo + k < hi && w[k] > 0.0) lastpos = my_lo + k;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) lastpos = max(lastpos, __shfl_xor(lastpos, o));
    tok = lastpos;
  }
  if (t == 0) a.bonus[b] = tok;
}

// One-wave draw from the group sums (the default for rows of at most 64 chunks): lane t
// holds chunk t's part; the chunk holding u * Z is found as in select_wave_kernel, then the
// 64-token group inside it from the group sums the bonus pass left, then the token inside the
// group, each lane recomputing one token's weight exactly as the bonus pass formed it.  Three
// dependent rounds of loads and one exponential per lane, against a workgroup that recomputes
// the whole chunk.  Rounding fallbacks as in the other draws: past the end of the chosen
// chunk or group, its last element of positive weight.
template <int VEC, int CS>
__global__ __launch_bounds__(kWave) void select_groups_kernel(VerifyArgs a) {
  constexpr int kG = CS / 64;                  // groups per chunk (<= 64)
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const BonusPlan pl = a.plans[b];
  const BonusPart bp = a.bparts[(size_t)b * a.C + (t < a.C ? t : 0)];
  const float u = a.uniforms[(size_t)b * a.N];
  if (pl.kind == 0) return;
  double Sc = 0.0, Qc = 0.0;
  float mc = -INFINITY;
  int amc = INT_MAX, nf = 0;
  if (t < a.C) {
    Sc = bp.S; Qc = bp.Q; mc = bp.m; amc = bp.argmax; nf = bp.nonfinite;
  }
  float m = mc;
  int am = amc;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {           // row max / lowest argmax / nonfinite
    const float m2 = __shfl_xor(m, o);
    const int am2 = __shfl_xor(am, o), nf2 = __shfl_xor(nf, o);
    if (m2 > m || (m2 == m && am2 < am)) { m = m2; am = am2; }
    nf |= nf2;
  }
  if (nf) {
    write_neutral_wave(a, b, err_word(pl.m, SPEC_ERR_NONFINITE));
    return;
  }
  if (pl.kind == 1) {
    if (t == 0) a.bonus[b] = am;
    return;
  }
  // chunk weights: as in select_wave_kernel; `slot` picks the group sums that match them
  double q, scale = 1.0;
  int what = 2;                                // 2: T (kind 2), 3: residual, 4: T_m (zero residual)
  if (pl.kind == 2) {
    scale = (mc == -INFINITY) ? 0.0 : exp((double)mc - (double)m);
    q = Sc * scale;
  } else if (wave_sum(Qc) > 0.0) {
    q = Qc;
    what = 3;
  } else {
    q = Sc;                                    // relative to the row max pl.M
    what = 4;
  }
  if (t >= a.C) q = 0.0;
  const double incl = wave_scan(q);
  const double thr = (double)u * __shfl(incl, kWave - 1);
  const unsigned long long over = __ballot(t < a.C && incl > thr);
  const unsigned long long mass = __ballot(t < a.C && q > 0.0);
  const int cs = over ? __ffsll(over) - 1 : (mass ? 63 - __clzll(mass) : 0);
  const double base = (over || mass) ? __shfl(incl - q, cs) : 0.0;
  const double sc = (over || mass) ? __shfl(scale, cs) : 1.0;
  const float mcs = __shfl(mc, cs);            // chunk max (kind 2 weights are relative to it)
  const int lo = cs * a.CS, hi = min(a.V, lo + a.CS);
  // the group
  const double* gs = a.gsum + ((size_t)b * a.C + cs) * kG * 2;
  const bool gin = t < kG && lo + t * 64 < hi;
  const double qg = gin ? gs[t * 2 + (what == 4 ? 1 : 0)] * sc : 0.0;
  const double inclg = wave_scan(qg);
  const unsigned long long overg = __ballot(gin && base + inclg > thr);
  const unsigned long long massg = __ballot(gin && qg > 0.0);
  const int gsel = overg ? __ffsll(overg) - 1 : (massg ? 63 - __clzll(massg) : 0);
  const double baseg = (overg || massg) ? base + __shfl(inclg - qg, gsel) : base;
  // the token: lane t recomputes the weight of token lo + 64 gsel + t
  const int v = lo + gsel * 64 + t;
  const bool tin = v < hi;
  const int at = tin ? v : lo;
  const float* row = a.logits + ((size_t)b * a.N + pl.m) * a.V;
  const float x = row[at];
  double w;
  if (what == 2) {
    w = (x == -INFINITY) ? 0.0 : exp((double)x - (double)mcs);
  } else if (what == 3) {
    const double inv = 1.0 / pl.S;
    w = fmax(exp((double)x - (double)pl.M) * inv - pl.cs * draft_at(a, b, pl.r, at), 0.0);
  } else {
    w = exp((double)x - (double)pl.M);
  }
  w = tin ? w * sc : 0.0;
  const double inclw = wave_scan(w);
  const unsigned long long overw = __ballot(tin && baseg + inclw > thr);
  const unsigned long long massw = __ballot(tin && w > 0.0);
  const int lane = overw ? __ffsll(overw) - 1 : (massw ? 63 - __clzll(massw) : -1);
  if (t == 0) a.bonus[b] = lane >= 0 ? lo + gsel * 64 + lane : -1;
}

// ------------------------------------------------------------------ host

struct VerifyLayout {
  int RC, CR, CS, C;
  int wk;               // WALK: workgroups per node
  bool store_w, listed;
  size_t rowparts, plans, bparts, weights, gsum, row_list, row_count, walk, wsync, wpart, total;
};

// WALK: workgroups per node.  Several only when every workgroup that can have work is resident
// at once (one 1024-thread workgroup per CU; all CUs of the current device but 16), counting the
// most nodes that can have two children, (N - 1) / 2 per sequence; at most one per 8K-token step
// of the row.  The tuning override walk_parts forces a count (1-16).
constexpr int kWalkMaxParts = 16;
constexpr int kWalkStep = 1024 * 8;     // tokens per streaming step of the chain
constexpr int kMaxWalkDevices = 64;
int walk_resident() {
  static std::atomic<int> cached[kMaxWalkDevices];   // 0: not looked up yet
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxWalkDevices) {
    (void)hipGetLastError();
    return 0;
  }
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
    v = std::max(1, cus - 16);
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}
int walk_parts(int B, int N, int V) {
  const long long multi = (long long)B * std::max(1, (N - 1) / 2);
  const int steps = (V + kWalkStep - 1) / kWalkStep;
  const int k = (int)std::min<long long>(std::min<long long>(kWalkMaxParts, walk_resident() / multi), steps);
  return std::max(1, std::min(tuning(kKnobWalkParts, k), kWalkMaxParts));
}

// The listed row pass pays one more launch, so it is used from this many (sequence, node,
// chunk) items of the plain grid up (the tuning override verify_rows_list forces either path).
constexpr size_t kListMinItems = 8192;

// Row-pass chunk: 8K logits (measured faster than 4K and 16K at batch 1 and 16); the tuning
// override verify_chunk (4096, 8192 or 16384) forces another.
constexpr int kRowChunkMin = 4096;
constexpr int kMaxVocab = 1 << 20;     // 256 chunks of 4096 logits in the bonus draw
int row_chunk() {
  const int v = tuning(kKnobVerifyChunk, 8192);
  return (v == 4096 || v == 8192 || v == 16384) ? v : 8192;
}

// The decision + bonus pass and the draw, for chunks of CS logits.
template <int VEC, int CS>
void launch_tail(const VerifyArgs& a, int B, bool wave_draw, hipStream_t s) {
  launch("verify_decide_bonus", decide_bonus_kernel<VEC, CS>, dim3((unsigned)((size_t)a.C * B)), dim3(kThreads), s, a);
  if (wave_draw) launch("verify_select", select_wave_kernel<VEC, CS>, dim3(B), dim3(kWave), s, a);
  else if (a.gsum) launch("verify_select", select_groups_kernel<VEC, CS>, dim3(B), dim3(kWave), s, a);
  else launch("verify_select", select_kernel<VEC, CS>, dim3(B), dim3(kThreads), s, a);
}

// `packed`: the layout of spec_verify_static, whose scratch array holds one call at a time, so
// the draw-weight region is taken only when this call stores weights.
VerifyLayout layout(int B, int N, int V, bool packed = false) {
  VerifyLayout L{};
  L.RC = row_chunk();
  L.CR = (V + L.RC - 1) / L.RC;
  const int c_small = (V + kChunkSmall - 1) / kChunkSmall;
  const int c_large = (V + kChunkLarge - 1) / kChunkLarge;
  L.CS = (B <= kSmallChunkMaxB && c_small <= kWave) ? kChunkSmall : kChunkLarge;
  L.C = L.CS == kChunkSmall ? c_small : c_large;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off += align_up(bytes, 256); return at; };
  // sized for the smallest chunk, so the size depends on the arguments alone
  L.rowparts = take((size_t)B * N * ((V + kRowChunkMin - 1) / kRowChunkMin) * sizeof(RowPart));
  L.plans = take((size_t)B * sizeof(BonusPlan));
  // the chunk parts and weights regions are sized for either chunking (the more chunks, the
  // longer padded row), so the workspace size grows with B whichever chunk size B selects
  L.bparts = take((size_t)B * c_small * sizeof(BonusPart));
  // Rows of at most 64 chunks are drawn by one wave from the 64-token group sums (measured
  // faster than scanning stored weights at every batch).  Longer rows are drawn by a
  // workgroup, over stored weights for batches up to kStoreWeightsMaxB; the tuning override
  // verify_store_w forces either way.  The weights region is reserved whenever a batch of this
  // vocabulary may store (or the override forces it), so that the workspace size grows with B
  // and a workspace sized for a batch also serves every smaller one.
  L.store_w = tuning(kKnobVerifyStoreW, (L.C > kWave && B <= kStoreWeightsMaxB) ? 1 : 0) != 0;
  const bool reserve_w = packed ? L.store_w : (L.store_w || c_large > kWave);
  L.weights = take(reserve_w ? (size_t)B * c_large * kChunkLarge * sizeof(double) : 0);
  // group sums of the one-wave draw without stored weights (reserved like the weights)
  const size_t groups = std::max((size_t)c_large * (kChunkLarge / 64), (size_t)c_small * (kChunkSmall / 64));
  L.gsum = take(packed && L.store_w ? 0 : (size_t)B * groups * 2 * sizeof(double));
  L.row_list = take((size_t)B * N * sizeof(int32_t));
  L.row_count = take(sizeof(int32_t));
  L.walk = take((size_t)3 * B * N * sizeof(double));
  L.wk = walk_parts(B, N, V);
  // sized for kWalkMaxParts whatever wk is, so that the size grows with B
  L.wsync = take((size_t)B * N * sizeof(int32_t));
  L.wpart = take((size_t)B * N * kWalkMaxParts * 4 * sizeof(double));
  const bool fits = (size_t)B * N <= (size_t)kListMax;
  L.listed = fits && tuning(kKnobVerifyRowsList, (size_t)B * N * L.CR >= kListMinItems ? 1 : 0) != 0;
  L.total = off;
  return L;
}

// Host-checkable arguments of spec_verify and spec_verify_static.
spec_status check_verify(const float* target_logits, const float* draft_probs, const int32_t* draft_row,
                         const int32_t* t2d, const int32_t* tokens, const int32_t* parents,
                         const float* uniforms, int B, int N, int V, int R, int Vd, int max_depth,
                         int mode, float eps, float delta, const int32_t* accept_len,
                         const int32_t* path, const int32_t* bonus_token, const int32_t* err) {
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES || V < 1 || max_depth < 0) return SPEC_EINVAL;
  if (!target_logits || !tokens || !parents || !uniforms || !accept_len || !path || !bonus_token || !err)
    return SPEC_EINVAL;
  if (mode != SPEC_VERIFY_GREEDY && mode != SPEC_VERIFY_TYPICAL && mode != SPEC_VERIFY_REJECT &&
      mode != SPEC_VERIFY_WALK)
    return SPEC_EINVAL;
  if (mode == SPEC_VERIFY_REJECT || mode == SPEC_VERIFY_WALK) {
    if (!draft_probs || !draft_row || R < 1 || Vd < 1) return SPEC_EINVAL;
    if (!t2d && Vd != V) return SPEC_EINVAL;
  }
  if (mode == SPEC_VERIFY_TYPICAL && (!(eps == eps) || !(delta == delta))) return SPEC_EINVAL;
  if (V > kMaxVocab) return SPEC_EUNSUPPORTED;
  const VerifyLayout L = layout(B, N, V);
  if (L.C > kThreads || (size_t)L.CR * N * B > (size_t)INT_MAX) return SPEC_EUNSUPPORTED;
  return SPEC_OK;
}

// The kernels of one verification, with the scratch regions of layout L at `w`.
spec_status run_verify(const float* target_logits, const float* draft_probs, const int32_t* draft_row,
                       const int32_t* t2d, const int32_t* tokens, const int32_t* parents,
                       const int32_t* n_nodes, const float* uniforms, int B, int N, int V, int R, int Vd,
                       int max_depth, int mode, float eps, float delta, int32_t* accept_len,
                       int32_t* path, int32_t* bonus_token, uint8_t* node_accept, int32_t* err,
                       const VerifyLayout& L, char* w, hipStream_t s) {
  VerifyArgs a{};
  a.logits = target_logits; a.draft = draft_probs; a.draft_row = draft_row; a.t2d = t2d;
  a.tokens = tokens; a.parents = parents; a.n_nodes = n_nodes; a.uniforms = uniforms;
  a.B = B; a.N = N; a.V = V; a.R = R; a.Vd = Vd; a.max_depth = max_depth; a.mode = mode;
  a.eps = eps; a.delta = delta; a.accept_len = accept_len; a.path = path; a.bonus = bonus_token;
  a.node_accept = node_accept; a.err = err; a.CR = L.CR; a.RC = L.RC; a.CS = L.CS; a.C = L.C;
  a.rowparts = reinterpret_cast<RowPart*>(w + L.rowparts);
  a.plans = reinterpret_cast<BonusPlan*>(w + L.plans);
  a.bparts = reinterpret_cast<BonusPart*>(w + L.bparts);
  a.weights = L.store_w ? reinterpret_cast<double*>(w + L.weights) : nullptr;
  a.gsum = (!L.store_w && L.C <= kWave) ? reinterpret_cast<double*>(w + L.gsum) : nullptr;
  a.row_list = reinterpret_cast<int32_t*>(w + L.row_list);
  a.row_count = reinterpret_cast<int32_t*>(w + L.row_count);
  a.wc = reinterpret_cast<double*>(w + L.walk);
  a.wf = a.wc + (size_t)B * N;
  a.wend = a.wf + (size_t)B * N;
  a.wk = L.wk;
  a.wspin = std::max(1, tuning(kKnobWalkSpin, kWalkSpinMax));
  const bool split = mode == SPEC_VERIFY_WALK && L.wk > 1;
  a.wsync = split ? reinterpret_cast<int32_t*>(w + L.wsync) : nullptr;
  a.wpart = split ? reinterpret_cast<double*>(w + L.wpart) : nullptr;
  if (!split) a.wk = 1;

  const dim3 blk(kThreads);
  const dim3 grid_rows((unsigned)((size_t)L.CR * N * B));
  // 16-byte loads need rows that start on 16-byte boundaries
  const bool vec4 = V % 4 == 0 && (reinterpret_cast<uintptr_t>(target_logits) & 15) == 0;
  const char* nr = "verify_rows";
  if (L.listed) {
    launch("verify_rows_list", rows_list_kernel, dim3(1), blk, s, a);
    if (L.RC == 16384) {
      if (vec4) launch(nr, rows_listed_kernel<4, 64>, grid_rows, blk, s, a);
      else launch(nr, rows_listed_kernel<1, 64>, grid_rows, blk, s, a);
    } else if (L.RC == 8192) {
      if (vec4) launch(nr, rows_listed_kernel<4, 32>, grid_rows, blk, s, a);
      else launch(nr, rows_listed_kernel<1, 32>, grid_rows, blk, s, a);
    } else {
      if (vec4) launch(nr, rows_listed_kernel<4, 16>, grid_rows, blk, s, a);
      else launch(nr, rows_listed_kernel<1, 16>, grid_rows, blk, s, a);
    }
  } else if (L.RC == 16384) {
    if (vec4) launch(nr, rows_kernel<4, 64>, grid_rows, blk, s, a);
    else launch(nr, rows_kernel<1, 64>, grid_rows, blk, s, a);
  } else if (L.RC == 8192) {
    if (vec4) launch(nr, rows_kernel<4, 32>, grid_rows, blk, s, a);
    else launch(nr, rows_kernel<1, 32>, grid_rows, blk, s, a);
  } else {
    if (vec4) launch(nr, rows_kernel<4, 16>, grid_rows, blk, s, a);
    else launch(nr, rows_kernel<1, 16>, grid_rows, blk, s, a);
  }
  if (mode == SPEC_VERIFY_WALK) {
    // 16-byte draft loads when the draft rows are the target vocabulary and aligned like the logits
    const bool dvec = draft_probs && !t2d && Vd % 4 == 0 && (reinterpret_cast<uintptr_t>(draft_probs) & 15) == 0;
    launch_chain<1024, 8>(a, dim3((unsigned)((size_t)B * N * a.wk)), vec4, dvec, s);
  }
  // the draw: one wave per sequence when the weights are stored and a wave holds the chunks
  const bool wave_draw = a.weights && L.C <= kWave;
  if (vec4) {
    if (L.CS == kChunkSmall) launch_tail<4, kChunkSmall>(a, B, wave_draw, s);
    else launch_tail<4, kChunkLarge>(a, B, wave_draw, s);
  } else {
    if (L.CS == kChunkSmall) launch_tail<1, kChunkSmall>(a, B, wave_draw, s);
    else launch_tail<1, kChunkLarge>(a, B, wave_draw, s);
  }
  return launch_status();
}

// Scratch of spec_verify_static: one fixed array per GPU, held until the process ends.  Host
// code never passes `scratch` itself (its host-side name is a stand-in, not a device address):
// static_scratch() looks up each device's address once, with that device current, and the
// kernels get that address.
constexpr size_t kStaticScratchBytes = SPEC_VERIFY_STATIC_MAX_BYTES;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// This GPU's address of `scratch`; `dev` must be the current device.
spec_status static_scratch(int dev, char** out) {
  if (dev < 0 || dev >= kMaxDevices) return SPEC_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return SPEC_EHIP;
    }
    g_scratch[dev] = p;
  }
  *out = static_cast<char*>(g_scratch[dev]);
  return SPEC_OK;
}

}  // namespace
}  // namespace spectree

using namespace spectree;

extern "C" size_t spec_verify_workspace(int B, int N, int V) {
  if (B < 1 || N < 1 || V < 1 || V > kMaxVocab) return 0;
  return layout(B, N, V).total;
}

extern "C" spec_status spec_verify(const float* target_logits, const float* draft_probs,
                                   const int32_t* draft_row, const int32_t* t2d,
                                   const int32_t* tokens, const int32_t* parents,
                                   const int32_t* n_nodes, const float* uniforms, int B, int N,
                                   int V, int R, int Vd, int max_depth, int mode, float eps,
                                   float delta, int32_t* accept_len, int32_t* path,
                                   int32_t* bonus_token, uint8_t* node_accept, int32_t* err,
                                   void* workspace, size_t ws_bytes, void* stream) {
  const spec_status st = check_verify(target_logits, draft_probs, draft_row, t2d, tokens, parents, uniforms, B, N,
                                      V, R, Vd, max_depth, mode, eps, delta, accept_len, path, bonus_token, err);
  if (st != SPEC_OK) return st;
  const VerifyLayout L = layout(B, N, V);
  if (!workspace || ws_bytes < L.total) return SPEC_EWORKSPACE;
  return run_verify(target_logits, draft_probs, draft_row, t2d, tokens, parents, n_nodes, uniforms, B, N, V, R,
                    Vd, max_depth, mode, eps, delta, accept_len, path, bonus_token, node_accept, err, L,
                    static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
}

extern "C" size_t spec_verify_static_bytes(int B, int N, int V) {
  if (B < 1 || N < 1 || V < 1 || V > kMaxVocab) return 0;
  return layout(B, N, V, true).total;
}

extern "C" spec_status spec_verify_static(const float* target_logits, const float* draft_probs,
                                          const int32_t* draft_row, const int32_t* t2d,
                                          const int32_t* tokens, const int32_t* parents,
                                          const int32_t* n_nodes, const float* uniforms, int B, int N,
                                          int V, int R, int Vd, int max_depth, int mode,
                                          float eps, float delta, int32_t* accept_len, int32_t* path,
                                          int32_t* bonus_token, uint8_t* node_accept, int32_t* err,
                                          void* stream) {
  const spec_status st = check_verify(target_logits, draft_probs, draft_row, t2d, tokens, parents, uniforms, B, N,
                                      V, R, Vd, max_depth, mode, eps, delta, accept_len, path, bonus_token, err);
  if (st != SPEC_OK) return st;
  const VerifyLayout L = layout(B, N, V, true);
  if (L.total > kStaticScratchBytes) return SPEC_ESCRATCH;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int cur = -1, sdev = -1;
  if (hipGetDevice(&cur) != hipSuccess) {
    (void)hipGetLastError();
    return SPEC_EHIP;
  }
  if (s != nullptr) {
    if (hipStreamGetDevice(s, &sdev) != hipSuccess) {
      (void)hipGetLastError();
      return SPEC_EHIP;
    }
    if (sdev != cur) return SPEC_EINVAL;      // the scratch address is the current device's
  }
  char* w = nullptr;
  const spec_status sc = static_scratch(cur, &w);
  if (sc != SPEC_OK) return sc;
  return run_verify(target_logits, draft_probs, draft_row, t2d, tokens, parents, n_nodes, uniforms, B, N, V, R,
                    Vd, max_depth, mode, eps, delta, accept_len, path, bonus_token, node_accept, err, L, w, s);
}
