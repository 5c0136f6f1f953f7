// Verification: per-node acceptance, longest accepted path, bonus token.
//
// Rules: "EAGLE-3とMedusaで実装するSpeculative Decoding実践ガイド", section
// "棄却サンプリング：出力品質を保証する" (accept with probability min(1, T[x]/D[x]); on a reject
// draw from norm(relu(T - D)); drop every candidate after a reject); "Medusa（マルチヘッド
// 投機的デコーディング）", section "Medusa-1とMedusa-2の違い" (typical acceptance against an
// entropy-based threshold); "多トークン予測（Medusa・EAGLE）", section
// "ツリー検証：候補を「木」に束ねて1回で確かめる" (keep the path that passes the longest).
//
// Four kernels, in stream order; no kernel synchronises workgroups (the kernel boundaries
// order their results), and every global load is issued before it is needed.
//   rows    grid (seq, node, chunk): rows of nodes with children are split into chunks of
//           16K logits; each workgroup streams its chunk once (float4 loads held in registers)
//           into (max, lowest argmax, sum exp(x - max), sum exp(x - max)(x - max)), fp32 exp
//           with fp64 sums.  Workgroups of leaf rows leave after a 1 KB look at the parents.
//   decide  one workgroup per sequence, one thread per node: merge of the row chunks,
//           validation, node tests in fp64, survival = AND over the parent chain, the deepest
//           survivor (LDS max on depth, -index), the path, and the plan of the bonus draw.
//   bonus   grid (seq, chunk) over the kept row m: chunk max / argmax, and fp64 chunk sums of
//           exp(x - max) and, for a residual draw, of relu(T - D) with T normalised by the row
//           statistics of the first kernel.
//   select  one workgroup per sequence: the chunk holding u * Z, then an in-order fp64 scan
//           inside it for the smallest token whose running sum exceeds u * Z.
#include <cfloat>
#include <climits>

#include "common.h"

namespace spectree {
namespace {

constexpr int kThreads = 256;
constexpr int kRowChunk = 16384;             // logits per workgroup in the row pass
constexpr int kRowPer = kRowChunk / kThreads;
constexpr int kBonusChunk = 4096;            // logits per workgroup in the bonus pass
constexpr int kPer = kBonusChunk / kThreads;
constexpr int kMaxRowChunks = 8;             // decide merges a row's chunks in batches of 8

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
  int CR;               // row-pass chunks per row (kRowChunk logits each)
  int CS, C;            // bonus-pass chunk size (kBonusChunk) and chunks per row
  RowPart* rowparts;    // [B, N, CR]
  BonusPlan* plans;     // [B]
  BonusPart* bparts;    // [B, C]
};

// ------------------------------------------------------------------ reductions

__device__ __forceinline__ void combine(double& S, double& A, float& m, int& am, double S2, double A2,
                                        float m2, int am2) {
  if (m2 > m || (m2 == m && am2 < am)) {
    const double sc = (m == -INFINITY) ? 0.0 : exp((double)m - (double)m2);
    const double d = (m == -INFINITY) ? 0.0 : (double)m - (double)m2;
    A = sc * (A + d * S) + A2;
    S = sc * S + S2;
    m = m2;
    am = am2;
  } else {
    const double sc = (m2 == -INFINITY) ? 0.0 : exp((double)m2 - (double)m);
    const double d = (m2 == -INFINITY) ? 0.0 : (double)m2 - (double)m;
    A = A + sc * (A2 + d * S2);
    S = S + sc * S2;
  }
}

// Block-wide reduction of (S, A, m, argmax, nonfinite); the result is returned to every thread.
__device__ void block_combine(double& S, double& A, float& m, int& am, int& nf) {
  __shared__ double sS[kThreads / kWave], sA[kThreads / kWave];
  __shared__ float sm[kThreads / kWave];
  __shared__ int sam[kThreads / kWave], snf[kThreads / kWave];
  for (int o = 32; o > 0; o >>= 1) {
    const double S2 = __shfl_xor(S, o), A2 = __shfl_xor(A, o);
    const float m2 = __shfl_xor(m, o);
    const int am2 = __shfl_xor(am, o), nf2 = __shfl_xor(nf, o);
    combine(S, A, m, am, S2, A2, m2, am2);
    nf |= nf2;
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { sS[w] = S; sA[w] = A; sm[w] = m; sam[w] = am; snf[w] = nf; }
  __syncthreads();
  S = sS[0]; A = sA[0]; m = sm[0]; am = sam[0]; nf = snf[0];
  for (int k = 1; k < kThreads / kWave; ++k) {
    combine(S, A, m, am, sS[k], sA[k], sm[k], sam[k]);
    nf |= snf[k];
  }
}

__device__ double block_sum(double v) {
  __shared__ double s[kThreads / kWave];
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = v;
  __syncthreads();
  return s[0] + s[1] + s[2] + s[3];
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

template <int VEC>
__global__ __launch_bounds__(kThreads) void rows_kernel(VerifyArgs a) {
  // 1-D grid over (seq, node, chunk): grid y/z are limited to 65536.
  const int c = blockIdx.x % a.CR;
  const int p = (blockIdx.x / a.CR) % a.N;
  const int b = blockIdx.x / (a.CR * a.N);
  const int t = threadIdx.x;
  const int n = a.n_nodes ? a.n_nodes[b] : a.N;
  if (n < 0 || n > a.N || p >= n) return;
  // only rows of nodes that some node names as its parent are read
  const int named = (t >= 1 && t < n && a.parents[(size_t)b * a.N + t] == p) ? 1 : 0;
  if (!__syncthreads_or(named)) return;

  const float* row = a.logits + ((size_t)b * a.N + p) * a.V;
  const int lo = c * kRowChunk;
  const int hi = min(a.V, lo + kRowChunk);
  float x[kRowPer];
  load_chunk<VEC>(row, lo, hi, x);
  float m = -INFINITY;
  int am = INT_MAX, nf = 0;
#pragma unroll
  for (int k = 0; k < kRowPer; ++k) {
    const int idx = chunk_index<VEC>(lo, k);
    if (idx < hi) {
      nf |= !isfinite(x[k]);
      if (x[k] > m || (x[k] == m && idx < am)) { m = x[k]; am = idx; }
    }
  }
  double S = 0.0, A = 0.0;
  if (m != -INFINITY && !nf) {
#pragma unroll
    for (int k = 0; k < kRowPer; ++k) {
      const float d = x[k] - m;            // -inf past the chunk -> exp 0
      const float ex = __expf(d);
      S += (double)ex;
      A += (ex > 0.f) ? (double)ex * (double)d : 0.0;
    }
  }
  if (am == INT_MAX) m = -INFINITY;
  block_combine(S, A, m, am, nf);
  if (t == 0) a.rowparts[((size_t)b * a.N + p) * a.CR + c] = RowPart{S, A, m, am, nf, 0};
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

__global__ __launch_bounds__(kThreads) void decide_kernel(VerifyArgs a) {
  __shared__ int s_par[SPEC_MAX_NODES];
  __shared__ int s_dep[SPEC_MAX_NODES];
  __shared__ int s_acc[SPEC_MAX_NODES];
  __shared__ int s_has[SPEC_MAX_NODES];
  __shared__ float s_mx[SPEC_MAX_NODES];
  __shared__ int s_am[SPEC_MAX_NODES];
  __shared__ double s_S[SPEC_MAX_NODES];
  __shared__ double s_H[SPEC_MAX_NODES];
  __shared__ int s_err, s_best, s_minchild;
  const int b = blockIdx.x;
  const int c = threadIdx.x;
  const int n = a.n_nodes ? a.n_nodes[b] : a.N;
  if (c == 0) { s_err = INT_MAX; s_best = -1; s_minchild = INT_MAX; }
  if (c < a.N) { s_par[c] = a.parents[(size_t)b * a.N + c]; s_has[c] = 0; s_acc[c] = 0; }
  __syncthreads();
  BonusPlan* plan = a.plans + b;
  if (n < 0 || n > a.N || n == 0) {
    write_neutral(a, b, n == 0 ? 0 : err_word(0, SPEC_ERR_NNODES));
    if (c == 0) *plan = BonusPlan{0, 0, 0, 0.f, 0.0};
    return;
  }

  // rows read: nodes named as a parent by some valid child
  if (c >= 1 && c < n) {
    const int p = s_par[c];
    if (p >= 0 && p < c) s_has[p] = 1;
  }
  __syncthreads();
  // this thread's loads, all issued before any is used: its own token / uniform / draft row,
  // and the chunk partials of its row if it has children
  RowPart q[kMaxRowChunks];
  const bool has = c < n && s_has[c];
  {
    const RowPart* rp = a.rowparts + ((size_t)b * a.N + (has ? c : 0)) * a.CR;
#pragma unroll
    for (int k = 0; k < kMaxRowChunks; ++k) q[k] = rp[k < a.CR ? k : 0];
  }
  int code = 0, depth = 0, tok = -1, drow = -1, dx = -1;
  float u = 0.f;
  if (c < n) {
    const int p = s_par[c];
    if (c == 0) {
      if (p != -1) code = SPEC_ERR_ROOT;
    } else if (p < 0 || p >= c) {
      code = SPEC_ERR_PARENT;
    } else {
      tok = a.tokens[(size_t)b * a.N + c];
      u = a.uniforms[(size_t)b * a.N + c];
      if (a.mode == SPEC_VERIFY_REJECT) drow = a.draft_row[(size_t)b * a.N + c];
      int j = c;
      while (j > 0) {
        const int pj = s_par[j];
        if (pj < 0 || pj >= j) break;
        j = pj;
        ++depth;
      }
      if (depth > a.max_depth) code = SPEC_ERR_DEPTH;
      else if (tok < 0 || tok >= a.V) code = SPEC_ERR_TOKEN;
      if (code == 0 && a.mode == SPEC_VERIFY_REJECT) {
        if (drow < 0 || drow >= a.R) code = SPEC_ERR_DRAFTROW;
        else if (a.t2d) {
          dx = a.t2d[tok];
          if (dx < -1 || dx >= a.Vd) code = SPEC_ERR_MAP;
        } else {
          dx = tok;
        }
      }
    }
    s_dep[c] = depth;
  }

  // ---- statistics of the rows that have children: merge their chunks
  if (has) {
    double S = 0.0, A = 0.0;
    float m = -INFINITY;
    int am = INT_MAX, nf = 0;
#pragma unroll
    for (int k = 0; k < kMaxRowChunks; ++k) {
      if (k >= a.CR) break;
      nf |= q[k].nonfinite;
      combine(S, A, m, am, q[k].S, q[k].A, q[k].m, q[k].argmax);
    }
    // vocabularies beyond kMaxRowChunks * kRowChunk: further batches
    const RowPart* rp = a.rowparts + ((size_t)b * a.N + c) * a.CR;
    for (int k0 = kMaxRowChunks; k0 < a.CR; k0 += kMaxRowChunks) {
#pragma unroll
      for (int k = 0; k < kMaxRowChunks; ++k) q[k] = rp[k0 + k < a.CR ? k0 + k : 0];
#pragma unroll
      for (int k = 0; k < kMaxRowChunks; ++k) {
        if (k0 + k >= a.CR) break;
        nf |= q[k].nonfinite;
        combine(S, A, m, am, q[k].S, q[k].A, q[k].m, q[k].argmax);
      }
    }
    if (nf) atomicMin(&s_err, err_word(c, SPEC_ERR_NONFINITE));
    s_mx[c] = m;
    s_am[c] = am;
    s_S[c] = S;
    s_H[c] = log(S) - A / S;
  }
  if (code) atomicMin(&s_err, err_word(c, code));
  __syncthreads();
  if (s_err != INT_MAX) {
    write_neutral(a, b, s_err);
    if (c == 0) *plan = BonusPlan{0, 0, 0, 0.f, 0.0};
    return;
  }

  // ---- per-node tests (fp64)
  if (c >= 1 && c < n) {
    const int p = s_par[c];
    const float lpx = a.logits[((size_t)b * a.N + p) * a.V + tok];
    const double T = exp((double)lpx - (double)s_mx[p]) / s_S[p];
    bool acc;
    if (a.mode == SPEC_VERIFY_GREEDY) {
      acc = tok == s_am[p];
    } else if (a.mode == SPEC_VERIFY_TYPICAL) {
      const double tau = fmin((double)a.eps, (double)a.delta * exp(-s_H[p]));
      acc = T >= tau;
    } else {
      const double d = dx >= 0 ? (double)a.draft[((size_t)b * a.R + drow) * a.Vd + dx] : 0.0;
      acc = (double)u * d < T;
    }
    s_acc[c] = acc ? 1 : 0;
  }
  if (c == 0) s_acc[0] = 1;
  __syncthreads();

  // ---- survival and the deepest survivor
  if (c < n) {
    bool ok = true;
    int j = c;
    while (j > 0) {
      ok = ok && s_acc[j];
      j = s_par[j];
    }
    if (ok) atomicMax(&s_best, (s_dep[c] << 9) | (511 - c));
  }
  if (c < a.N && a.node_accept) a.node_accept[(size_t)b * a.N + c] = (c < n) ? (uint8_t)s_acc[c] : 0;
  __syncthreads();
  const int m = 511 - (s_best & 511);
  const int dm = s_best >> 9;
  if (c >= 1 && c < n && s_par[c] == m) atomicMin(&s_minchild, c);
  for (int j = c; j <= a.max_depth; j += kThreads)
    if (j > dm) a.path[(size_t)b * (a.max_depth + 1) + j] = -1;
  __syncthreads();
  if (c == 0) {
    int j = m;
    for (int d = dm; d >= 0; --d) {
      a.path[(size_t)b * (a.max_depth + 1) + d] = j;
      j = s_par[j];
    }
    a.accept_len[b] = dm;
    a.err[b] = 0;
    BonusPlan pl{m, 0, 0, 0.f, 0.0};
    if (a.mode == SPEC_VERIFY_GREEDY) {
      if (s_has[m]) a.bonus[b] = s_am[m];
      else pl.kind = 1;
    } else if (a.mode == SPEC_VERIFY_TYPICAL) {
      pl.kind = 2;
    } else if (s_minchild != INT_MAX) {
      pl.kind = 3;
      pl.r = a.draft_row[(size_t)b * a.N + s_minchild];
      pl.M = s_mx[m];
      pl.S = s_S[m];
    } else {
      pl.kind = 2;
    }
    *plan = pl;
  }
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

__global__ __launch_bounds__(kThreads) void bonus_kernel(VerifyArgs a) {
  const int c = blockIdx.x % a.C, b = blockIdx.x / a.C;
  const BonusPlan pl = a.plans[b];
  if (pl.kind == 0) return;
  const float* row = a.logits + ((size_t)b * a.N + pl.m) * a.V;
  const int lo = c * a.CS, hi = min(a.V, lo + a.CS);
  float x[kPer];
  load_chunk<1>(row, lo, hi, x);
  float m = -INFINITY;
  int am = INT_MAX, nf = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int idx = chunk_index<1>(lo, k);
    if (idx < hi) {
      nf |= !isfinite(x[k]);
      if (x[k] > m || (x[k] == m && idx < am)) { m = x[k]; am = idx; }
    }
  }
  double S = 0.0, Q = 0.0, dummy = 0.0;
  if (pl.kind == 3) {
    // exp(x - M) with the row max, and relu(T - D) with T normalised by the row statistics
    m = pl.M;
    double d[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int v = chunk_index<1>(lo, k);
      d[k] = draft_at(a, b, pl.r, v < hi ? v : lo);
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int v = chunk_index<1>(lo, k);
      if (v < hi && !nf) {
        const double e = exp((double)x[k] - (double)m);
        S += e;
        Q += fmax(e / pl.S - d[k], 0.0);
      }
    }
    Q = block_sum(Q);
    S = block_sum(S);
    int nf2 = nf;
    nf = __syncthreads_or(nf2);
  } else {
    block_combine(S, dummy, m, am, nf);    // chunk max / argmax / nonfinite, in every thread
    if (!nf && pl.kind == 2 && m != -INFINITY) {
#pragma unroll
      for (int k = 0; k < kPer; ++k) S += (x[k] == -INFINITY) ? 0.0 : exp((double)x[k] - (double)m);
    }
    S = block_sum(S);
  }
  if (threadIdx.x == 0) a.bparts[(size_t)b * a.C + c] = BonusPart{S, Q, m, am, nf, 0};
}

// Weight of token v for draw `kind`: 2 -> exp(x - M) (T up to the common factor 1/S),
// 3 -> relu(exp(x - M) / S - D[v]).
__device__ __forceinline__ double draw_weight(const VerifyArgs& a, int b, int kind, int r, float x, int v,
                                              float M, double S) {
  const double e = exp((double)x - (double)M);
  if (kind == 2) return e;
  return fmax(e / S - draft_at(a, b, r, v), 0.0);
}

// Smallest token of chunk [lo, hi) whose running sum (from `base`, fp64, ascending token order)
// exceeds thr; -1 if none.  Thread t owns a contiguous run of the chunk.
__device__ int scan_chunk(const VerifyArgs& a, int b, int kind, int r, const float* row, int lo, int hi,
                          float M, double S, double base, double thr) {
  __shared__ double s_pre[kThreads];
  __shared__ int s_hit;
  const int per = (hi - lo + kThreads - 1) / kThreads;   // <= kPer
  const int my_lo = lo + (int)threadIdx.x * per;
  float xv[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int v = my_lo + k;
    const bool in = k < per && v < hi;
    const float val = row[in ? v : lo];
    xv[k] = val;
  }
  double w[kPer];
  double mine = 0.0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int v = my_lo + k;
    w[k] = (k < per && v < hi) ? draw_weight(a, b, kind, r, xv[k], v, M, S) : 0.0;
    mine += w[k];
  }
  __syncthreads();
  if (threadIdx.x == 0) s_hit = INT_MAX;
  s_pre[threadIdx.x] = mine;
  __syncthreads();
  // inclusive scan of the per-thread sums in thread order
  for (int o = 1; o < kThreads; o <<= 1) {
    const double add = (int)threadIdx.x >= o ? s_pre[threadIdx.x - o] : 0.0;
    __syncthreads();
    s_pre[threadIdx.x] += add;
    __syncthreads();
  }
  const double before = base + (threadIdx.x ? s_pre[threadIdx.x - 1] : 0.0);
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

// Chunk holding thr among the fp64 chunk sums q[0..C), and the sum before it.
__device__ int pick_chunk(const double* q, int C, double thr, double& base) {
  double acc = 0.0, acc_last = 0.0;
  int last = 0;
  for (int k = 0; k < C; ++k) {
    if (acc + q[k] > thr) { base = acc; return k; }
    if (q[k] > 0.0) { last = k; acc_last = acc; }
    acc += q[k];
  }
  base = acc_last;                          // rounding put thr past the end
  return last;
}

// Inverse-CDF draw with u = uniforms[b, 0] over the weights of `kind`, given their chunk sums.
__device__ int draw(const VerifyArgs& a, int b, int kind, int r, const float* row, const double* q, float M,
                    double S) {
  __shared__ int s_tok;
  double Z = 0.0;
  for (int k = 0; k < a.C; ++k) Z += q[k];
  const double u = (double)a.uniforms[(size_t)b * a.N];
  const double thr = u * Z;
  double base;
  const int cs = pick_chunk(q, a.C, thr, base);
  const int lo = cs * a.CS, hi = min(a.V, lo + a.CS);
  int tok = scan_chunk(a, b, kind, r, row, lo, hi, M, S, base, thr);
  if (tok < 0) {                            // rounding put thr at the chunk's end
    if (threadIdx.x == 0) {
      s_tok = -1;
      for (int v = hi - 1; v >= lo; --v)
        if (draw_weight(a, b, kind, r, row[v], v, M, S) > 0.0) { s_tok = v; break; }
    }
    __syncthreads();
    tok = s_tok;
  }
  return tok;
}

__global__ __launch_bounds__(kThreads) void select_kernel(VerifyArgs a) {
  __shared__ double s_q[kThreads];
  const int b = blockIdx.x;
  const BonusPlan pl = a.plans[b];
  if (pl.kind == 0) return;
  const int t = threadIdx.x;
  // merge the chunk parts (one per thread)
  double S = 0.0, dummy = 0.0, Qc = 0.0;
  float m = -INFINITY;
  int am = INT_MAX, nf = 0;
  if (t < a.C) {
    const BonusPart bp = a.bparts[(size_t)b * a.C + t];
    S = bp.S; Qc = bp.Q; m = bp.m; am = bp.argmax; nf = bp.nonfinite;
  }
  const double Sc = S;
  const float mc = m;
  block_combine(S, dummy, m, am, nf);
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
    if (t < a.C) s_q[t] = (mc == -INFINITY) ? 0.0 : Sc * exp((double)mc - (double)m);
    __syncthreads();
    tok = draw(a, b, 2, pl.r, row, s_q, m, S);
  } else {
    if (t < a.C) s_q[t] = Qc;
    __syncthreads();
    double Z = 0.0;
    for (int k = 0; k < a.C; ++k) Z += s_q[k];
    if (Z > 0.0) {
      tok = draw(a, b, 3, pl.r, row, s_q, pl.M, pl.S);
    } else {                                // residual of zero mass: draw from T_m
      __syncthreads();
      if (t < a.C) s_q[t] = Sc;             // chunk sums of exp(x - M), M the row max
      __syncthreads();
      tok = draw(a, b, 2, pl.r, row, s_q, pl.M, pl.S);
    }
  }
  if (t == 0) a.bonus[b] = tok;
}

// ------------------------------------------------------------------ host

struct VerifyLayout {
  int CR, CS, C;
  size_t rowparts, plans, bparts, total;
};

VerifyLayout layout(int B, int N, int V) {
  VerifyLayout L{};
  L.CR = (V + kRowChunk - 1) / kRowChunk;
  L.CS = kBonusChunk;
  L.C = (V + L.CS - 1) / L.CS;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off += align_up(bytes, 256); return at; };
  L.rowparts = take((size_t)B * N * L.CR * sizeof(RowPart));
  L.plans = take((size_t)B * sizeof(BonusPlan));
  L.bparts = take((size_t)B * L.C * sizeof(BonusPart));
  L.total = off;
  return L;
}

}  // namespace
}  // namespace spectree

using namespace spectree;

extern "C" size_t spec_verify_workspace(int B, int N, int V) {
  if (B < 1 || N < 1 || V < 1) return 0;
  return layout(B, N, V).total;
}

extern "C" spec_status spec_verify(const float* target_logits, const float* draft_probs,
                                   const int32_t* draft_row, const int32_t* t2d,
                                   const int32_t* tokens, const int32_t* parents,
                                   const int32_t* n_nodes, const float* uniforms, int B, int N,
                                   int V, int R, int Vd, int max_depth, spec_mode mode, float eps,
                                   float delta, int32_t* accept_len, int32_t* path,
                                   int32_t* bonus_token, uint8_t* node_accept, int32_t* err,
                                   void* workspace, size_t ws_bytes, void* stream) {
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES || V < 1 || max_depth < 0) return SPEC_EINVAL;
  if (!target_logits || !tokens || !parents || !uniforms || !accept_len || !path || !bonus_token || !err)
    return SPEC_EINVAL;
  if (mode != SPEC_VERIFY_GREEDY && mode != SPEC_VERIFY_TYPICAL && mode != SPEC_VERIFY_REJECT) return SPEC_EINVAL;
  if (mode == SPEC_VERIFY_REJECT) {
    if (!draft_probs || !draft_row || R < 1 || Vd < 1) return SPEC_EINVAL;
    if (!t2d && Vd != V) return SPEC_EINVAL;
  }
  if (mode == SPEC_VERIFY_TYPICAL && (!(eps == eps) || !(delta == delta))) return SPEC_EINVAL;
  const VerifyLayout L = layout(B, N, V);
  if (L.C > kThreads || (size_t)L.CR * N * B > (size_t)INT_MAX) return SPEC_EUNSUPPORTED;
  if (!workspace || ws_bytes < L.total) return SPEC_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);

  VerifyArgs a{};
  a.logits = target_logits; a.draft = draft_probs; a.draft_row = draft_row; a.t2d = t2d;
  a.tokens = tokens; a.parents = parents; a.n_nodes = n_nodes; a.uniforms = uniforms;
  a.B = B; a.N = N; a.V = V; a.R = R; a.Vd = Vd; a.max_depth = max_depth; a.mode = mode;
  a.eps = eps; a.delta = delta; a.accept_len = accept_len; a.path = path; a.bonus = bonus_token;
  a.node_accept = node_accept; a.err = err; a.CR = L.CR; a.CS = L.CS; a.C = L.C;
  char* w = static_cast<char*>(workspace);
  a.rowparts = reinterpret_cast<RowPart*>(w + L.rowparts);
  a.plans = reinterpret_cast<BonusPlan*>(w + L.plans);
  a.bparts = reinterpret_cast<BonusPart*>(w + L.bparts);

  const dim3 blk(kThreads);
  const dim3 grid_rows((unsigned)((size_t)L.CR * N * B)), grid_chunks((unsigned)((size_t)L.C * B));
  if (V % 4 == 0) launch("verify_rows", rows_kernel<4>, grid_rows, blk, s, a);
  else launch("verify_rows", rows_kernel<1>, grid_rows, blk, s, a);
  launch("verify_decide", decide_kernel, dim3(B), blk, s, a);
  launch("verify_bonus", bonus_kernel, grid_chunks, blk, s, a);
  launch("verify_select", select_kernel, dim3(B), blk, s, a);
  return launch_status();
}
