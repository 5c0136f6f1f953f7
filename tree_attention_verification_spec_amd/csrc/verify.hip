// Verification: per-node acceptance, longest accepted path, bonus token.
//
// Rules: "EAGLE-3とMedusaで実装するSpeculative Decoding実践ガイド", section
// "棄却サンプリング：出力品質を保証する" (accept with probability min(1, T[x]/D[x]); on a reject
// draw from norm(relu(T - D)); drop every candidate after a reject); "Medusa（マルチヘッド
// 投機的デコーディング）", section "Medusa-1とMedusa-2の違い" (typical acceptance against an
// entropy-based threshold); "多トークン予測（Medusa・EAGLE）", section
// "ツリー検証：候補を「木」に束ねて1回で確かめる" (keep the path that passes the longest).
//
// Kernels, in stream order:
//   rowstats  grid (chunk, node, seq): for every node that has a child, the vocabulary row is
//             split into chunks; each workgroup streams one chunk once (16-byte loads) and
//             emits (max, lowest argmax, sum exp(x - max), sum exp(x - max) (x - max)).
//             Workgroups of leaf rows leave after a 1 KB look at the parent array.
//   decide    one workgroup per sequence, one thread per node: validation, merge of the chunk
//             statistics, per-node test (fp64), survival = AND over the ancestor chain, the
//             deepest survivor through an LDS max on (depth, -index), the path, and the plan
//             of the bonus draw.
//   bonus_a   grid (chunk, seq): for the winning row m (when its draw needs the row): chunk
//             max / argmax and sum exp(x - chunk max) in fp64.
//   bonus_b   grid (chunk, seq): chunk sums of the distribution to draw from (T_m or the
//             residual relu(T_m - D)), fp64.
//   select    one workgroup per sequence: the chunk that holds u * Z, then an in-order fp64
//             scan inside that chunk for the smallest token whose running sum exceeds u * Z.
#include <cfloat>
#include <climits>

#include "common.h"

namespace spectree {
namespace {

constexpr int kThreads = 256;

struct RowPart {      // statistics of one chunk of one logits row
  double S;           // sum exp(x - m)
  double A;           // sum exp(x - m) * (x - m)
  float m;            // chunk max
  int argmax;         // lowest index of the chunk max
  int nonfinite;
  int pad;
};

struct BonusPlan {
  int m;              // winning node
  int kind;           // 0 done, 1 argmax of row m, 2 draw from T_m, 3 draw from the residual
  int r;              // draft row for the residual
  int pad;
};

struct BonusPart {
  double S;           // sum exp(x - m) over the chunk (fp64)
  double Q;           // chunk sum of the distribution to draw from
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
  int CS, C;          // chunk size (elements) and chunks per row
  RowPart* rowparts;  // [B, N, C]
  BonusPlan* plans;   // [B]
  BonusPart* bparts;  // [B, C]
};

__device__ __forceinline__ void combine(double& S, double& A, float& m, int& am, double S2, double A2,
                                        float m2, int am2) {
  if (m2 > m || (m2 == m && am2 < am)) {
    const double sc = (m == -INFINITY) ? 0.0 : exp((double)m - (double)m2);
    const double d = (double)m - (double)m2;
    A = sc * (A + (m == -INFINITY ? 0.0 : d * S)) + A2;
    S = sc * S + S2;
    m = m2;
    am = am2;
  } else {
    const double sc = (m2 == -INFINITY) ? 0.0 : exp((double)m2 - (double)m);
    const double d = (double)m2 - (double)m;
    A = A + sc * (A2 + (m2 == -INFINITY ? 0.0 : d * S2));
    S = S + sc * S2;
  }
}

// Block-wide reduction of (S, A, m, argmax, nonfinite); result valid in thread 0.
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
  if ((threadIdx.x & 63) == 0) { sS[w] = S; sA[w] = A; sm[w] = m; sam[w] = am; snf[w] = nf; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < kThreads / kWave; ++k) {
      combine(S, A, m, am, sS[k], sA[k], sm[k], sam[k]);
      nf |= snf[k];
    }
  }
}

__device__ __forceinline__ bool is_internal(const VerifyArgs& a, int b, int p, int n) {
  const int t = threadIdx.x;
  const int has = (t >= 1 && t < n && a.parents[(size_t)b * a.N + t] == p) ? 1 : 0;
  return __syncthreads_or(has) != 0;
}

template <int VEC>
__global__ __launch_bounds__(kThreads) void rowstats_kernel(VerifyArgs a) {
  // 1-D grid over (seq, node, chunk): grid y/z are limited to 65536.
  const int c = blockIdx.x % a.C;
  const int p = (blockIdx.x / a.C) % a.N;
  const int b = blockIdx.x / (a.C * a.N);
  const int n = a.n_nodes ? a.n_nodes[b] : a.N;
  if (n < 0 || n > a.N || p >= n) return;
  if (!is_internal(a, b, p, n)) return;
  const float* row = a.logits + ((size_t)b * a.N + p) * a.V;
  const int lo = c * a.CS;
  const int hi = min(a.V, lo + a.CS);
  constexpr int PER = 8192 / kThreads / VEC;   // max loads per thread (CS <= 8192)
  float x[PER][VEC];
  float m = -INFINITY;
  int am = INT_MAX, nf = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int base = lo + (k * kThreads + threadIdx.x) * VEC;
    if (VEC == 4 && base + 3 < hi) {
      const float4 v4 = *reinterpret_cast<const float4*>(row + base);
      x[k][0] = v4.x; x[k][VEC > 1 ? 1 : 0] = v4.y; x[k][VEC > 2 ? 2 : 0] = v4.z; x[k][VEC > 3 ? 3 : 0] = v4.w;
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) x[k][e] = (base + e < hi) ? row[base + e] : -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int idx = base + e;
      if (idx < hi) {
        const float v = x[k][e];
        nf |= !isfinite(v);
        if (v > m || (v == m && idx < am)) { m = v; am = idx; }
      }
    }
  }
  float s = 0.f, acc = 0.f;
  if (m != -INFINITY && !nf) {
#pragma unroll
    for (int k = 0; k < PER; ++k)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float d = x[k][e] - m;       // -inf outside the chunk -> exp 0
        const float ex = __expf(d);
        s += ex;
        acc += (ex > 0.f) ? ex * d : 0.f;
      }
  }
  double S = s, A = acc;
  if (am == INT_MAX) m = -INFINITY;
  block_combine(S, A, m, am, nf);
  if (threadIdx.x == 0) {
    RowPart rp;
    rp.S = S; rp.A = A; rp.m = m; rp.argmax = am; rp.nonfinite = nf; rp.pad = 0;
    a.rowparts[((size_t)b * a.N + p) * a.C + c] = rp;
  }
}

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
    if (c == 0) *plan = BonusPlan{0, 0, 0, 0};
    return;
  }

  // ---- structural checks
  int code = 0, depth = 0, tok = -1, drow = -1;
  if (c < n) {
    const int p = s_par[c];
    if (c == 0) {
      if (p != -1) code = SPEC_ERR_ROOT;
    } else if (p < 0 || p >= c) {
      code = SPEC_ERR_PARENT;
    } else {
      int j = c;
      while (j > 0) {
        const int pj = s_par[j];
        if (pj < 0 || pj >= j) break;
        j = pj;
        ++depth;
      }
      tok = a.tokens[(size_t)b * a.N + c];
      if (depth > a.max_depth) code = SPEC_ERR_DEPTH;
      else if (tok < 0 || tok >= a.V) code = SPEC_ERR_TOKEN;
      if (code == 0 && a.mode == SPEC_VERIFY_REJECT) {
        drow = a.draft_row[(size_t)b * a.N + c];
        if (drow < 0 || drow >= a.R) code = SPEC_ERR_DRAFTROW;
        else if (a.t2d) {
          const int dx = a.t2d[tok];
          if (dx < -1 || dx >= a.Vd) code = SPEC_ERR_MAP;
        }
      }
      s_has[p] = 1;
    }
    s_dep[c] = depth;
  }
  __syncthreads();

  // ---- statistics of rows that have children
  if (c < n && s_has[c]) {
    double S = 0.0, A = 0.0;
    float m = -INFINITY;
    int am = INT_MAX, nf = 0;
    const RowPart* rp = a.rowparts + ((size_t)b * a.N + c) * a.C;
    for (int k = 0; k < a.C; ++k) {
      const RowPart q = rp[k];
      nf |= q.nonfinite;
      combine(S, A, m, am, q.S, q.A, q.m, q.argmax);
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
    if (c == 0) *plan = BonusPlan{0, 0, 0, 0};
    return;
  }

  // ---- per-node tests
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
      double d;
      if (a.t2d) {
        const int dx = a.t2d[tok];
        d = dx >= 0 ? (double)a.draft[((size_t)b * a.R + drow) * a.Vd + dx] : 0.0;
      } else {
        d = (double)a.draft[((size_t)b * a.R + drow) * a.Vd + tok];
      }
      const double u = (double)a.uniforms[(size_t)b * a.N + c];
      acc = u * d < T;
    }
    s_acc[c] = acc ? 1 : 0;
  }
  if (c == 0) s_acc[0] = 1;
  __syncthreads();

  // ---- survival (AND over the chain below the root) and the deepest survivor
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
    BonusPlan pl{m, 0, 0, 0};
    if (a.mode == SPEC_VERIFY_GREEDY) {
      if (s_has[m]) a.bonus[b] = s_am[m];
      else pl.kind = 1;
    } else if (a.mode == SPEC_VERIFY_TYPICAL) {
      pl.kind = 2;
    } else if (s_minchild != INT_MAX) {
      pl.kind = 3;
      pl.r = a.draft_row[(size_t)b * a.N + s_minchild];
    } else {
      pl.kind = 2;
    }
    *plan = pl;
  }
}

__global__ __launch_bounds__(kThreads) void bonus_a_kernel(VerifyArgs a) {
  const int c = blockIdx.x % a.C, b = blockIdx.x / a.C;
  const BonusPlan pl = a.plans[b];
  if (pl.kind == 0) return;
  const float* row = a.logits + ((size_t)b * a.N + pl.m) * a.V;
  const int lo = c * a.CS, hi = min(a.V, lo + a.CS);
  float m = -INFINITY;
  int am = INT_MAX, nf = 0;
  for (int v = lo + threadIdx.x; v < hi; v += kThreads) {
    const float x = row[v];
    nf |= !isfinite(x);
    if (x > m || (x == m && v < am)) { m = x; am = v; }
  }
  // chunk max first, then fp64 sum of exp(x - chunk max)
  __shared__ float s_m[kThreads / kWave];
  __shared__ int s_am[kThreads / kWave], s_nf[kThreads / kWave];
  __shared__ double s_S[kThreads / kWave];
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o);
    const int am2 = __shfl_xor(am, o), nf2 = __shfl_xor(nf, o);
    if (m2 > m || (m2 == m && am2 < am)) { m = m2; am = am2; }
    nf |= nf2;
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { s_m[w] = m; s_am[w] = am; s_nf[w] = nf; }
  __syncthreads();
  m = s_m[0]; am = s_am[0]; nf = s_nf[0];
  for (int k = 1; k < kThreads / kWave; ++k) {
    if (s_m[k] > m || (s_m[k] == m && s_am[k] < am)) { m = s_m[k]; am = s_am[k]; }
    nf |= s_nf[k];
  }
  double S = 0.0;
  if (!nf && pl.kind != 1)
    for (int v = lo + threadIdx.x; v < hi; v += kThreads) S += exp((double)row[v] - (double)m);
  S = wave_sum(S);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_S[w] = S;
  __syncthreads();
  if (threadIdx.x == 0) {
    BonusPart bp;
    bp.S = s_S[0] + s_S[1] + s_S[2] + s_S[3];
    bp.Q = 0.0; bp.m = m; bp.argmax = am; bp.nonfinite = nf; bp.pad = 0;
    a.bparts[(size_t)b * a.C + c] = bp;
  }
}

// Merge the chunk statistics of row m: global max, lowest argmax, fp64 normaliser.
__device__ void row_totals(const VerifyArgs& a, int b, float& M, int& am, double& S, int& nf) {
  M = -INFINITY; am = INT_MAX; nf = 0;
  for (int k = 0; k < a.C; ++k) {
    const BonusPart bp = a.bparts[(size_t)b * a.C + k];
    nf |= bp.nonfinite;
    if (bp.m > M || (bp.m == M && bp.argmax < am)) { M = bp.m; am = bp.argmax; }
  }
  S = 0.0;
  for (int k = 0; k < a.C; ++k) {
    const BonusPart bp = a.bparts[(size_t)b * a.C + k];
    S += bp.S * exp((double)bp.m - (double)M);
  }
}

// Probability of token v under the draw of plan `kind` (2: T_m, 3: relu(T_m - D)).
__device__ __forceinline__ double draw_weight(const VerifyArgs& a, int b, int kind, int r, const float* row,
                                              int v, float M, double S) {
  const double t = exp((double)row[v] - (double)M) / S;
  if (kind == 2) return t;
  double d;
  if (a.t2d) {
    // Only candidate tokens' entries are validated; any other entry outside [0, Vd) reads as
    // "not in the draft vocabulary".
    const int dx = a.t2d[v];
    d = (dx >= 0 && dx < a.Vd) ? (double)a.draft[((size_t)b * a.R + r) * a.Vd + dx] : 0.0;
  } else {
    d = (double)a.draft[((size_t)b * a.R + r) * a.Vd + v];
  }
  return fmax(t - d, 0.0);
}

__global__ __launch_bounds__(kThreads) void bonus_b_kernel(VerifyArgs a) {
  const int c = blockIdx.x % a.C, b = blockIdx.x / a.C;
  const BonusPlan pl = a.plans[b];
  if (pl.kind != 2 && pl.kind != 3) return;
  float M; int am, nf; double S;
  row_totals(a, b, M, am, S, nf);
  if (nf) return;
  const float* row = a.logits + ((size_t)b * a.N + pl.m) * a.V;
  const int lo = c * a.CS, hi = min(a.V, lo + a.CS);
  double q = 0.0;
  for (int v = lo + threadIdx.x; v < hi; v += kThreads) q += draw_weight(a, b, pl.kind, pl.r, row, v, M, S);
  q = wave_sum(q);
  __shared__ double s_q[kThreads / kWave];
  if ((threadIdx.x & 63) == 0) s_q[threadIdx.x >> 6] = q;
  __syncthreads();
  if (threadIdx.x == 0) a.bparts[(size_t)b * a.C + c].Q = s_q[0] + s_q[1] + s_q[2] + s_q[3];
}

// In-order inclusive scan (fp64) over one chunk with the whole block; returns in every thread
// the smallest token of [lo, hi) whose running sum from `base` exceeds thr, or -1.
__device__ int scan_chunk(const VerifyArgs& a, int b, int kind, int r, const float* row, int lo, int hi,
                          float M, double S, double base, double thr, double& chunk_total) {
  __shared__ double s_tot[kThreads];
  __shared__ int s_hit;
  const int per = (hi - lo + kThreads - 1) / kThreads;
  const int my_lo = lo + threadIdx.x * per;
  const int my_hi = min(hi, my_lo + per);
  double mine = 0.0;
  for (int v = my_lo; v < my_hi; ++v) mine += draw_weight(a, b, kind, r, row, v, M, S);
  s_tot[threadIdx.x] = mine;
  if (threadIdx.x == 0) s_hit = INT_MAX;
  __syncthreads();
  double before = base;
  for (int k = 0; k < (int)threadIdx.x; ++k) before += s_tot[k];
  if (before + mine > thr) {
    double run = before;
    for (int v = my_lo; v < my_hi; ++v) {
      const double w = draw_weight(a, b, kind, r, row, v, M, S);
      run += w;
      if (run > thr) { atomicMin(&s_hit, v); break; }
    }
  }
  __syncthreads();
  double tot = 0.0;
  for (int k = 0; k < kThreads; ++k) tot += s_tot[k];
  chunk_total = tot;
  const int hit = s_hit;
  __syncthreads();
  return hit == INT_MAX ? -1 : hit;
}

__global__ __launch_bounds__(kThreads) void select_kernel(VerifyArgs a) {
  const int b = blockIdx.x;
  const BonusPlan pl = a.plans[b];
  if (pl.kind == 0) return;
  float M; int am, nf; double S;
  row_totals(a, b, M, am, S, nf);
  if (nf) {
    write_neutral(a, b, err_word(pl.m, SPEC_ERR_NONFINITE));
    return;
  }
  if (pl.kind == 1) {
    if (threadIdx.x == 0) a.bonus[b] = am;
    return;
  }
  const float* row = a.logits + ((size_t)b * a.N + pl.m) * a.V;
  const double u = (double)a.uniforms[(size_t)b * a.N];
  int kind = pl.kind;
  double Z = 0.0;
  for (int k = 0; k < a.C; ++k) Z += a.bparts[(size_t)b * a.C + k].Q;
  int tok = -1;
  if (kind == 3 && !(Z > 0.0)) kind = 2;   // residual of zero mass: draw from T_m
  if (kind == pl.kind) {
    const double thr = u * Z;
    double base = 0.0, base_last = 0.0;
    int cstar = -1, last = 0;
    for (int k = 0; k < a.C; ++k) {
      const double q = a.bparts[(size_t)b * a.C + k].Q;
      if (base + q > thr) { cstar = k; break; }
      if (q > 0.0) { last = k; base_last = base; }
      base += q;
    }
    if (cstar < 0) { cstar = last; base = base_last; }   // rounding put u * Z past the end
    double tot;
    const int lo = cstar * a.CS, hi = min(a.V, lo + a.CS);
    tok = scan_chunk(a, b, kind, pl.r, row, lo, hi, M, S, base, thr, tot);
    if (tok < 0) {                          // rounding put u * Z at the chunk's end
      for (int v = hi - 1; v >= lo; --v)
        if (draw_weight(a, b, kind, pl.r, row, v, M, S) > 0.0) { tok = v; break; }
    }
  } else {
    // Degenerate residual: chunk by chunk over T_m until the running sum passes u * Z_T.
    double ZT = 0.0, tot = 0.0;
    for (int k = 0; k < a.C; ++k) {
      const int lo = k * a.CS, hi = min(a.V, lo + a.CS);
      scan_chunk(a, b, 2, pl.r, row, lo, hi, M, S, 0.0, INFINITY, tot);
      ZT += tot;
    }
    const double thr = u * ZT;
    double base = 0.0;
    for (int k = 0; k < a.C && tok < 0; ++k) {
      const int lo = k * a.CS, hi = min(a.V, lo + a.CS);
      tok = scan_chunk(a, b, 2, pl.r, row, lo, hi, M, S, base, thr, tot);
      base += tot;
    }
    if (tok < 0) tok = am;
  }
  if (threadIdx.x == 0) a.bonus[b] = tok;
}

int chunk_size(int B, int N) { return (long)B * N >= 512 ? 8192 : 4096; }

struct VerifyLayout {
  int CS, C;
  size_t rowparts, plans, bparts, total;
};

VerifyLayout layout(int B, int N, int V) {
  VerifyLayout L{};
  L.CS = chunk_size(B, N);
  L.C = (V + L.CS - 1) / L.CS;
  size_t off = 0;
  L.rowparts = off; off += align_up((size_t)B * N * L.C * sizeof(RowPart), 256);
  L.plans = off;    off += align_up((size_t)B * sizeof(BonusPlan), 256);
  L.bparts = off;   off += align_up((size_t)B * L.C * sizeof(BonusPart), 256);
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
  if ((size_t)L.C * N * B > (size_t)INT_MAX) return SPEC_EINVAL;
  if (!workspace || ws_bytes < L.total) return SPEC_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);

  VerifyArgs a{};
  a.logits = target_logits; a.draft = draft_probs; a.draft_row = draft_row; a.t2d = t2d;
  a.tokens = tokens; a.parents = parents; a.n_nodes = n_nodes; a.uniforms = uniforms;
  a.B = B; a.N = N; a.V = V; a.R = R; a.Vd = Vd; a.max_depth = max_depth; a.mode = mode;
  a.eps = eps; a.delta = delta; a.accept_len = accept_len; a.path = path; a.bonus = bonus_token;
  a.node_accept = node_accept; a.err = err; a.CS = L.CS; a.C = L.C;
  char* w = static_cast<char*>(workspace);
  a.rowparts = reinterpret_cast<RowPart*>(w + L.rowparts);
  a.plans = reinterpret_cast<BonusPlan*>(w + L.plans);
  a.bparts = reinterpret_cast<BonusPart*>(w + L.bparts);

  const dim3 blk(kThreads);
  const dim3 grid_rows((unsigned)((size_t)L.C * N * B)), grid_chunks((unsigned)((size_t)L.C * B));
  if (V % 4 == 0) launch("verify_rowstats", rowstats_kernel<4>, grid_rows, blk, s, a);
  else launch("verify_rowstats", rowstats_kernel<1>, grid_rows, blk, s, a);
  launch("verify_decide", decide_kernel, dim3(B), blk, s, a);
  launch("verify_bonus_a", bonus_a_kernel, grid_chunks, blk, s, a);
  launch("verify_bonus_b", bonus_b_kernel, grid_chunks, blk, s, a);
  launch("verify_select", select_kernel, dim3(B), blk, s, a);
  return launch_status();
}
