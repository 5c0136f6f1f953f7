// Dynamic candidate-tree selection: keep the best N-node subtree of a drafted candidate tree.
//
// "多トークン予測（Medusa・EAGLE）", section "ツリー検証：候補を「木」に束ねて1回で確かめる": a
// larger tree raises the expected accepted length but costs verification work, and EAGLE-2's
// dynamic tree shapes the tree by the context's confidence.  "Medusa（マルチヘッド投機的
// デコーディング）", section "EAGLE: Medusaの発展形", and "EAGLE-3とMedusaで実装するSpeculative
// Decoding実践ガイド", section "EAGLE-1/2からの進化", name the same context-aware tree.
//
// A candidate's value is the product of its draft probabilities along the path from the root,
// multiplied root first in fp64 (the root counts 1).  The root and the N - 1 other candidates of
// largest value are kept, ties to the lower index; with every probability in [0, 1] a parent
// never ranks below its child, so the kept set is a tree.  It is written in candidate order
// (topological) with renumbered parents.
//
// One 1024-thread workgroup per sequence, candidates in LDS (C <= 4096):
//   1. load and validate (error words reduced with an LDS atomicMin: smallest (node, code) wins);
//   2. values level by level: a candidate whose parent's value is known takes parent * p; one
//      round per tree level, two barriers per round (reads, then writes);
//   3. a bitonic sort of (value desc, index asc) over the candidates padded to a power of two
//      (the root gets key 2, above every value; padding -1, below every value);
//   4. the first N sorted entries are flagged, a block scan over the flags in candidate order
//      numbers the kept candidates, and threads j < N write output node j.
// Pools that already fit (n_cand <= N) keep everything and skip steps 2-3.
#include <climits>

#include "common.h"

namespace spectree {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelPer = SPEC_MAX_CANDIDATES / kSelThreads;  // candidates per thread

// true if (ka, ia) comes before (kb, ib): larger value first, then lower index
__device__ __forceinline__ bool precedes(double ka, int ia, double kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__global__ __launch_bounds__(kSelThreads) void tree_select_kernel(
    const int32_t* __restrict__ cand_parents, const float* __restrict__ cand_prob,
    const int32_t* __restrict__ n_cand, const int32_t* __restrict__ cand_tokens,
    const int32_t* __restrict__ cand_row, int C, int N, int32_t* __restrict__ sel,
    int32_t* __restrict__ parents, int32_t* __restrict__ tokens, int32_t* __restrict__ draft_row,
    int32_t* __restrict__ n_nodes, int32_t* __restrict__ err) {
  __shared__ double s_key[SPEC_MAX_CANDIDATES];   // values, then sort keys
  __shared__ short s_idx[SPEC_MAX_CANDIDATES];    // sort payload, then new index (-1: dropped)
  __shared__ short s_par[SPEC_MAX_CANDIDATES];
  __shared__ unsigned char s_keep[SPEC_MAX_CANDIDATES];
  __shared__ int s_sel[SPEC_MAX_NODES];
  __shared__ int s_wsum[kSelWaves];
  __shared__ int s_err;
  const int b = blockIdx.x;
  const int t = threadIdx.x, lane = t & (kWave - 1), wv = t >> 6;
  const int n_raw = n_cand ? n_cand[b] : C;
  const bool bad_n = n_raw < 0 || n_raw > C;
  const int n = bad_n ? 0 : n_raw;
  const size_t base = (size_t)b * C;
  if (t == 0) s_err = INT_MAX;
  __syncthreads();

  // ---- 1. load and validate (candidate i = t + k * 1024: coalesced)
  float pr[kSelPer];
#pragma unroll
  for (int k = 0; k < kSelPer; ++k) {
    const int i = t + k * kSelThreads;
    pr[k] = 0.f;
    if (i < n) {
      const int p = cand_parents[base + i];
      const float q = cand_prob[base + i];
      int code = 0;
      if (i == 0) {
        if (p != -1) code = SPEC_ERR_ROOT;
      } else if (p < 0 || p >= i) {
        code = SPEC_ERR_PARENT;
      } else if (!(q >= 0.f && q <= 1.f)) {   // NaN fails both comparisons
        code = SPEC_ERR_PROB;
      }
      if (code) atomicMin(&s_err, err_word(i, code));
      s_par[i] = (short)((code || i == 0) ? 0 : p);
      s_key[i] = (i == 0) ? 1.0 : -1.0;         // -1: value not known yet
      s_keep[i] = 0;
      pr[k] = q;
    }
  }
  __syncthreads();
  const int e = bad_n ? err_word(0, SPEC_ERR_NNODES) : (s_err == INT_MAX ? 0 : s_err);
  const int kept = e ? 0 : min(n, N);
  const size_t obase = (size_t)b * N;
  if (kept == 0) {
    for (int j = t; j < N; j += kSelThreads) {
      sel[obase + j] = -1;
      parents[obase + j] = -1;
      if (tokens) tokens[obase + j] = -1;
      if (draft_row) draft_row[obase + j] = -1;
    }
    if (t == 0) {
      n_nodes[b] = 0;
      err[b] = e;
    }
    return;
  }

  if (n <= N) {
#pragma unroll
    for (int k = 0; k < kSelPer; ++k) {
      const int i = t + k * kSelThreads;
      if (i < n) s_keep[i] = 1;
    }
  } else {
    // ---- 2. values, one tree level per round (every parent index is below its child's, so
    // round r settles every candidate of depth r; at most n - 1 rounds)
    for (;;) {
      double nv[kSelPer];
      bool upd[kSelPer];
      int pending = 0;
#pragma unroll
      for (int k = 0; k < kSelPer; ++k) {
        const int i = t + k * kSelThreads;
        upd[k] = false;
        nv[k] = 0.0;
        if (i > 0 && i < n && s_key[i] < 0.0) {
          const double pv = s_key[s_par[i]];
          if (pv >= 0.0) {
            nv[k] = pv * (double)pr[k];
            upd[k] = true;
          } else {
            pending = 1;
          }
        }
      }
      const int more = __syncthreads_or(pending);
#pragma unroll
      for (int k = 0; k < kSelPer; ++k)
        if (upd[k]) s_key[t + k * kSelThreads] = nv[k];
      __syncthreads();
      if (!more) break;
    }

    // ---- 3. bitonic sort over E = 2^ceil(log2 n) entries: the root first, then value desc,
    // index asc; padding (-1) last
    int E = 1;
    while (E < n) E <<= 1;
#pragma unroll
    for (int k = 0; k < kSelPer; ++k) {
      const int i = t + k * kSelThreads;
      if (i < E) {
        if (i == 0) s_key[0] = 2.0;
        else if (i >= n) s_key[i] = -1.0;
        s_idx[i] = (short)i;
      }
    }
    __syncthreads();
    for (int size = 2; size <= E; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int q = t; q < (E >> 1); q += kSelThreads) {
          const int lo = 2 * q - (q & (stride - 1));
          const int hi = lo + stride;
          const double ka = s_key[lo], kb = s_key[hi];
          const int ia = s_idx[lo], ib = s_idx[hi];
          const bool up = (lo & size) == 0;
          const bool swap = up ? precedes(kb, ib, ka, ia) : precedes(ka, ia, kb, ib);
          if (swap) {
            s_key[lo] = kb;
            s_key[hi] = ka;
            s_idx[lo] = (short)ib;
            s_idx[hi] = (short)ia;
          }
        }
        __syncthreads();
      }
    }
    for (int r = t; r < N; r += kSelThreads) s_keep[s_idx[r]] = 1;
  }
  __syncthreads();

  // ---- 4. number the kept candidates in candidate order: thread t owns 4t .. 4t+3
  int cnt = 0;
#pragma unroll
  for (int k = 0; k < kSelPer; ++k) {
    const int i = kSelPer * t + k;
    cnt += (i < n && s_keep[i]) ? 1 : 0;
  }
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) s_wsum[wv] = incl;
  __syncthreads();
  int off = incl - cnt;
  for (int q = 0; q < wv; ++q) off += s_wsum[q];
#pragma unroll
  for (int k = 0; k < kSelPer; ++k) {
    const int i = kSelPer * t + k;
    if (i < n) {
      const bool keep = s_keep[i];
      s_idx[i] = (short)(keep ? off : -1);
      if (keep) s_sel[off] = i;
      off += keep ? 1 : 0;
    }
  }
  __syncthreads();
  for (int j = t; j < N; j += kSelThreads) {
    int c = -1, p = -1, tok = -1, row = -1;
    if (j < kept) {
      c = s_sel[j];
      p = c == 0 ? -1 : s_idx[s_par[c]];
      if (cand_tokens) tok = cand_tokens[base + c];
      if (cand_row) row = cand_row[base + c];
    }
    sel[obase + j] = c;
    parents[obase + j] = p;
    if (tokens) tokens[obase + j] = tok;
    if (draft_row) draft_row[obase + j] = row;
  }
  if (t == 0) {
    n_nodes[b] = kept;
    err[b] = 0;
  }
}

}  // namespace
}  // namespace spectree

using namespace spectree;

extern "C" spec_status spec_tree_select(const int32_t* cand_parents, const float* cand_prob,
                                        const int32_t* n_cand, const int32_t* cand_tokens,
                                        const int32_t* cand_row, int B, int C, int N,
                                        int32_t* sel, int32_t* parents, int32_t* tokens,
                                        int32_t* draft_row, int32_t* n_nodes, int32_t* err,
                                        void* stream) {
  if (B < 1 || C < 1 || C > SPEC_MAX_CANDIDATES || N < 1 || N > SPEC_MAX_NODES) return SPEC_EINVAL;
  if (!cand_parents || !cand_prob || !sel || !parents || !n_nodes || !err) return SPEC_EINVAL;
  if ((cand_tokens == nullptr) != (tokens == nullptr)) return SPEC_EINVAL;
  if ((cand_row == nullptr) != (draft_row == nullptr)) return SPEC_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch("tree_select", tree_select_kernel, dim3(B), dim3(kSelThreads), s, cand_parents, cand_prob,
         n_cand, cand_tokens, cand_row, C, N, sel, parents, tokens, draft_row, n_nodes, err);
  return launch_status();
}
