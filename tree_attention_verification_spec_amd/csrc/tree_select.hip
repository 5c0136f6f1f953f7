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
//      (the root gets key 2, above every value; padding -1, below every value), held in
//      registers: wave shuffles for strides below 64, LDS for strides 64-512, and in-thread
//      swaps for larger ones, so only 10-18 stages of the sort need a barrier;
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
constexpr int kSelLog2Max = 12;                                // log2 of SPEC_MAX_CANDIDATES

// true if (ka, ia) comes before (kb, ib): larger value first, then lower index
__device__ __forceinline__ bool precedes(double ka, int ia, double kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// The value of lane (lane ^ m) for m < 64; m is a constant after unrolling.  Quad permutes
// (DPP) for 1 and 2, the swizzle's bit mode (and 0x1f, xor m, inside 32 lanes) for 4 to 16,
// ds_bpermute for 32.
__device__ __forceinline__ int lane_xor(int v, int m) {
  if (m == 1) return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad 1 0 3 2
  if (m == 2) return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad 2 3 0 1
  if (m == 4) return __builtin_amdgcn_ds_swizzle(v, 0x1F | (4 << 10));
  if (m == 8) return __builtin_amdgcn_ds_swizzle(v, 0x1F | (8 << 10));
  if (m == 16) return __builtin_amdgcn_ds_swizzle(v, 0x1F | (16 << 10));
  return __shfl_xor(v, m);
}
__device__ __forceinline__ double lane_xor(double v, int m) {
  const long long b = __double_as_longlong(v);
  const int lo = lane_xor((int)(b & 0xffffffffll), m);
  const int hi = lane_xor((int)(b >> 32), m);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// One compare-exchange of a bitonic stage seen from one position: (k, i) is this position's
// entry and (ok, oi) its partner's; `lo` says this is the lower position of the pair, `up` that
// the pair's block is sorted in precedence order.  The lower position of an up block (and the
// upper of a down block) takes the entry that comes first.
__device__ __forceinline__ void bitonic_pick(double& k, int& i, double ok, int oi, bool lo, bool up) {
  const bool mine_first = precedes(k, i, ok, oi);
  if ((lo == up) != mine_first) {
    k = ok;
    i = oi;
  }
}

// Both positions of the pair in one thread (strides of 1024 and more): a at the lower one.
__device__ __forceinline__ void bitonic_in_thread(double& ka, int& ia, double& kb, int& ib, bool up) {
  const bool a_first = precedes(ka, ia, kb, ib);
  if (a_first != up) {
    const double tk = ka;
    const int ti = ia;
    ka = kb;
    ia = ib;
    kb = tk;
    ib = ti;
  }
}

__global__ __launch_bounds__(kSelThreads) void tree_select_kernel(
    const int32_t* __restrict__ cand_parents, const float* __restrict__ cand_prob,
    const int32_t* __restrict__ n_cand, const int32_t* __restrict__ cand_tokens,
    const int32_t* __restrict__ cand_row, int C, int N, int32_t* __restrict__ sel,
    int32_t* __restrict__ parents, int32_t* __restrict__ tokens, int32_t* __restrict__ draft_row,
    int32_t* __restrict__ n_nodes, int32_t* __restrict__ err) {
  __shared__ double s_key[SPEC_MAX_CANDIDATES];   // values, then sort exchange buffer 0
  __shared__ double s_key2[SPEC_MAX_CANDIDATES];  // sort exchange buffer 1
  __shared__ short s_idx[SPEC_MAX_CANDIDATES];    // sort exchange, then new index (-1: dropped)
  __shared__ short s_idx2[SPEC_MAX_CANDIDATES];
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

    // ---- 3. bitonic sort over E = 2^ceil(log2 n) positions: the root first, then value desc,
    // index asc; padding (-1) last.  Position r * 1024 + t lives in register slot r of thread t:
    // strides below 64 exchange by wave shuffles, strides of 1024 and more stay inside a thread,
    // the others go through LDS (two buffers in turn: one barrier per stage).
    int E = 1;
    while (E < n) E <<= 1;
    const int R = E > kSelThreads ? E / kSelThreads : 1;
    double key[kSelPer];
    int idx[kSelPer];
#pragma unroll
    for (int r = 0; r < kSelPer; ++r) {
      const int q = r * kSelThreads + t;
      key[r] = q == 0 ? 2.0 : (q < n ? s_key[q] : -1.0);
      idx[r] = q;
    }
    int buf = 0;
    // both loops unrolled, so every stage's stride is a constant: strides 1 and 2 exchange by
    // DPP, 4 to 16 by ds_swizzle, 32 by ds_bpermute
#pragma unroll
    for (int ls = 1; ls <= kSelLog2Max; ++ls) {
      const int size = 1 << ls;
      if (size > E) break;
#pragma unroll
      for (int lt = ls - 1; lt >= 0; --lt) {
        const int stride = 1 << lt;
        if (stride >= kSelThreads) {
          if (stride == kSelThreads) {
            bitonic_in_thread(key[0], idx[0], key[1], idx[1], (0 * kSelThreads & size) == 0);
            if (R == 4) bitonic_in_thread(key[2], idx[2], key[3], idx[3], (2 * kSelThreads & size) == 0);
          } else {
            bitonic_in_thread(key[0], idx[0], key[2], idx[2], (0 * kSelThreads & size) == 0);
            bitonic_in_thread(key[1], idx[1], key[3], idx[3], (1 * kSelThreads & size) == 0);
          }
        } else if (stride >= kWave) {
          double* kb = buf ? s_key2 : s_key;
          short* ib = buf ? s_idx2 : s_idx;
#pragma unroll
          for (int r = 0; r < kSelPer; ++r) {
            if (r < R) {
              kb[r * kSelThreads + t] = key[r];
              ib[r * kSelThreads + t] = (short)idx[r];
            }
          }
          __syncthreads();
#pragma unroll
          for (int r = 0; r < kSelPer; ++r) {
            if (r < R) {
              const int q = r * kSelThreads + t;
              bitonic_pick(key[r], idx[r], kb[q ^ stride], ib[q ^ stride], (q & stride) == 0,
                           (q & size) == 0);
            }
          }
          buf ^= 1;
        } else {
#pragma unroll
          for (int r = 0; r < kSelPer; ++r) {
            if (r < R) {
              const int q = r * kSelThreads + t;
              const double ok = lane_xor(key[r], stride);
              const int oi = lane_xor(idx[r], stride);
              bitonic_pick(key[r], idx[r], ok, oi, (q & stride) == 0, (q & size) == 0);
            }
          }
        }
      }
    }
    if (t < N) s_keep[idx[0]] = 1;           // positions 0 .. N-1 (N <= 256 < 1024: slot 0)
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
