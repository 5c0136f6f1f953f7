// Candidate-tree kernels: ancestor mask / depths / positions, and Medusa tree assembly.
//
// Ancestor-only visibility: "多トークン予測（Medusa・EAGLE）", section
// "ツリー検証：候補を「木」に束ねて1回で確かめる"; "EAGLE-3とMedusaで実装するSpeculative
// Decoding実践ガイド", section "Tree Attention：候補を木構造で探索する".  Assembly from per-head
// candidates: "Medusa（マルチヘッド投機的デコーディング）", section "ツリー構造の候補構築".
//
// One workgroup per sequence, one thread per node (N <= 256).  The parent array sits in LDS;
// each thread climbs from its node to the root, OR-ing one bit per node met into up to four
// 64-bit words held in registers.  Error words are reduced with an LDS atomicMin, so the
// smallest (node, code) pair wins.
#include <climits>

#include "common.h"

namespace spectree {
namespace {

__device__ __forceinline__ void set_bit(int j, uint64_t& w0, uint64_t& w1, uint64_t& w2,
                                        uint64_t& w3) {
  const uint64_t bit = 1ull << (j & 63);
  const int w = j >> 6;
  w0 |= (w == 0) ? bit : 0ull;
  w1 |= (w == 1) ? bit : 0ull;
  w2 |= (w == 2) ? bit : 0ull;
  w3 |= (w == 3) ? bit : 0ull;
}

__global__ __launch_bounds__(SPEC_MAX_NODES) void tree_build_kernel(
    const int32_t* __restrict__ parents, const int32_t* __restrict__ depths_in,
    const int32_t* __restrict__ prefix_len, const int32_t* __restrict__ n_nodes, int N, int W,
    uint64_t* __restrict__ mask, int32_t* __restrict__ positions, int32_t* __restrict__ depths,
    int32_t* __restrict__ err) {
  __shared__ int s_par[SPEC_MAX_NODES];
  __shared__ int s_err;
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  const int n = n_nodes ? n_nodes[b] : N;
  const int P = prefix_len ? prefix_len[b] : 0;
  if (i == 0) s_err = INT_MAX;
  if (i < N) s_par[i] = parents[(size_t)b * N + i];
  __syncthreads();

  int seq_err = 0;
  if (n < 0 || n > N) seq_err = err_word(0, SPEC_ERR_NNODES);
  else if (P < 0) seq_err = err_word(0, SPEC_ERR_PREFIX);

  uint64_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
  int depth = -1;
  if (seq_err == 0 && i < n) {
    int code = 0;
    const int p = s_par[i];
    if (i == 0) {
      if (p != -1) code = SPEC_ERR_ROOT;
    } else if (p < 0 || p >= i) {
      code = SPEC_ERR_PARENT;
    }
    if (code == 0) {
      int j = i;
      depth = 0;
      set_bit(j, w0, w1, w2, w3);
      while (j > 0) {
        const int pj = s_par[j];
        if (pj < 0 || pj >= j) break;  // a broken link is reported at that (smaller) node
        set_bit(pj, w0, w1, w2, w3);
        j = pj;
        ++depth;
      }
      if (depths_in && depths_in[(size_t)b * N + i] != depth) code = SPEC_ERR_DEPTH;
    }
    if (code) atomicMin(&s_err, err_word(i, code));
  }
  __syncthreads();

  const int e = seq_err ? seq_err : (s_err == INT_MAX ? 0 : s_err);
  if (i == 0) err[b] = e;
  if (i < N) {
    const bool ok = (e == 0) && (i < n);
    const size_t row = (size_t)b * N + i;
    uint64_t* m = mask + row * W;
    m[0] = ok ? w0 : 0ull;
    if (W > 1) m[1] = ok ? w1 : 0ull;
    if (W > 2) m[2] = ok ? w2 : 0ull;
    if (W > 3) m[3] = ok ? w3 : 0ull;
    depths[row] = ok ? depth : -1;
    positions[row] = ok ? P + depth : -1;
  }
}

__global__ __launch_bounds__(SPEC_MAX_NODES) void tree_assemble_kernel(
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ parents,
    const int32_t* __restrict__ root_tokens, int N, int H, int k, int32_t* __restrict__ tokens,
    int32_t* __restrict__ draft_row, int32_t* __restrict__ err) {
  __shared__ int s_par[SPEC_MAX_NODES];
  __shared__ int s_err;
  const int b = blockIdx.x;
  const int i = threadIdx.x;
  if (i == 0) s_err = INT_MAX;
  if (i < N) s_par[i] = parents[i];
  __syncthreads();

  int depth = 0, rank = 0;
  if (i < N) {
    int code = 0;
    const int p = s_par[i];
    if (i == 0) {
      if (p != -1) code = SPEC_ERR_ROOT;
    } else if (p < 0 || p >= i) {
      code = SPEC_ERR_PARENT;
    } else {
      int j = i;
      while (j > 0) {
        const int pj = s_par[j];
        if (pj < 0 || pj >= j) break;
        j = pj;
        ++depth;
      }
      for (int s = 1; s < i; ++s) rank += (s_par[s] == p) ? 1 : 0;
      if (depth > H || rank >= k) code = SPEC_ERR_RANK;
    }
    if (code) atomicMin(&s_err, err_word(i, code));
  }
  __syncthreads();

  const int e = s_err == INT_MAX ? 0 : s_err;
  if (i == 0) err[b] = e;
  if (i < N) {
    const size_t row = (size_t)b * N + i;
    int tok = -1, dr = -1;
    if (e == 0) {
      if (i == 0) {
        tok = root_tokens ? root_tokens[b] : -1;
      } else {
        tok = topk_idx[((size_t)b * H + (depth - 1)) * k + rank];
        dr = depth - 1;
      }
    }
    tokens[row] = tok;
    draft_row[row] = dr;
  }
}

}  // namespace
}  // namespace spectree

using namespace spectree;

extern "C" spec_status spec_tree_build(const int32_t* parents, const int32_t* depths_in,
                                       const int32_t* prefix_len, const int32_t* n_nodes, int B,
                                       int N, uint64_t* mask, int32_t* positions,
                                       int32_t* depths, int32_t* err, void* stream) {
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES) return SPEC_EINVAL;
  if (!parents || !mask || !positions || !depths || !err) return SPEC_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int W = (N + 63) / 64;
  launch("tree_build", tree_build_kernel, dim3(B), dim3(SPEC_MAX_NODES), s, parents, depths_in, prefix_len,
         n_nodes, N, W, mask, positions, depths, err);
  return launch_status();
}

extern "C" spec_status spec_tree_assemble(const int32_t* topk_idx, const int32_t* parents,
                                          const int32_t* root_tokens, int B, int N, int H, int k,
                                          int32_t* tokens, int32_t* draft_row, int32_t* err,
                                          void* stream) {
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES || H < 1 || k < 1) return SPEC_EINVAL;
  if (!topk_idx || !parents || !tokens || !draft_row || !err) return SPEC_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  launch("tree_assemble", tree_assemble_kernel, dim3(B), dim3(SPEC_MAX_NODES), s, topk_idx, parents,
         root_tokens, N, H, k, tokens, draft_row, err);
  return launch_status();
}
