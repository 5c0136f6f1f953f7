// EAGLE-style tree assembly: the children of each node take the top candidates of the draft
// distribution computed at that node ("多トークン予測（Medusa・EAGLE）", section
// "EAGLE：token ではなく「特徴量」を先読みする": each drafted step yields a candidate distribution
// through the LM head, repeated into a tree; "EAGLE-3とMedusaで実装するSpeculative Decoding実践
// ガイド", section "Tree Attention：候補を木構造で探索する": several candidates per position).
//
// Order: probability high to low, draft id low to high on ties (-0.0 equals 0.0).  Every entry
// of a row gets a unique 64-bit key, (order-preserving bits of the probability) << 32 |
// (~id), so "better" is simply "larger key" and no two entries tie.
//
// Two kernels in stream order (the kernel boundary orders them; no workgroup waits on another;
// large grids first list the nodes with children, see assemble_list_kernel):
//   chunks  grid (j, sequence, chunk of 8192 draft ids), j slowest: workgroup (j, b, c) finds
//           (from the parent array, one load per thread) the j-th node of sequence b that has
//           children (k of them) and ranks chunk c of that node's draft row: 32 entries per
//           thread in registers.  Within each wave the k-th largest lane maximum is a lower
//           bound of the chunk's k-th largest key (k <= 64; past that the k-th largest of all
//           thread maxima), the largest such bound is tau, and only entries >= tau (typically a
//           few more than k) are gathered
//           in LDS and ranked exactly by pairwise counts; past 256 of them (a wide node) k
//           rounds of a block max take the keys in order instead.  The chunk's best
//           min(k, chunk length) keys go to the workspace, in order, at the node's slot range
//           (slots are the prefix sums of the child counts: one per child per chunk), with a
//           NaN flag.  Leaf nodes' workgroups leave after one look at the parent array.
//   merge   one workgroup per sequence: validation, the written list entries and NaN flags
//           staged in LDS in one round of loads, then one wave per node with children merges
//           its chunk lists (lane = chunk, k rounds of a wave max), maps the draft ids through
//           d2t, and the sequence's error word is the smallest (node, code) pair.
#include <climits>

#include "common.h"

namespace spectree {
namespace {

constexpr int kAT = 256;                     // chunk workgroup
constexpr int kAPer = 32;                    // entries per thread
constexpr int kAChunk = kAT * kAPer;         // draft ids per chunk
constexpr int kAMaxChunks = 32;              // Vd <= 262144
constexpr int kMT = 1024;                    // merge workgroup
constexpr int kACand = 256;                  // candidate buffer (entries >= tau)

struct RowsArgs {
  const float* draft;        // [B, R, Vd]
  const int32_t* parents;    // [B, N]
  const int32_t* draft_row;  // [B, N]
  const int32_t* d2t;        // [Vd] or NULL
  const int32_t* n_nodes;    // [B] or NULL
  const int32_t* root_tokens;
  int B, N, R, Vd, V, CA;
  int32_t* tokens;
  float* cand_prob;
  int32_t* err;
  uint64_t* keys;            // [B, CA, N]: slot s of a chunk's list
  int32_t* nonfinite;        // [B, CA, N]: per (chunk, node with children)
  int4* list;                // [B * N]: (b N + node, children, first slot, draft row) of each node
                             // with children, in (sequence, node) order (listed path)
  int32_t* list_count;       // [1]: entries of list
};

// The listed path: one workgroup first lists the nodes with children, then workgroup i of the
// chunk pass takes the i-th listed (node, chunk) item, so that the workgroups with work come
// first and start their chunk loads after one lookup.  Used for B * N <= kAListMax and grids of
// at least kAListMinItems (node, chunk) items.
constexpr int kAListMax = 4096;
constexpr int kAListThreads = 1024;
constexpr int kAListPer = kAListMax / kAListThreads;
constexpr size_t kAListMinItems = 8192;

// Order-preserving bits of a float (-0.0 folded into 0.0): larger float, larger bits; a NaN
// gets 0, below every number.
__device__ __forceinline__ uint32_t ord_bits(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return isnan(x) ? 0u : o;
}
// Inverse of ord_bits (0, a NaN's bits, gives a NaN).
__device__ __forceinline__ float from_ord(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
// Key of draft id `id` with order bits o: larger key = ranked first.  Never 0.
__device__ __forceinline__ uint64_t make_key(uint32_t o, int id) {
  return ((uint64_t)o << 32) | (uint64_t)(0xffffffffu - (uint32_t)id);
}

// Chunk c of the draft row r of node p of sequence b, which has k children whose keys go to slots
// off .. off + k - 1 of the chunk's list: the chunk's best min(k, chunk length) keys, in order,
// and its NaN flag.
__device__ void rank_chunk(const RowsArgs& a, int b, int p, int k, int off, int r, int c) {
  constexpr int kWavesA = kAT / kWave;
  __shared__ uint32_t s_max[kAT];
  __shared__ uint64_t s_cand[kACand];
  __shared__ uint64_t s_wmax[kWavesA];
  __shared__ uint32_t s_wtau[kWavesA];
  __shared__ uint32_t s_tau;
  __shared__ int s_count;
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  if (t == 0) s_count = 0;                        // read after the barriers below
  const int lo = c * kAChunk;
  const int len = min(kAChunk, a.Vd - lo);
  const int kk = min(k, len);
  const float* row = a.draft + ((size_t)b * a.R + r) * a.Vd;

  // second round: the chunk, 32 entries per thread, kept as order bits; entry e of thread t is
  // draft id lo + (e / 4 * kAT + t) * 4 + e % 4 (addresses past the chunk read its first entry)
  uint32_t o[kAPer];
  int nan = 0;
  const bool vec4 = (a.Vd % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.draft) & 15) == 0);
  if (vec4) {
    float4 v[kAPer / 4];
#pragma unroll
    for (int q = 0; q < kAPer / 4; ++q) {
      const int id = lo + (q * kAT + t) * 4;
      v[q] = *reinterpret_cast<const float4*>(row + (id < lo + len ? id : lo));
    }
#pragma unroll
    for (int q = 0; q < kAPer / 4; ++q) {
      o[4 * q] = ord_bits(v[q].x); o[4 * q + 1] = ord_bits(v[q].y);
      o[4 * q + 2] = ord_bits(v[q].z); o[4 * q + 3] = ord_bits(v[q].w);
    }
  } else {
    float x[kAPer];
#pragma unroll
    for (int e = 0; e < kAPer; ++e) {
      const int id = lo + (e / 4 * kAT + t) * 4 + e % 4;
      x[e] = row[id < lo + len ? id : lo];
    }
#pragma unroll
    for (int e = 0; e < kAPer; ++e) o[e] = ord_bits(x[e]);
  }
  auto in_chunk = [&](int e) { return lo + (e / 4 * kAT + t) * 4 + e % 4 < lo + len; };
  uint32_t mx = 0;
#pragma unroll
  for (int e = 0; e < kAPer; ++e) {
    const bool in = in_chunk(e);
    nan |= (in && o[e] == 0u) ? 1 : 0;
    mx = (in && o[e] > mx) ? o[e] : mx;
  }
  // tau: a lower bound of the value of the chunk's kk-th best entry.  kk <= 64: the largest,
  // over the waves, of the wave's kk-th largest lane maximum (those kk lanes hold kk distinct
  // entries at or above it); otherwise the kk-th largest of all thread maxima.
  if (kk <= kWave) {
    int above = 0;
#pragma unroll
    for (int l = 0; l < kWave; ++l) above += __shfl(mx, l) > mx ? 1 : 0;
    uint32_t wt = above < kk ? mx : 0xffffffffu;
#pragma unroll
    for (int sh = 32; sh > 0; sh >>= 1) wt = min(wt, (uint32_t)__shfl_xor(wt, sh));
    if (lane == 0) s_wtau[w] = wt;
    nan = __syncthreads_or(nan);
    if (t == 0) {
      uint32_t tv = 0u;
#pragma unroll
      for (int q = 0; q < kWavesA; ++q) tv = max(tv, s_wtau[q]);
      s_tau = tv;
    }
  } else {
    s_max[t] = mx;
    if (t == 0) s_tau = 0xffffffffu;
    nan = __syncthreads_or(nan);
    int above = 0;
#pragma unroll 16
    for (int j = 0; j < kAT; ++j) above += s_max[j] > mx ? 1 : 0;
    if (above < kk) atomicMin(&s_tau, mx);
  }
  __syncthreads();
  const uint32_t tau = s_tau;
  // the candidates: every entry whose value reaches tau (a NaN only when tau is 0), as keys
#pragma unroll
  for (int e = 0; e < kAPer; ++e) {
    if (in_chunk(e) && o[e] >= tau) {
      const int at = atomicAdd(&s_count, 1);
      if (at < kACand) s_cand[at] = make_key(o[e], lo + (e / 4 * kAT + t) * 4 + e % 4);
    }
  }
  __syncthreads();
  const int C = s_count;
  uint64_t* dst = a.keys + ((size_t)b * a.CA + c) * a.N + off;
  if (C <= kACand) {
    // few candidates: each one's rank is the number of larger keys (keys are unique)
    if (t < C) {
      const uint64_t me = s_cand[t];
      int rank = 0;
      for (int j = 0; j < C; ++j) rank += s_cand[j] > me ? 1 : 0;
      if (rank < kk) dst[rank] = me;
    }
  } else {
    // many candidates (a wide node, or heavy ties): kk rounds, each taking the largest key
    // below the previous one
    uint64_t prev = ~0ull;
    for (int j = 0; j < kk; ++j) {
      uint64_t best = 0ull;
#pragma unroll
      for (int e = 0; e < kAPer; ++e) {
        const uint64_t key = make_key(o[e], lo + (e / 4 * kAT + t) * 4 + e % 4);
        best = (in_chunk(e) && key < prev && key > best) ? key : best;
      }
#pragma unroll
      for (int sh = 32; sh > 0; sh >>= 1) {
        const uint64_t other = __shfl_xor(best, sh);
        best = other > best ? other : best;
      }
      if (lane == 0) s_wmax[w] = best;
      __syncthreads();
      best = s_wmax[0];
#pragma unroll
      for (int q = 1; q < kWavesA; ++q) best = s_wmax[q] > best ? s_wmax[q] : best;
      __syncthreads();
      if (t == 0) dst[j] = best;
      prev = best;
    }
  }
  if (t == 0) a.nonfinite[((size_t)b * a.CA + c) * a.N + p] = nan;
}

__global__ __launch_bounds__(kAT) void assemble_chunks_kernel(RowsArgs a) {
  constexpr int kWavesA = kAT / kWave;
  __shared__ int s_rows[SPEC_MAX_NODES];
  __shared__ int s_has[SPEC_MAX_NODES];
  __shared__ int s_wtot[kWavesA];
  __shared__ int s_first, s_p;
  // workgroup -> (j-th node with children of sequence b, chunk c), j slowest: the workgroups
  // with work are dispatched first, and the ones past a sequence's last such node leave early
  const int c = blockIdx.x % a.CA;
  const int rest = blockIdx.x / a.CA;
  const int b = rest % a.B;
  const int jn = rest / a.B;
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  // first round of loads, all independent: n, this thread's parent entry and draft row
  const int n = a.n_nodes ? a.n_nodes[b] : a.N;
  const size_t ti = (size_t)b * a.N + min(t, a.N - 1);
  const int par_t = a.parents[ti];
  const int row_t = a.draft_row[ti];
  if (n < 1 || n > a.N || jn >= n) return;
  // valid node t (t < n, parent in [0, t)); nodes named by a valid node have children
  const bool valid = t >= 1 && t < n && par_t >= 0 && par_t < t;
  if (t < a.N) { s_rows[t] = row_t; s_has[t] = 0; }
  if (t == 0) { s_first = INT_MAX; s_p = -1; }
  __syncthreads();
  if (valid) s_has[par_t] = 1;
  __syncthreads();
  const bool has = t < n && s_has[t];
  const uint64_t bal = __ballot(has);
  if (lane == 0) s_wtot[w] = __popcll(bal);
  __syncthreads();
  int before = __popcll(bal & ((1ull << lane) - 1ull)), total = 0;
#pragma unroll
  for (int q = 0; q < kWavesA; ++q) {
    before += q < w ? s_wtot[q] : 0;
    total += s_wtot[q];
  }
  if (jn >= total) return;                        // past the last node with children
  if (has && before == jn) s_p = t;
  __syncthreads();
  const int p = s_p;
  const bool mine = valid && par_t == p;
  if (mine) atomicMin(&s_first, t);
  const int k = __syncthreads_count(mine);
  const int off = __syncthreads_count(valid && par_t < p);
  const int r = s_rows[s_first];
  if (r < 0 || r >= a.R) return;                  // the merge reports it
  rank_chunk(a, b, p, k, off, r, c);
}

// Exclusive prefix over the workgroup of two counts (thread order); the totals to every thread.
__device__ __forceinline__ int2 list_scan(int x, int y, int2& total) {
  constexpr int kW = kAListThreads / kWave;
  __shared__ int2 s_w[kW];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int ix = x, iy = y;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int ux = __shfl_up(ix, o), uy = __shfl_up(iy, o);
    if (lane >= o) { ix += ux; iy += uy; }
  }
  if (lane == kWave - 1) s_w[w] = make_int2(ix, iy);
  __syncthreads();
  int bx = 0, by = 0, tx = 0, ty = 0;
#pragma unroll
  for (int q = 0; q < kW; ++q) {
    const int2 v = s_w[q];
    if (q < w) { bx += v.x; by += v.y; }
    tx += v.x; ty += v.y;
  }
  total = make_int2(tx, ty);
  return make_int2(bx + ix - x, by + iy - y);
}

// Lists the nodes with children of every sequence, in (sequence, node) order: thread t owns the
// contiguous (sequence, node) entries [t per, t per + per); their parent, draft row and n_nodes
// loads are requested at once.  A node's entry: its children count k, its first slot (the
// children of lower-index nodes of the sequence) and the draft row of its lowest-index child;
// nodes whose row is out of range are left out (the merge reports them), as are sequences with
// an invalid n_nodes (they have no valid children).
__global__ __launch_bounds__(kAListThreads) void assemble_list_kernel(RowsArgs a) {
  __shared__ int s_cnt[kAListMax];
  __shared__ int s_first[kAListMax];
  __shared__ int s_drow[kAListMax];
  __shared__ int s_base[kAListMax];             // first slot of each entry's sequence
  const int t = threadIdx.x;
  const int total = a.B * a.N;
  const int per = (total + kAListThreads - 1) / kAListThreads;   // <= kAListPer
  const int i0 = t * per;
  int par[kAListPer], nn[kAListPer], dr[kAListPer];
#pragma unroll
  for (int k = 0; k < kAListPer; ++k) {
    const int i = min(i0 + k, total - 1);
    par[k] = a.parents[i];
    dr[k] = a.draft_row[i];
    nn[k] = a.n_nodes ? a.n_nodes[i / a.N] : a.N;
  }
#pragma unroll
  for (int k = 0; k < kAListPer; ++k)
    if (k < per && i0 + k < total) { s_cnt[i0 + k] = 0; s_first[i0 + k] = INT_MAX; s_drow[i0 + k] = dr[k]; }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kAListPer; ++k) {
    const int i = i0 + k;
    if (k < per && i < total) {
      const int b = i / a.N, c = i - b * a.N, n = nn[k], p = par[k];
      if (n >= 1 && n <= a.N && c >= 1 && c < n && p >= 0 && p < c) {
        atomicAdd(&s_cnt[b * a.N + p], 1);
        atomicMin(&s_first[b * a.N + p], c);
      }
    }
  }
  __syncthreads();
  int cnt[kAListPer], row[kAListPer];
  int sc = 0, sl = 0;
#pragma unroll
  for (int k = 0; k < kAListPer; ++k) {
    const int i = i0 + k;
    const bool in = k < per && i < total;
    cnt[k] = in ? s_cnt[i] : 0;
    row[k] = cnt[k] > 0 ? s_drow[(i / a.N) * a.N + s_first[i]] : -1;
    sc += cnt[k];
    sl += (cnt[k] > 0 && row[k] >= 0 && row[k] < a.R) ? 1 : 0;
  }
  int2 all;
  const int2 ex = list_scan(sc, sl, all);
  // the first slot of each sequence: the running count at its node 0
  int rc = ex.x;
#pragma unroll
  for (int k = 0; k < kAListPer; ++k) {
    const int i = i0 + k;
    if (k < per && i < total && i % a.N == 0) s_base[i / a.N] = rc;
    rc += cnt[k];
  }
  __syncthreads();
  rc = ex.x;
  int at = ex.y;
#pragma unroll
  for (int k = 0; k < kAListPer; ++k) {
    const int i = i0 + k;
    if (k < per && i < total && cnt[k] > 0 && row[k] >= 0 && row[k] < a.R)
      a.list[at++] = make_int4(i, cnt[k], rc - s_base[i / a.N], row[k]);
    rc += cnt[k];
  }
  if (t == 0) *a.list_count = all.y;
}

// Workgroup it takes chunk it % CA of the (it / CA)-th listed node; the rest leave after one
// look at the count.  The count and the entry are requested together (the entry's index is
// clamped into the list).
__global__ __launch_bounds__(kAT) void assemble_listed_kernel(RowsArgs a) {
  const int it = blockIdx.x;
  const int c = it % a.CA, i = it / a.CA;
  const int count = *a.list_count;
  const int4 e = a.list[min(i, a.B * a.N - 1)];
  if (i >= count) return;
  const int b = e.x / a.N;
  rank_chunk(a, b, e.x - b * a.N, e.y, e.z, e.w, c);
}

// One workgroup per sequence: bookkeeping one thread per node, the chunk lists staged in LDS
// in one round of loads, then one wave per node with children merges its lists.
__global__ __launch_bounds__(kMT) void assemble_merge_kernel(RowsArgs a) {
  constexpr int kWaves = kMT / kWave;
  constexpr int kWords = SPEC_MAX_NODES / 64;
  __shared__ int s_par[SPEC_MAX_NODES];
  __shared__ int s_row[SPEC_MAX_NODES];
  __shared__ int s_k[SPEC_MAX_NODES];          // valid children per node
  __shared__ int s_off[SPEC_MAX_NODES];        // first slot of each node's list
  __shared__ int s_first[SPEC_MAX_NODES];      // first child
  __shared__ int s_owner[SPEC_MAX_NODES];      // node owning each slot
  __shared__ int s_listed[SPEC_MAX_NODES];     // node with children and a valid row
  __shared__ int s_nf[SPEC_MAX_NODES];         // a NaN in the node's row
  __shared__ int s_list[SPEC_MAX_NODES];
  __shared__ unsigned long long s_kids[SPEC_MAX_NODES][kWords];   // children of each node, as bits
  __shared__ int s_wsum[4];
  __shared__ uint64_t s_sel[SPEC_MAX_NODES];   // selected key per slot
  __shared__ uint64_t s_keys[kAMaxChunks * SPEC_MAX_NODES];   // [chunk][slot]
  __shared__ int s_nlist, s_err;
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int N = a.N;
  const int n = a.n_nodes ? a.n_nodes[b] : N;
  const size_t base = (size_t)b * N;
  const int par_t = a.parents[base + min(t, N - 1)];
  const int row_t = a.draft_row[base + min(t, N - 1)];
  if (t == 0) { s_err = INT_MAX; s_nlist = 0; }
  if (t < N) {
    s_par[t] = par_t; s_row[t] = row_t; s_k[t] = 0; s_first[t] = INT_MAX; s_sel[t] = 0ull;
    s_listed[t] = 0; s_nf[t] = 0;
#pragma unroll
    for (int q = 0; q < kWords; ++q) s_kids[t][q] = 0ull;
  }
  __syncthreads();
  if (n < 0 || n > N) {
    if (t < N) {
      a.tokens[base + t] = -1;
      a.cand_prob[base + t] = __uint_as_float(0x7fc00000u);
    }
    if (t == 0) a.err[b] = err_word(0, SPEC_ERR_NNODES);
    return;
  }
  int code = 0;
  const bool valid = t >= 1 && t < n && par_t >= 0 && par_t < t;
  if (t == 0 && n > 0 && par_t != -1) code = SPEC_ERR_ROOT;
  if (t >= 1 && t < n && !valid) code = SPEC_ERR_PARENT;
  if (valid) {
    atomicAdd(&s_k[par_t], 1);
    atomicMin(&s_first[par_t], t);
    atomicOr(&s_kids[par_t][t >> 6], 1ull << (t & 63));
  }
  __syncthreads();
  // slot offsets: exclusive scan of the child counts over nodes (waves 0-3 hold nodes 0-255)
  int kt = (t < n) ? s_k[t] : 0;
  int incl = kt;
#pragma unroll
  for (int sh = 1; sh < kWave; sh <<= 1) {
    const int y = __shfl_up(incl, sh);
    if (lane >= sh) incl += y;
  }
  if (w < 4 && lane == kWave - 1) s_wsum[w] = incl;
  int rank = 0;
  if (valid) {
    // sibling rank: earlier children of the same node, from its child bits
#pragma unroll
    for (int q = 0; q < kWords; ++q) {
      const unsigned long long bits = s_kids[par_t][q];
      const int lim = t - 64 * q;
      rank += lim >= 64 ? __popcll(bits) : (lim > 0 ? __popcll(bits & ((1ull << lim) - 1ull)) : 0);
    }
    const int r0 = s_row[s_first[par_t]];
    if (row_t < 0 || row_t >= a.R || row_t != r0) code = SPEC_ERR_DRAFTROW;
    else if (rank >= a.Vd) code = SPEC_ERR_RANK;
  }
  __syncthreads();
  if (t < n) {
    int off = incl - kt;
    for (int q = 0; q < w; ++q) off += s_wsum[q];
    s_off[t] = off;
    if (kt > 0) {
      const int r0 = s_row[s_first[t]];
      if (r0 >= 0 && r0 < a.R) {
        s_listed[t] = 1;
        s_list[atomicAdd(&s_nlist, 1)] = t;
      }
    }
  }
  __syncthreads();
  if (valid) s_owner[s_off[par_t] + rank] = par_t;
  const int S = n >= 1 ? s_off[n - 1] + s_k[n - 1] : 0;   // slots: one per valid child
  __syncthreads();
  // stage the written list entries and the NaN flags, every load issued before any is used
  for (int i = t; i < a.CA * S; i += kMT) {
    const int l = i / S, slot = i - l * S;
    const int p = s_owner[slot];
    const int cnt = min(s_k[p], min(kAChunk, a.Vd - l * kAChunk));
    if (s_listed[p] && slot - s_off[p] < cnt) s_keys[l * SPEC_MAX_NODES + slot] = a.keys[((size_t)b * a.CA + l) * N + slot];
  }
  for (int i = t; i < a.CA * n; i += kMT) {
    const int l = i / n, p = i - l * n;
    if (s_listed[p] && a.nonfinite[((size_t)b * a.CA + l) * N + p]) atomicOr(&s_nf[p], 1);
  }
  __syncthreads();
  if (t < n && s_listed[t] && s_nf[t]) atomicMin(&s_err, err_word(s_first[t], SPEC_ERR_NONFINITE));
  // merge: wave w takes listed nodes w, w + kWaves, ...; lane l holds chunk l's list head
  const int nl = s_nlist;
  for (int li = w; li < nl; li += kWaves) {
    const int p = s_list[li];
    const int k = s_k[p], off = s_off[p];
    const int len = lane < a.CA ? min(kAChunk, a.Vd - lane * kAChunk) : 0;
    const int cnt = min(k, len);
    const uint64_t* lst = s_keys + lane * SPEC_MAX_NODES + off;
    int h = 0;
    uint64_t key = cnt > 0 ? lst[0] : 0ull;
    const int take = min(k, a.Vd);
    for (int j = 0; j < take; ++j) {
      uint64_t best = key;
#pragma unroll
      for (int sh = 32; sh > 0; sh >>= 1) {
        const uint64_t other = __shfl_xor(best, sh);
        best = other > best ? other : best;
      }
      if (lane == 0) s_sel[off + j] = best;
      if (key == best && best != 0ull) {              // keys are unique: one lane advances
        ++h;
        key = h < cnt ? lst[h] : 0ull;
      }
    }
  }
  __syncthreads();
  // children: draft id, probability (a NaN for a NaN entry), token through d2t
  int tok = -1;
  float prob = __uint_as_float(0x7fc00000u);
  if (valid && code == 0) {
    const uint64_t key = s_sel[s_off[par_t] + rank];
    const int id = (int)(0xffffffffu - (uint32_t)(key & 0xffffffffull));
    prob = from_ord((uint32_t)(key >> 32));
    if (key != 0ull && id >= 0 && id < a.Vd) {
      tok = a.d2t ? a.d2t[id] : id;
      if (tok < 0 || tok >= a.V) code = SPEC_ERR_MAP;
    }
  }
  if (code) atomicMin(&s_err, err_word(t, code));
  __syncthreads();
  const int e = s_err == INT_MAX ? 0 : s_err;
  if (t == 0) a.err[b] = e;
  if (t < N) {
    const bool ok = e == 0 && t < n;
    if (t == 0) {
      a.tokens[base] = ok ? (a.root_tokens ? a.root_tokens[b] : -1) : -1;
      a.cand_prob[base] = ok ? 1.0f : __uint_as_float(0x7fc00000u);
    } else {
      a.tokens[base + t] = ok ? tok : -1;
      a.cand_prob[base + t] = ok ? prob : __uint_as_float(0x7fc00000u);
    }
  }
}

}  // namespace
}  // namespace spectree

using namespace spectree;

namespace {
spec_status check_rows_shape(int B, int N, int R, int Vd, int V) {
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES || R < 1 || Vd < 1 || V < 1) return SPEC_EINVAL;
  if (Vd > kAMaxChunks * kAChunk) return SPEC_EUNSUPPORTED;
  if ((long long)B * N * ((Vd + kAChunk - 1) / kAChunk) > INT_MAX) return SPEC_EUNSUPPORTED;
  return SPEC_OK;
}
}  // namespace

extern "C" size_t spec_tree_assemble_rows_workspace(int B, int N, int Vd) {
  if (check_rows_shape(B, N, 1, Vd, 1) != SPEC_OK) return 0;
  const size_t CA = (size_t)(Vd + kAChunk - 1) / kAChunk;
  return align_up((size_t)B * CA * N * sizeof(uint64_t), 256) + align_up((size_t)B * CA * N * sizeof(int32_t), 256) +
         align_up((size_t)B * N * sizeof(int4), 256) + align_up(sizeof(int32_t), 256);
}

extern "C" spec_status spec_tree_assemble_rows(const float* draft_probs, const int32_t* parents,
                                               const int32_t* draft_row, const int32_t* d2t,
                                               const int32_t* n_nodes, const int32_t* root_tokens,
                                               int B, int N, int R, int Vd, int V, int32_t* tokens,
                                               float* cand_prob, int32_t* err, void* workspace,
                                               size_t ws_bytes, void* stream) {
  const spec_status st = check_rows_shape(B, N, R, Vd, V);
  if (st != SPEC_OK) return st;
  if (!draft_probs || !parents || !draft_row || !tokens || !cand_prob || !err) return SPEC_EINVAL;
  if (!d2t && V != Vd) return SPEC_EINVAL;
  const size_t need = spec_tree_assemble_rows_workspace(B, N, Vd);
  if (!workspace || ws_bytes < need) return SPEC_EWORKSPACE;
  RowsArgs a{};
  a.draft = draft_probs; a.parents = parents; a.draft_row = draft_row; a.d2t = d2t; a.n_nodes = n_nodes;
  a.root_tokens = root_tokens; a.B = B; a.N = N; a.R = R; a.Vd = Vd; a.V = V;
  a.CA = (Vd + kAChunk - 1) / kAChunk;
  a.tokens = tokens; a.cand_prob = cand_prob; a.err = err;
  char* w = static_cast<char*>(workspace);
  a.keys = reinterpret_cast<uint64_t*>(w);
  size_t off = align_up((size_t)B * a.CA * N * sizeof(uint64_t), 256);
  a.nonfinite = reinterpret_cast<int32_t*>(w + off);
  off += align_up((size_t)B * a.CA * N * sizeof(int32_t), 256);
  a.list = reinterpret_cast<int4*>(w + off);
  off += align_up((size_t)B * N * sizeof(int4), 256);
  a.list_count = reinterpret_cast<int32_t*>(w + off);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)((size_t)B * N * a.CA));
  if ((size_t)B * N <= (size_t)kAListMax && (size_t)B * N * a.CA >= kAListMinItems) {
    launch("assemble_list", assemble_list_kernel, dim3(1), dim3(kAListThreads), s, a);
    launch("assemble_chunks", assemble_listed_kernel, grid, dim3(kAT), s, a);
  } else {
    launch("assemble_chunks", assemble_chunks_kernel, grid, dim3(kAT), s, a);
  }
  launch("assemble_merge", assemble_merge_kernel, dim3(B), dim3(kMT), s, a);
  return launch_status();
}
