// KV-cache compaction that closes a verification round ("EAGLE-3とMedusaで実装するSpeculative
// Decoding実践ガイド", section "Speculative Decodingの動作原理を理解する": each cycle verifies with
// one pass over the KV cache, and every candidate after a rejected one is discarded).  Tree node
// i's K/V sits at slot P + i; after verification the root and the accepted path are committed,
// so node path[j] moves to slot P + j (j = 1..accept_len) and the prefix grows by accept_len + 1.
//
// One wave per (layer, sequence, KV head, cache): a pure copy of at most max_depth rows, bound by
// latency, not bandwidth.  The wave copies the rows in passes of increasing j, each pass loading
// all of its rows before storing any.  That order is safe in place: a pass stores slots P + j
// with j at most the pass's largest index, while every later pass reads slots P + path[j'] with
// path[j'] >= j' (indices increase along the path), and a slot that an earlier pass read and a
// later pass overwrites was read before that earlier pass stored anything.
#include <climits>

#include "common.h"

namespace spectree {
namespace {

struct KvArgs {
  char* k;
  char* v;
  const int32_t* prefix_len;
  int32_t* prefix_out;
  const int32_t* path;
  const int32_t* accept_len;
  const int32_t* err;
  size_t layer_bytes;   // distance between layers
  int L, B, Hkv, S_max, max_depth;
  int row_bytes;        // head_dim * element size, a multiple of 16 and at most 64 * 16
};

__global__ __launch_bounds__(kWave) void kv_compact_kernel(KvArgs a) {
  int w = blockIdx.x;
  const int which = w & 1;              // 0: K cache, 1: V cache
  w >>= 1;
  const int h = w % a.Hkv;
  w /= a.Hkv;
  const int b = w % a.B;
  const int l = w / a.B;
  const int lane = threadIdx.x;
  const int P = a.prefix_len[b];
  const int A = a.accept_len[b];
  const int e = a.err ? a.err[b] : 0;
  const int32_t* pb = a.path + (size_t)b * (a.max_depth + 1);
  // The path must be a root-first chain of increasing node indices whose last slot lies in the
  // cache (so do all others); a sequence that fails this, or whose verification reported an
  // error, keeps its cache and prefix as they were.
  bool ok = e == 0 && A >= 0 && A <= a.max_depth && P >= 0;
  if (ok) {
    bool good = true;
    for (int j = lane; j <= A; j += kWave) {
      const int pj = pb[j];
      good = good && (j == 0 ? pj == 0 : pj > pb[j - 1]);
      if (j == A) good = good && (long long)P + pj < (long long)a.S_max;
    }
    ok = __all(good);
  }
  if (a.prefix_out && l == 0 && h == 0 && which == 0 && lane == 0) a.prefix_out[b] = ok ? P + A + 1 : P;
  if (!ok || A == 0) return;
  char* base = (which ? a.v : a.k) + (size_t)l * a.layer_bytes +
               ((size_t)b * a.Hkv + h) * (size_t)a.S_max * a.row_bytes;
  const int cpr = a.row_bytes / 16;       // 16-byte chunks per row
  const int rpp = kWave / cpr;            // rows per pass
  const int sub = lane / cpr, ch = lane - sub * cpr;
  for (int j0 = 1; j0 <= A; j0 += rpp) {
    const int j = j0 + sub;
    const bool act = sub < rpp && j <= A;
    int4 x = {0, 0, 0, 0};
    if (act) x = *reinterpret_cast<const int4*>(base + (size_t)(P + pb[j]) * a.row_bytes + ch * 16);
    // the store depends on this pass's load, so every lane's load of the pass has completed
    // before any lane stores
    if (act) *reinterpret_cast<int4*>(base + (size_t)(P + j) * a.row_bytes + ch * 16) = x;
  }
}

}  // namespace
}  // namespace spectree

using namespace spectree;

extern "C" spec_status spec_kv_compact(void* k_cache, void* v_cache, size_t layer_stride, int L,
                                       const int32_t* prefix_len, int32_t* prefix_len_out,
                                       const int32_t* path, const int32_t* accept_len,
                                       const int32_t* err, int B, int Hkv, int S_max, int head_dim,
                                       int max_depth, int dtype, void* stream) {
  if (!k_cache || !v_cache || !prefix_len || !path || !accept_len) return SPEC_EINVAL;
  if (L < 1 || B < 1 || Hkv < 1 || S_max < 1 || head_dim < 1 || max_depth < 0) return SPEC_EINVAL;
  if (prefix_len_out && prefix_len_out == prefix_len) return SPEC_EINVAL;
  if (dtype != SPEC_BF16 && dtype != SPEC_F32) return SPEC_EUNSUPPORTED;
  const int esize = dtype == SPEC_BF16 ? 2 : 4;
  const long long row_bytes = (long long)head_dim * esize;
  if (row_bytes % 16 != 0 || row_bytes > 16LL * kWave) return SPEC_EUNSUPPORTED;
  const size_t layer_elems = (size_t)B * Hkv * S_max * head_dim;
  if (L > 1 && layer_stride < layer_elems) return SPEC_EINVAL;
  if ((reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) % 16 != 0 ||
      (L > 1 && (layer_stride * esize) % 16 != 0))
    return SPEC_EUNSUPPORTED;
  const size_t waves = (size_t)L * B * Hkv * 2;
  if (waves > (size_t)INT_MAX) return SPEC_EUNSUPPORTED;

  KvArgs a{};
  a.k = static_cast<char*>(k_cache);
  a.v = static_cast<char*>(v_cache);
  a.prefix_len = prefix_len;
  a.prefix_out = prefix_len_out;
  a.path = path;
  a.accept_len = accept_len;
  a.err = err;
  a.layer_bytes = (L > 1 ? layer_stride : layer_elems) * esize;
  a.L = L; a.B = B; a.Hkv = Hkv; a.S_max = S_max; a.max_depth = max_depth;
  a.row_bytes = (int)row_bytes;
  launch("kv_compact", kv_compact_kernel, dim3((unsigned)waves), dim3(kWave),
         static_cast<hipStream_t>(stream), a);
  return launch_status();
}
