// Tree attention: every tree node's query attends to the shared committed prefix and to its
// own ancestors only ("多トークン予測（Medusa・EAGLE）", section
// "ツリー検証：候補を「木」に束ねて1回で確かめる"; "EAGLE-3とMedusaで実装するSpeculative
// Decoding実践ガイド", sections "並列検証：ターゲットモデルの1回のforward passで一括確認する"
// and "Tree Attention：候補を木構造で探索する").
//
// bf16 path (MFMA, gfx950).  A work unit is one (sequence b, key/value head g).  Its query rows
// are the N tree nodes x the G query heads that share g, M = N * G rows, row r = node r / G,
// head g * G + r % G.  All of them read the same keys, so each 64-key tile is fetched from HBM
// once per workgroup (16-byte loads, 16 lanes per 256-byte key row), staged in LDS and reused
// by every row of the workgroup.
//
// Each wave owns 16 * CB query rows.  Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_16x16x32_bf16: A = a 16-key x 32-dim slice of K read from LDS, B = Q^T held in
// registers for the whole kernel.  The accumulator layout gives lane l the query row l % 16
// and keys 4 * (l / 16) + i, which is the B-operand layout of the next product
// O^T = V^T P^T, so the softmax weights never leave their lanes.  V stays row-major in LDS; its
// A-operand fragments (one output dimension per lane, 8 keys in the slots) come from the LDS
// transpose read ds_read_b64_tr_b16: within each 16-lane group, lane L reads 4 dimensions of
// key key0 + L / 4 and lane j receives dimension j of those 4 keys.  Every per-row quantity
// (running max, sum, rescale) lives in the lanes of that row.  The reference max of the
// exponentials moves only when a tile's max exceeds it by more than a slack of 2^8, so the O
// rescale is rare (softmax does not depend on the reference); a tile whose weights all stay
// below 2^8 against the current references needs no row max at all.
//
// Tiles are double-buffered: the next tile's global loads (buffer loads with 32-bit offsets
// into the head's K and V) are issued into registers before the current tile is computed and
// written to the other LDS buffer afterwards, so there is one barrier per tile and the HBM
// latency hides behind the MFMA work.  Tiles that lie wholly in the prefix and inside the
// split skip all masking; the others mask with one 64-bit visibility word per row.
//
// Work split: grid = units x row blocks x key splits.  A split covers a contiguous key range
// of the unit (prefix and tree slots alike), computed on the device from prefix_len and
// n_nodes.  With more than one split, each workgroup stores its output normalised by its own
// sum (bf16) and its (max, sum) to the workspace and a second kernel merges them as a convex
// combination (the kernel boundary orders the two; no workgroup waits on another).  Workgroups
// of one unit are placed on one XCD (dispatch goes round-robin over the 8 XCDs) in both
// kernels, so the unit's K/V tiles, Q rows and partials share that XCD's L2; in a batch the
// sequences are dispatched longest first.
//
// fp32 path: a plain exact-fp32 kernel (one workgroup per query row) for small fp32 inputs.
#include <climits>

#include "common.h"

namespace spectree {
namespace {

constexpr int kKT = 64;        // keys per tile
constexpr int kThreads = 256;  // merge kernel workgroup
constexpr int kMaxLptSeqs = 256;  // longest-first ordering for batches up to this size
constexpr int kMaxWords = (SPEC_MAX_NODES + 63) / 64;   // ancestor words per tree node
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kLazy = 8;       // reference-max slack (log2 units): weights below 256

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
// Buffer loads: a per-workgroup descriptor (scalar registers) and 32-bit byte offsets per lane.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
__device__ __forceinline__ BufRsrc buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ bf16x8 buf_ld8(BufRsrc r, uint32_t lane_off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, 0, 0));
}
// Largest K or V cache of one (sequence, KV head) in bytes that the bf16 kernel addresses
// with 32-bit offsets.
constexpr long long kMaxHeadCacheBytes = 1ll << 31;
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* prefix_len;
  const uint64_t* mask;
  const int32_t* n_nodes;
  int B, N, Hq, Hkv, G, S_max, W;
  float scale;                 // softmax scale
  float scale_log2;            // scale * log2(e)
  void* out;
  float* lse;
  int32_t* err;
  // workspace
  float2* part_ml;             // [U, S, Mpad]: (max, sum) of each split
  __bf16* part_o;              // [U, S, Mpad, D]: each split's output normalised by its own sum
  int R, S, Mpad;
  int prio;                    // raise wave priority around the MFMA blocks
  float lazy;                  // reference-max slack in log2 units (0: exact running max)
  uint32_t lazy_bits;          // bf16 bit pattern of 2^lazy (positive bf16 order as integers)
  int lpt;                     // dispatch sequences longest first (batches of 2..256)
};

__device__ __forceinline__ bool seq_valid(int n, int P, int N, int S_max) {
  return n >= 0 && n <= N && P >= 0 && P + n <= S_max;
}

__device__ __forceinline__ int seq_err(int n, int P, int N, int S_max) {
  if (n < 0 || n > N) return err_word(0, SPEC_ERR_NNODES);
  if (P < 0 || P + n > S_max) return err_word(0, SPEC_ERR_PREFIX);
  return 0;
}

// Map the linear workgroup id to (unit, row block, split) so that all workgroups of a unit
// land on the same XCD (hardware dispatches consecutive workgroup ids round-robin over 8
// XCDs).  With a.lpt, sequences are taken longest first (prefix + nodes, ties by index): every
// workgroup ranks the B lengths in LDS, and since each XCD takes its workgroups in id order,
// the longest sequences' splits start first and the short ones fill in behind them.  Returns
// false for padding workgroups.
__device__ __forceinline__ bool decode_wg(const AttnArgs& a, int& u, int& rb, int& split) {
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int per_unit = a.R * a.S;
  const int lu = slot / per_unit;
  const int w = slot - lu * per_unit;
  u = xcd + 8 * lu;
  rb = w % a.R;
  split = w / a.R;
  if (u >= a.B * a.Hkv) return false;
  if (a.lpt) {
    __shared__ int s_len[kMaxLptSeqs];
    __shared__ int s_order[kMaxLptSeqs];
    for (int t = threadIdx.x; t < a.B; t += blockDim.x) {
      const int n = a.n_nodes ? a.n_nodes[t] : a.N;
      const int P = a.prefix_len[t];
      s_len[t] = (n >= 0 && n <= a.N && P >= 0 && P + n <= a.S_max) ? P + n : 0;
    }
    __syncthreads();
    for (int t = threadIdx.x; t < a.B; t += blockDim.x) {
      const int lt = s_len[t];
      int r = 0;
      for (int j = 0; j < a.B; ++j) r += (s_len[j] > lt || (s_len[j] == lt && j < t)) ? 1 : 0;
      s_order[r] = t;
    }
    __syncthreads();
    const int seq = u / a.Hkv;                   // rank of the sequence this workgroup takes
    u = s_order[seq] * a.Hkv + (u - seq * a.Hkv);
  }
  return true;
}

// A-operand fragment of V^T for output dims [d0, d0 + 16) and keys c32 + {4 lg + s, 16 + 4 lg + s}.
template <int VS>
__device__ __forceinline__ bf16x8 v_fragment(const __bf16* vt, int d0, int c32, int lg, int l16) {
  const __bf16* p0 = vt + (c32 + 4 * lg + (l16 >> 2)) * VS + d0 + 4 * (l16 & 3);
  const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p0);
  const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p0 + 16 * VS));
  typedef short short8_t __attribute__((ext_vector_type(8)));
  const short8_t both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, both);
}

// WAVES waves per workgroup, 16 * CB query rows per wave.  Two waves per SIMD are requested (at
// most 256 registers per lane): while one wave runs its softmax on the VALU the other keeps the
// matrix cores busy.
template <int D, int CB, int WAVES>
__global__ __launch_bounds__(WAVES * kWave) __attribute__((amdgpu_waves_per_eu(2)))
void tree_attn_bf16_kernel(AttnArgs a) {
  constexpr int THREADS = WAVES * kWave;
  // LDS row strides (elements): K rows 4 banks apart, V rows 8 banks apart, so the 16-byte K
  // reads and the 8-byte transpose reads of V meet no bank conflicts within a pass.
  constexpr int KS = D + 8;
  constexpr int VS = D + 16;
  constexpr int DS = D / 32;         // 32-dim steps of the score product
  constexpr int DB = D / 16;         // 16-dim blocks of the output
  constexpr int ROWS_WAVE = 16 * CB;
  constexpr int RBS = WAVES * ROWS_WAVE;
  constexpr int CPK = D / 8;         // 16-byte chunks per key row
  constexpr int KPP = THREADS / CPK; // keys per load pass
  constexpr int PASSES = kKT / KPP;
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[2][kKT * KS];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[2][kKT * VS];
  __shared__ uint64_t s_mask[RBS * kMaxWords];   // ancestor words of the workgroup's rows
  int u, rb, split;
  if (!decode_wg(a, u, rb, split)) return;
  const int b = u / a.Hkv;
  const int g = u - b * a.Hkv;
  const int n = a.n_nodes ? a.n_nodes[b] : a.N;
  const int P = a.prefix_len[b];
  const int M = a.N * a.G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  const __bf16* __restrict__ qp = static_cast<const __bf16*>(a.q);
  const __bf16* __restrict__ kp = static_cast<const __bf16*>(a.k);
  const __bf16* __restrict__ vp = static_cast<const __bf16*>(a.v);
  __bf16* __restrict__ op = static_cast<__bf16*>(a.out);

  if (!seq_valid(n, P, a.N, a.S_max)) {
    if (split == 0) {
      if (a.err && g == 0 && rb == 0 && tid == 0) a.err[b] = seq_err(n, P, a.N, a.S_max);
      for (int idx = tid; idx < RBS * D; idx += THREADS) {
        const int r = rb * RBS + idx / D;
        if (r >= M) continue;
        const int i = r / a.G, h = g * a.G + r % a.G;
        op[(((size_t)b * a.N + i) * a.Hq + h) * D + idx % D] = (__bf16)0.f;
        if (a.lse && idx % D == 0) a.lse[((size_t)b * a.N + i) * a.Hq + h] = -INFINITY;
      }
    }
    return;
  }
  if (a.err && g == 0 && rb == 0 && split == 0 && tid == 0) a.err[b] = 0;

  // Key range of this split, tile aligned.
  const int total = P + n;
  int span = (total + a.S - 1) / a.S;
  span = (span + kKT - 1) / kKT * kKT;
  const int k0 = split * span;
  const int k1 = min(total, k0 + span);

  // Rows of this lane: r = rb * RBS + wave * ROWS_WAVE + cb * 16 + l16.
  int row_node[CB];
  bool row_ok[CB];
  bf16x8 qf[CB][DS];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int r = rb * RBS + wave * ROWS_WAVE + cb * 16 + l16;
    const int i = r / a.G;
    row_node[cb] = i;
    row_ok[cb] = r < M && i < n;
    const int h = g * a.G + r % a.G;
    const __bf16* src = qp + (((size_t)b * a.N + i) * a.Hq + h) * D + 8 * lg;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      qf[cb][ds] = row_ok[cb] ? *reinterpret_cast<const bf16x8*>(src + ds * 32) : bf16x8{};
  }
  // The ancestor words of the workgroup's rows (W <= kMaxWords per row), requested with Q so
  // that no tile loads mask words behind the prefetch (the memory counter drains in issue
  // order), and kept in LDS: only tiles that reach the tree slots read them.  Word indices are
  // clamped into the row; a clamped word is never selected below.
  constexpr int MW_PER = (RBS * kMaxWords + THREADS - 1) / THREADS;
  uint64_t mw[MW_PER];
#pragma unroll
  for (int k = 0; k < MW_PER; ++k) {
    const int e = min(k * THREADS + tid, RBS * kMaxWords - 1);
    const int r = rb * RBS + e / kMaxWords;
    const int node = min(r / a.G, a.N - 1);
    mw[k] = a.mask[((size_t)b * a.N + node) * a.W + min(e % kMaxWords, a.W - 1)];
  }

  f32x4 o_acc[DB][CB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) o_acc[db][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Row sums of the weights are a 17th output block: A = ones in its first row, so element 0
  // of lanes 0..15 accumulates sum_k P[k][row l16] on the matrix cores, with the same bf16
  // weights as the product and the same rescaling.
  f32x4 o_sum[CB];
  float m_run[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    m_run[cb] = -INFINITY;
    o_sum[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bf16x8 ones_frag;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones_frag[e] = (__bf16)(l16 == 0 ? 1.f : 0.f);

  const size_t kv_base = ((size_t)b * a.Hkv + g) * (size_t)a.S_max * D;
  const uint32_t head_bytes = (uint32_t)a.S_max * (D * 2);   // < 2^31 (checked on the host)
  const BufRsrc krs = buf_rsrc(kp + kv_base, head_bytes);
  const BufRsrc vrs = buf_rsrc(vp + kv_base, head_bytes);
  const int ld_key = tid / CPK;
  const int ld_chunk = tid % CPK;
  // Next tile into registers, consumed only by the next stage(), so the loads stay in flight
  // while this tile is computed.  A key past the split loads the split's last key instead
  // (k1 >= 1 whenever a tile exists): finite data whose score is masked to -inf, so its weight
  // is exactly 0, and all lanes then read one address.
  bf16x8 kreg[PASSES], vreg[PASSES];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      const int s = min(t0 + pass * KPP + ld_key, k1 - 1);
      const uint32_t at = (uint32_t)s * (D * 2) + ld_chunk * 16;
      kreg[pass] = buf_ld8(krs, at);
      vreg[pass] = buf_ld8(vrs, at);
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      const int key = pass * KPP + ld_key;
      *reinterpret_cast<bf16x8*>(&k_lds[buf][key * KS + ld_chunk * 8]) = kreg[pass];
      *reinterpret_cast<bf16x8*>(&v_lds[buf][key * VS + ld_chunk * 8]) = vreg[pass];
    }
  };

  // Q and the ancestor words pass through an empty asm once the first tile is requested: the
  // compiler waits for their loads there, where it still counts exactly (they precede the
  // tile's loads, which stay in flight), and inside the loop they are plain registers.
  // Without it the loop's merged load state makes a tile re-wait for them at a count that
  // also drains the prefetch.
  auto settle = [&]() {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) asm volatile("" : "+v"(qf[cb][ds]));
#pragma unroll
    for (int k = 0; k < MW_PER; ++k) {
      const int e = k * THREADS + tid;
      if (e < RBS * kMaxWords) s_mask[e] = mw[k];
    }
  };
  if (k0 < k1) {
    fetch(k0);
    settle();
  } else {
    settle();
  }

  // ---- S^T = K Q^T for the 64 keys of the tile in buffer `buf`.  The MFMA blocks run at
  // raised wave priority: a wave that reaches one gets the issue slot first, so the two waves
  // of a SIMD drift apart and one's softmax (VALU) overlaps the other's products.
  auto qk = [&](int buf, f32x4 (&s_acc)[4][CB]) {
    const __bf16* kt = k_lds[buf];
    if (a.prio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) s_acc[kb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(&kt[(kb * 16 + l16) * KS + ds * 32 + 8 * lg]);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          s_acc[kb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[cb][ds], s_acc[kb][cb], 0, 0, 0);
      }
    }
    if (a.prio) __builtin_amdgcn_s_setprio(0);
  };

  // ---- mask (MASKED tiles only), online softmax in base 2, P^T packed as bf16, for the tile
  // starting at key t0.  The max is taken on raw scores (the scale is positive, so it commutes
  // with the max) and each weight is exp2(s * scale_log2 - m) with one FMA.  Rows past the
  // workload have Q = 0 and are discarded at the end, so wholly-prefix tiles need no per-score
  // select.  The reference max m_run moves only when a score exceeds it by more than a.lazy
  // (log2 units): softmax is the same for any reference, weights stay below 2^lazy, and the O
  // rescale is rarely needed.  alpha[cb] receives the factor the output accumulated so far must
  // take (1 where the reference did not move); returns whether any row of the wave moved.
  //
  // Fast path, once every live row of the wave has a reference: the weights are formed against
  // the current references straight away, and one integer max over their bf16 bit patterns
  // (non-negative bf16 values order like their bits; NaN sorts above every number) tells
  // whether any of them passed 2^lazy.  If none did, no reference moves and the tile needs no
  // row max at all; otherwise the tile takes the general path below, which forms the weights
  // again.  `ready` (wave-uniform) records that every live row has a finite reference.
  auto softmax = [&](auto masked, int t0, f32x4 (&s_acc)[4][CB], bf16x8 (&pb)[2][CB], float (&alpha)[CB],
                     bool& ready) {
    constexpr bool MASKED = decltype(masked)::value;
    // tree index of the tile's first key (negative inside the prefix); the ancestor words of
    // the tile's tree keys are word jw and jw + 1 (tree keys j < n <= 64 W)
    const int j0 = t0 - P;
    const int jw = j0 >> 6;                     // floor division
    const int lim = k1 - t0;                    // keys of the tile inside the split (>= 1)
    float x[CB][4][4];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[cb][kb][e] = s_acc[kb][cb][e];
      if constexpr (MASKED) {
        // Visibility of the tile's 64 keys for this row, bit i for key t0 + i: prefix keys
        // always, tree key j when bit j of the row's ancestor words is set, nothing past the
        // split or in a row past the workload.  Each lane then takes the 4 bits of each of its
        // key groups and turns a score into -inf with one bit-insert.
        const uint64_t* mrow = s_mask + (wave * ROWS_WAVE + cb * 16 + l16) * kMaxWords;
        const uint64_t wlo = mrow[min(max(jw, 0), kMaxWords - 1)];
        const uint64_t whi = mrow[min(max(jw + 1, 0), kMaxWords - 1)];
        uint64_t vis;
        if (j0 >= 0) {
          const int sh = j0 & 63;
          vis = sh ? (wlo >> sh) | (whi << (64 - sh)) : wlo;
        } else if (j0 > -64) {                  // jw = -1: whi is word 0, keys i < -j0 prefix
          const int sh = -j0;
          vis = (whi << sh) | ((1ull << sh) - 1);
        } else {
          vis = ~0ull;
        }
        if (lim < 64) vis &= (1ull << lim) - 1;
        if (!row_ok[cb]) vis = 0;
        const uint64_t mine = vis >> (4 * lg);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const uint32_t q = (uint32_t)(mine >> (16 * kb));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t keep = (uint32_t)__builtin_amdgcn_sbfe((int)q, e, 1);   // 0 or ~0
            x[cb][kb][e] = __uint_as_float((__float_as_uint(x[cb][kb][e]) & keep) | (0xff800000u & ~keep));
          }
        }
      }
    }
    auto pack = [&](int cb, const float (&w)[4][4]) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        bf16x8 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pk[e] = (__bf16)w[2 * c][e];
          pk[4 + e] = (__bf16)w[2 * c + 1][e];
        }
        pb[c][cb] = pk;
      }
    };
    if (ready) {
      u16x8 top = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const float m_use = (m_run[cb] == -INFINITY) ? 0.f : m_run[cb];   // rows past the workload
        float w[4][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int e = 0; e < 4; ++e) w[kb][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[cb][kb][e], a.scale_log2, -m_use));
        pack(cb, w);
#pragma unroll
        for (int c = 0; c < 2; ++c) top = __builtin_elementwise_max(top, __builtin_bit_cast(u16x8, pb[c][cb]));
      }
      const u16x4 t4 = __builtin_elementwise_max(top.lo, top.hi);
      const u16x2 t2 = __builtin_elementwise_max(t4.lo, t4.hi);
      const uint32_t t1 = t2.x > t2.y ? t2.x : t2.y;
      if (__ballot(t1 > a.lazy_bits) == 0) return false;
    }
    bool moved = false, unset = false;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float mloc = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) mloc = fmaxf(mloc, x[cb][kb][e]);
      mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_tile = mloc * a.scale_log2;
      const bool grow = m_tile > m_run[cb] + a.lazy;   // false while both are -inf
      alpha[cb] = grow ? __builtin_amdgcn_exp2f(m_run[cb] - m_tile) : 1.f;   // 0 from -inf
      m_run[cb] = grow ? m_tile : m_run[cb];
      moved = moved || __ballot(grow) != 0;
      unset = unset || (row_ok[cb] && m_run[cb] == -INFINITY);
      const float m_use = (m_run[cb] == -INFINITY) ? 0.f : m_run[cb];
      float w[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) w[kb][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[cb][kb][e], a.scale_log2, -m_use));
      pack(cb, w);
    }
    ready = __ballot(unset) == 0;
    return moved;
  };
  auto rescale = [&](const float (&alpha)[CB]) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      o_sum[cb] *= alpha[cb];
#pragma unroll
      for (int db = 0; db < DB; ++db) o_acc[db][cb] *= alpha[cb];
    }
  };
  // ---- O^T += V^T P^T with the tile in buffer `buf`.
  auto pv = [&](int buf, const bf16x8 (&pb)[2][CB]) {
    const __bf16* vt = v_lds[buf];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 af = v_fragment<VS>(vt, db * 16, c * 32, lg, l16);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          o_acc[db][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, pb[c][cb], o_acc[db][cb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        o_sum[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_frag, pb[c][cb], o_sum[cb], 0, 0, 0);
  };
  // wholly prefix and wholly inside the split: no mask
  auto is_plain = [&](int t0) { return t0 + kKT <= k1 && t0 + kKT <= P; };

  int buf = 0;
  bool ready = false;
  for (int t0 = k0; t0 < k1; t0 += kKT) {
    stage(buf);
    __syncthreads();
    fetch(t0 + kKT);   // unconditional (past the split it reloads its last key) so no branch
                       // leaves the compiler unsure how many loads are still in flight
    f32x4 s_acc[4][CB];
    qk(buf, s_acc);
    bf16x8 pb[2][CB];
    float alpha[CB];
    const bool moved = is_plain(t0) ? softmax(std::false_type{}, t0, s_acc, pb, alpha, ready)
                                    : softmax(std::true_type{}, t0, s_acc, pb, alpha, ready);
    if (moved) rescale(alpha);
    if (a.prio) __builtin_amdgcn_s_setprio(1);
    pv(buf, pb);
    if (a.prio) __builtin_amdgcn_s_setprio(0);
    buf ^= 1;
  }

  // Row sums: element 0 of lane l16 (the first 16 lanes) holds the sum of row l16.
  float l_run[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) l_run[cb] = __shfl(o_sum[cb][0], l16);

  if (a.S == 1) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int r = rb * RBS + wave * ROWS_WAVE + cb * 16 + l16;
      if (r >= M) continue;
      const int i = r / a.G, h = g * a.G + r % a.G;
      const bool live = row_ok[cb] && l_run[cb] > 0.f;
      const float inv = live ? 1.f / l_run[cb] : 0.f;
      __bf16* dst = op + (((size_t)b * a.N + i) * a.Hq + h) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(o_acc[db][cb][e] * inv);
        *reinterpret_cast<bf16x4*>(dst + db * 16 + 4 * lg) = o4;
      }
      if (a.lse && lg == 0)
        a.lse[((size_t)b * a.N + i) * a.Hq + h] = live ? (m_run[cb] + log2f(l_run[cb])) * kLn2 : -INFINITY;
    }
    return;
  }

  // ---- several splits: store each split's output normalised by its own sum (bf16, like the
  // final output; the merge takes a convex combination of them) and its (max, sum) in fp32.
  const size_t pbase = ((size_t)u * a.S + split) * a.Mpad;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) {
    const int r = rb * RBS + wave * ROWS_WAVE + cb * 16 + l16;
    const bool live = row_ok[cb] && l_run[cb] > 0.f;
    const float inv = live ? 1.f / l_run[cb] : 0.f;
    __bf16* dst = a.part_o + (pbase + r) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      bf16x4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(o_acc[db][cb][e] * inv);
      *reinterpret_cast<bf16x4*>(dst + db * 16 + 4 * lg) = o4;
    }
    if (lg == 0) a.part_ml[pbase + r] = make_float2(live ? m_run[cb] : -INFINITY, live ? l_run[cb] : 0.f);
  }
}

// Merge of the key splits.  Thread -> (row, 8 output dims), 16-byte loads; a workgroup covers
// 256 / (D / 8) rows of one unit.  The splits are folded with a running max, SB splits' loads
// issued together (SB >= S up to 8, so no load is repeated); the partial loads do not wait for
// the sequence's validity, which only decides the store.  Workgroups of a unit run on the
// unit's XCD (as in the main kernel), where its partials sit in L2.
template <int D, int SB>
__global__ __launch_bounds__(kThreads) void tree_attn_merge_kernel(AttnArgs a) {
  constexpr int C8 = D / 8;
  constexpr int ROWS = kThreads / C8;          // rows per workgroup (16 at D = 128)
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int per_unit = a.Mpad / ROWS;
  const int lu = slot / per_unit;
  const int u = xcd + 8 * lu;
  if (u >= a.B * a.Hkv) return;
  const int r = (slot - lu * per_unit) * ROWS + threadIdx.x / C8;
  const int d8 = threadIdx.x % C8;
  const int M = a.N * a.G;
  if (r >= M) return;
  const int b = u / a.Hkv, g = u - b * a.Hkv;
  const int n = a.n_nodes ? a.n_nodes[b] : a.N;
  const int P = a.prefix_len[b];
  float mrun = -INFINITY, L = 0.f;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  for (int s0 = 0; s0 < a.S; s0 += SB) {
    float2 ml[SB];
    bf16x8 po[SB];
#pragma unroll
    for (int k = 0; k < SB; ++k) {
      const int s = min(s0 + k, a.S - 1);
      const size_t pr = ((size_t)u * a.S + s) * a.Mpad + r;
      ml[k] = a.part_ml[pr];
      po[k] = *reinterpret_cast<const bf16x8*>(a.part_o + pr * D + 8 * d8);
    }
#pragma unroll
    for (int k = 0; k < SB; ++k) {
      if (s0 + k >= a.S || ml[k].x == -INFINITY) continue;
      const float mn = fmaxf(mrun, ml[k].x);
      const float sc_old = __builtin_amdgcn_exp2f(mrun - mn);   // 0 when mrun = -inf
      const float w = ml[k].y * __builtin_amdgcn_exp2f(ml[k].x - mn);   // this split's weight
      L = L * sc_old + w;
      f32x4 p0, p1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p0[e] = (float)po[k][e];
        p1[e] = (float)po[k][4 + e];
      }
      acc0 = acc0 * sc_old + p0 * w;
      acc1 = acc1 * sc_old + p1 * w;
      mrun = mn;
    }
  }
  if (!seq_valid(n, P, a.N, a.S_max)) return;  // the main kernel wrote zeros and the error
  const int i = r / a.G, h = g * a.G + r % a.G;
  const bool live = i < n && L > 0.f;
  const float inv = live ? 1.f / L : 0.f;
  bf16x8 o8;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o8[e] = (__bf16)(acc0[e] * inv);
    o8[4 + e] = (__bf16)(acc1[e] * inv);
  }
  __bf16* op = static_cast<__bf16*>(a.out);
  *reinterpret_cast<bf16x8*>(op + (((size_t)b * a.N + i) * a.Hq + h) * D + 8 * d8) = o8;
  if (a.lse && d8 == 0) a.lse[((size_t)b * a.N + i) * a.Hq + h] = live ? (mrun + log2f(L)) * kLn2 : -INFINITY;
}

// Exact fp32 path: one workgroup of 256 threads per query row (b, node, head).  Keys are taken
// 256 at a time: each thread scores one key, the chunk is folded into a running max / sum,
// and thread t accumulates output dimension t % D over the keys t / D, t / D + 256 / D, ...
template <int D>
__global__ __launch_bounds__(256) void tree_attn_f32_kernel(AttnArgs a) {
  constexpr int SLICES = 256 / D;
  __shared__ float q_s[D];
  __shared__ float p_s[256];
  __shared__ float red[256];
  __shared__ float o_s[256];
  const int row = blockIdx.x;
  const int h = row % a.Hq;
  const int i = (row / a.Hq) % a.N;
  const int b = row / (a.Hq * a.N);
  const int g = h / a.G;
  const int tid = threadIdx.x;
  const int n = a.n_nodes ? a.n_nodes[b] : a.N;
  const int P = a.prefix_len[b];
  const float* qp = static_cast<const float*>(a.q);
  const float* kp = static_cast<const float*>(a.k);
  const float* vp = static_cast<const float*>(a.v);
  float* op = static_cast<float*>(a.out) + (((size_t)b * a.N + i) * a.Hq + h) * D;
  const bool valid = seq_valid(n, P, a.N, a.S_max);
  if (a.err && i == 0 && h == 0 && tid == 0) a.err[b] = seq_err(n, P, a.N, a.S_max);
  if (!valid || i >= n) {
    if (tid < D) op[tid] = 0.f;
    if (a.lse && tid == 0) a.lse[((size_t)b * a.N + i) * a.Hq + h] = -INFINITY;
    return;
  }
  if (tid < D) q_s[tid] = qp[(((size_t)b * a.N + i) * a.Hq + h) * D + tid];
  const uint64_t* mrow = a.mask + ((size_t)b * a.N + i) * a.W;
  const size_t kv_base = ((size_t)b * a.Hkv + g) * (size_t)a.S_max * D;
  const float scale = a.scale;
  __syncthreads();

  const int total = P + n;
  float m_run = -INFINITY, l_run = 0.f, o_run = 0.f;
  const int dcol = tid % D, slice = tid / D;
  for (int c0 = 0; c0 < total; c0 += 256) {
    const int s = c0 + tid;
    float sc = -INFINITY;
    bool vis = s < total;
    if (vis && s >= P) vis = (mrow[(s - P) >> 6] >> ((s - P) & 63)) & 1ull;
    if (vis) {
      const float* krow = kp + kv_base + (size_t)s * D;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(q_s[d], krow[d], dot);
      sc = dot * scale;
    }
    red[tid] = sc;
    __syncthreads();
    for (int st = 128; st > 0; st >>= 1) {
      if (tid < st) red[tid] = fmaxf(red[tid], red[tid + st]);
      __syncthreads();
    }
    const float cmax = red[0];
    __syncthreads();
    const float m_new = fmaxf(m_run, cmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = expf(m_run - m_use);
    const float p = expf(sc - m_use);
    p_s[tid] = p;
    red[tid] = p;
    __syncthreads();
    for (int st = 128; st > 0; st >>= 1) {
      if (tid < st) red[tid] += red[tid + st];
      __syncthreads();
    }
    l_run = l_run * alpha + red[0];
    o_run *= alpha;
    for (int kk = slice; kk < 256; kk += SLICES) {
      const int s2 = c0 + kk;
      if (s2 < total && p_s[kk] != 0.f) o_run = fmaf(p_s[kk], vp[kv_base + (size_t)s2 * D + dcol], o_run);
    }
    m_run = m_new;
    __syncthreads();
  }
  o_s[tid] = o_run;
  __syncthreads();
  if (tid < D) {
    float o = 0.f;
    for (int sl = 0; sl < SLICES; ++sl) o += o_s[sl * D + tid];
    op[tid] = l_run > 0.f ? o / l_run : 0.f;
  }
  if (a.lse && tid == 0)
    a.lse[((size_t)b * a.N + i) * a.Hq + h] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
}

struct Plan {
  int CB, WAVES, RBS, R, S, Mpad, units, wgs, lpt;
};

// Launch shape.  Few (sequence, KV head) units -> 64-row workgroups (4 waves of 16 rows) and
// more key splits so that all CUs work; many units -> 256-row workgroups (8 waves of 32 rows:
// the K/V tile in LDS serves 4x more rows per read) and few splits.  Splits are chosen for
// about 256 workgroups (one round; an unsplit problem needs no merge), at least two for a large
// batch (its sequences may differ in length), and every split keeps at least two tiles.
// The tuning overrides attn_cb, attn_waves, attn_splits and attn_lpt force the choice (tests;
// results do not depend on them).
// Shapes both paths accept: sizes in range and a grid that fits (checked in 64-bit before any
// 32-bit arithmetic of the plan).  Shared by the workspace query and the call.
spec_status check_shape(int B, int N, int Hq, int Hkv, int head_dim, int S_max, int dtype) {
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES || Hq < 1 || Hkv < 1 || S_max < 1) return SPEC_EINVAL;
  if (Hq % Hkv != 0) return SPEC_EUNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return SPEC_EUNSUPPORTED;
  if ((long long)S_max * head_dim * 2 >= kMaxHeadCacheBytes) return SPEC_EUNSUPPORTED;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EUNSUPPORTED;
  // fp32: one workgroup per query row; bf16: at most (units rounded to 8) x row blocks x splits
  // with splits <= S_max / 128 + 1 and row blocks <= N * G / 64 + 1
  const long long units = (long long)B * Hkv;
  const long long rows = (long long)N * (Hq / Hkv);
  if ((long long)B * N * Hq > INT_MAX / 2 || units > INT_MAX / 8) return SPEC_EUNSUPPORTED;
  if ((units + 8) * (rows / 64 + 1) * ((long long)S_max / 128 + 1) > INT_MAX / 2) return SPEC_EUNSUPPORTED;
  return SPEC_OK;
}

Plan make_plan(int B, int N, int Hq, int Hkv, int D, int S_max) {
  Plan p{};
  const int G = Hq / Hkv;
  const int M = N * G;
  p.units = B * Hkv;
  const int big = p.units * ((M + 255) / 256) >= 64;
  p.CB = tuning(kKnobAttnCB, big ? 2 : 1);
  p.WAVES = tuning(kKnobAttnWaves, big ? 8 : 4);
  if (p.CB != 1 && p.CB != 2) p.CB = 1;
  if (p.WAVES != 4 && p.WAVES != 8) p.WAVES = 4;
  p.RBS = p.WAVES * 16 * p.CB;
  p.R = (M + p.RBS - 1) / p.RBS;
  p.Mpad = p.R * p.RBS;
  const int target = 256;   // one workgroup per CU, all in one round (measured best)
  const int tiles = S_max / kKT + (S_max % kKT != 0);
  int S = (target + p.units * p.R - 1) / (p.units * p.R);
  // Batches may mix prefix lengths: at least two splits, taken longest sequence first, so that
  // the halves of long sequences are not left running alone at the end.
  p.lpt = B >= 2 && B <= kMaxLptSeqs;
  if (big && p.lpt && S < 2) S = 2;
  S = tuning(kKnobAttnSplits, S);
  p.lpt = tuning(kKnobAttnLpt, p.lpt) != 0 && B >= 2 && B <= kMaxLptSeqs;
  if (S > tiles / 2) S = tiles / 2;
  if (S < 1) S = 1;
  p.S = S;
  const int per_xcd = (p.units + 7) / 8;
  p.wgs = 8 * per_xcd * p.R * p.S;
  return p;
}

template <int D>
void launch_bf16(const Plan& p, const AttnArgs& a, hipStream_t s) {
  const dim3 grid(p.wgs);
  const char* nm = "tree_attn_bf16";
  if (p.WAVES == 8) {
    if (p.CB == 2) launch(nm, tree_attn_bf16_kernel<D, 2, 8>, grid, dim3(8 * kWave), s, a);
    else launch(nm, tree_attn_bf16_kernel<D, 1, 8>, grid, dim3(8 * kWave), s, a);
  } else {
    if (p.CB == 2) launch(nm, tree_attn_bf16_kernel<D, 2, 4>, grid, dim3(4 * kWave), s, a);
    else launch(nm, tree_attn_bf16_kernel<D, 1, 4>, grid, dim3(4 * kWave), s, a);
  }
}

size_t workspace_bytes(const Plan& p, int D) {
  if (p.S == 1) return 0;
  size_t off = align_up((size_t)p.units * p.S * p.Mpad * sizeof(float2), 256);
  off += align_up((size_t)p.units * p.S * p.Mpad * D * sizeof(__bf16), 256);
  return off;
}

}  // namespace
}  // namespace spectree

using namespace spectree;

extern "C" size_t spec_tree_attn_workspace(int B, int N, int Hq, int Hkv, int head_dim, int S_max,
                                           int dtype) {
  if (check_shape(B, N, Hq, Hkv, head_dim, S_max, dtype) != SPEC_OK || dtype != SPEC_BF16) return 0;
  return workspace_bytes(make_plan(B, N, Hq, Hkv, head_dim, S_max), head_dim);
}

extern "C" spec_status spec_tree_attn(const void* q, const void* k_cache, const void* v_cache,
                                      const int32_t* prefix_len, const uint64_t* tree_mask,
                                      const int32_t* n_nodes, int B, int N, int Hq, int Hkv,
                                      int head_dim, int S_max, float scale, int dtype,
                                      void* out, float* lse, int32_t* err, void* workspace,
                                      size_t ws_bytes, void* stream) {
  if (B < 1 || N < 1 || N > SPEC_MAX_NODES || Hq < 1 || Hkv < 1 || S_max < 1) return SPEC_EINVAL;
  if (!q || !k_cache || !v_cache || !prefix_len || !tree_mask || !out) return SPEC_EINVAL;
  const spec_status shape = check_shape(B, N, Hq, Hkv, head_dim, S_max, dtype);
  if (shape != SPEC_OK) return shape;
  if (!(scale > 0.f) || !(scale < INFINITY)) return SPEC_EINVAL;   // positive and finite
  hipStream_t s = static_cast<hipStream_t>(stream);

  AttnArgs a{};
  a.q = q; a.k = k_cache; a.v = v_cache; a.prefix_len = prefix_len; a.mask = tree_mask;
  a.n_nodes = n_nodes; a.B = B; a.N = N; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
  a.S_max = S_max; a.W = (N + 63) / 64; a.scale = scale; a.scale_log2 = scale * kLog2e;
  a.out = out; a.lse = lse; a.err = err;

  if (dtype == SPEC_F32) {
    const dim3 grid(B * N * Hq);
    if (head_dim == 64) launch("tree_attn_f32", tree_attn_f32_kernel<64>, grid, dim3(256), s, a);
    else launch("tree_attn_f32", tree_attn_f32_kernel<128>, grid, dim3(256), s, a);
    return launch_status();
  }

  const Plan p = make_plan(B, N, Hq, Hkv, head_dim, S_max);
  const size_t need = workspace_bytes(p, head_dim);
  if (need > 0 && (!workspace || ws_bytes < need)) return SPEC_EWORKSPACE;
  a.R = p.R; a.S = p.S; a.Mpad = p.Mpad;
  a.prio = tuning(kKnobAttnPrio, 1);
  const int lazy = std::max(0, tuning(kKnobAttnLazy, kLazy));
  a.lazy = (float)lazy;
  a.lazy_bits = lazy < 128 ? (uint32_t)(127 + lazy) << 7 : 0x7F80u;   // 2^lazy, or +inf
  a.lpt = p.lpt;
  if (p.S > 1) {
    char* w = static_cast<char*>(workspace);
    size_t off = 0;
    a.part_ml = reinterpret_cast<float2*>(w + off);
    off += align_up((size_t)p.units * p.S * p.Mpad * sizeof(float2), 256);
    a.part_o = reinterpret_cast<__bf16*>(w + off);
  }
  if (head_dim == 128) launch_bf16<128>(p, a, s);
  else launch_bf16<64>(p, a, s);
  if (p.S > 1) {
    const int rows_per_wg = kThreads / (head_dim / 8);
    const dim3 mgrid(8 * ((p.units + 7) / 8) * (p.Mpad / rows_per_wg));
    const char* mn = "tree_attn_merge";
    const dim3 mb(kThreads);
    if (head_dim == 128) {
      if (p.S <= 2) launch(mn, tree_attn_merge_kernel<128, 2>, mgrid, mb, s, a);
      else if (p.S <= 4) launch(mn, tree_attn_merge_kernel<128, 4>, mgrid, mb, s, a);
      else launch(mn, tree_attn_merge_kernel<128, 8>, mgrid, mb, s, a);
    } else {
      if (p.S <= 2) launch(mn, tree_attn_merge_kernel<64, 2>, mgrid, mb, s, a);
      else if (p.S <= 4) launch(mn, tree_attn_merge_kernel<64, 4>, mgrid, mb, s, a);
      else launch(mn, tree_attn_merge_kernel<64, 8>, mgrid, mb, s, a);
    }
  }
  return launch_status();
}
