// Internal helpers shared by the HIP sources of libspectree (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spectree.h"

namespace spectree {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ int err_word(int node, int code) { return (node << 8) | code; }

// Wave-wide reductions (64 lanes).  __shfl_xor lowers to DPP / ds_swizzle / bpermute.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// ---------------------------------------------------------------- host side

// Kernel timing hooks (runtime.hip).  prof_begin returns an opaque token passed to prof_end.
int prof_begin(const char* name, hipStream_t stream);
void prof_end(int token, hipStream_t stream);

struct ProfScope {
  int token;
  hipStream_t stream;
  ProfScope(const char* name, hipStream_t s) : token(prof_begin(name, s)), stream(s) {}
  ~ProfScope() { prof_end(token, stream); }
};

inline spec_status launch_status() {
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace spectree
