// Internal helpers shared by the HIP sources of libspectree (gfx950 only).
#pragma once

#include <hip/hip_ext.h>
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

// Kernel timing (runtime.hip).  When timing is on, prof_pair() creates a start/stop event pair
// registered under `name` and returns true; the launch then goes through
// hipExtLaunchKernelGGL, whose events are stamped by the kernel's own dispatch, so they bracket
// exactly that kernel's execution on `stream`.
bool prof_pair(const char* name, hipEvent_t* start, hipEvent_t* stop);

template <typename F, typename... Args>
inline void launch(const char* name, F kernel, dim3 grid, dim3 block, hipStream_t stream, Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (prof_pair(name, &e0, &e1)) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, e0, e1, 0, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
  }
}

inline spec_status launch_status() {
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace spectree
