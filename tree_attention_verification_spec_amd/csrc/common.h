// Internal helpers shared by the HIP sources of libspectree (gfx950 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>
#include <utility>

#include "spectree.h"
#include "internal.h"

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
// registered under `name` and returns true; the launch then goes through hipExtLaunchKernel,
// whose events are stamped by the kernel's own dispatch, so they bracket exactly that kernel's
// execution on `stream`.
bool prof_pair(const char* name, hipEvent_t* start, hipEvent_t* stop);

// Launch status of the calling thread's current library call: the first failed launch since
// the last launch_status() (runtime.hip).
void note_launch(hipError_t r);

// Launches `kernel` with its arguments converted to the kernel's parameter types; the
// launch's own return code is recorded (an error left pending by an earlier, unrelated HIP
// call is not reported against this one).
template <typename... KArgs, typename... Args>
inline void launch(const char* name, void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                   Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  std::tuple<std::decay_t<KArgs>...> vals(std::forward<Args>(args)...);
  void* argv[sizeof...(KArgs)];
  std::apply([&argv](auto&... v) {
    int i = 0;
    ((argv[i++] = static_cast<void*>(&v)), ...);
  }, vals);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t r;
  if (prof_pair(name, &e0, &e1)) {
    r = hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, stream, e0, e1, 0);
  } else {
    r = hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, stream);
  }
  note_launch(r);
}

// SPEC_OK unless a launch of this call failed; clears the record for the next call.
spec_status launch_status();

// Tuning overrides (runtime.hip): launch-shape choices that tests force through
// spec_internal_tune() (internal.h), never read from the environment.  Results do not depend
// on them.  tuning() returns the forced value, or `fallback` when none is set.
enum Knob {
  kKnobAttnCB, kKnobAttnWaves, kKnobAttnSplits, kKnobAttnLpt, kKnobAttnPrio, kKnobAttnLazy,
  kKnobVerifyChunk, kKnobVerifyStoreW, kKnobVerifyRowsList,
  kKnobResRowBlocks, kKnobLmRowBlocks, kKnobWalkParts, kKnobWalkSpin,
  kKnobCount
};
int tuning(Knob k, int fallback);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace spectree
