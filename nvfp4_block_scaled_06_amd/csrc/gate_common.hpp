// Device helpers shared by the gate kernels (gfx950 only): MFMA wrappers,
// compile-time loops, operand chunk loads and the cross-workgroup logits
// handoff.
#pragma once

#include "nvfp4_device.hpp"
#include "router_internal.hpp"

namespace nvr {

__device__ __forceinline__ f32x4_t mfma16(half8_t a, half8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32(half8_t a, half8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Compile-time loop: f(IntC<I>{}) for I = B .. E-1.
template <int V>
struct IntC {
  static constexpr int value = V;
};
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IntC<B>{});
    static_for<B + 1, E>(f);
  }
}

// 32 elements of one row starting at element k0 (a multiple of 32): 16 code
// bytes and the 2 scale bytes of its two blocks; zeros when masked off.
struct Chunk32 {
  u32x4_t c;
  uint32_t s;
};

__device__ __forceinline__ Chunk32 load_chunk(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                              int64_t row, int64_t D, int64_t k0, bool ok) {
  Chunk32 ch;
  ch.c = u32x4_t{0u, 0u, 0u, 0u};
  ch.s = 0u;
  if (ok) {
    ch.c = *reinterpret_cast<const u32x4_t*>(codes + row * (D / 2) + k0 / 2);
    ch.s = *reinterpret_cast<const uint16_t*>(scales + row * (D / 16) + k0 / 16);
  }
  return ch;
}

// Cross-workgroup handoff of the logits without agent-scope fences (on gfx950
// those write back and invalidate the whole L2 and cost tens of
// microseconds per launch). Logits are written and read with agent-scope
// atomic stores and loads, which go to the device-coherent level and bypass
// the non-coherent caches. Each thread waits for its own stores to complete
// before the workgroup barrier, and only then does one thread count the
// workgroup's arrival; the workgroup that arrives last reads every logit.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Counts this workgroup's arrival and reports (uniformly) whether it is the
// last of `total`. The counter goes back to zero in release_counter().
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t total, uint32_t* s_flag) {
  __builtin_amdgcn_s_waitcnt(0);  // this thread's coherent stores have completed
  __syncthreads();
  if (threadIdx.x == 0)
    *s_flag = (__hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == total - 1) ? 1u : 0u;
  __syncthreads();
  return *s_flag != 0u;
}

// A uniform fp32 operand in device memory, read with a vector load where the
// call stands: the compiler would otherwise sink a scalar load of it to its
// first use and expose a whole memory round trip there.
__device__ __forceinline__ float load_early(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void release_counter(uint32_t* counter) {
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


}  // namespace nvr
