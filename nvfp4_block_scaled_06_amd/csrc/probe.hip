// Streaming-read probe: the time one launch needs to read a buffer once,
// with 16-byte loads spread over as many workgroups as the buffer allows.
// It measures the bandwidth a kernel can reach for a given footprint (HBM at
// a gigabyte, launch and cache latency at the decode gate's megabyte), the
// denominator against which the gate kernels' own rates are read. Not part
// of the router path.
#include "../../include/nvfp4_router.h"
#include "router_internal.hpp"

namespace nvr {

constexpr int kProbeThreads = 256;
constexpr int kProbeMaxGrid = 8192;

// Buffers larger than the Infinity Cache are streamed with nontemporal loads
// (the faster way to read HBM once); smaller ones with ordinary loads, which
// the caches keep.
constexpr int64_t kProbeStreamBytes = 256ll << 20;

template <bool NT>
__device__ __forceinline__ u32x4_t probe_load(const u32x4_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}

template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4_t* __restrict__ p, int64_t nvec,
                                                                   uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[kProbeThreads / 64];
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + 3 * stride < nvec; i += 4 * stride) {
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = probe_load<NT>(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < nvec; i += stride) {
    const u32x4_t v = probe_load<NT>(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// MFMA probe: every wavefront runs `iters` rounds of four independent
// 32x32x16 f16 MFMA chains (no memory traffic in the loop), then stores one
// float per thread so the work is kept. Launched with four wavefronts per
// SIMD on every compute unit, it measures the matrix-core rate the chip
// sustains at its running clock.
constexpr int kMfmaProbeGrid = 1024;  // workgroups of 256 threads: 4 per CU, one wavefront each per SIMD

__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(int iters, float* __restrict__ sink) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  typedef float f16x __attribute__((ext_vector_type(16)));
  const int lane = threadIdx.x & 63;
  h8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)((lane + i) & 7) * (_Float16)0.125f;
    b[i] = (_Float16)((lane * 3 + i) & 7) * (_Float16)0.0625f;
  }
  f16x acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
  }
  float r = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) r += acc[j][v];
  sink[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = r;
}

}  // namespace nvr

extern "C" int router_probe_mfma(int64_t iters, float* sink, size_t sink_floats, void* stream) {
  if (iters < 1 || iters > (int64_t(1) << 24) || !sink || reinterpret_cast<uintptr_t>(sink) % 4 != 0 ||
      sink_floats < (size_t)nvr::kMfmaProbeGrid * nvr::kProbeThreads)
    return ROUTER_EINVAL;
  nvr::probe_mfma_kernel<<<nvr::kMfmaProbeGrid, nvr::kProbeThreads, 0, static_cast<hipStream_t>(stream)>>>((int)iters,
                                                                                                          sink);
  return hipGetLastError() == hipSuccess ? ROUTER_OK : ROUTER_EHIP;
}

extern "C" int router_probe_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words, void* stream) {
  if (!buf || !sink || sink_words == 0 || bytes == 0 || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(buf) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
    return ROUTER_EINVAL;
  const int64_t nvec = (int64_t)(bytes / 16);
  int64_t grid = (nvec + nvr::kProbeThreads - 1) / nvr::kProbeThreads;
  if (grid > (int64_t)sink_words) grid = (int64_t)sink_words;
  if (grid > nvr::kProbeMaxGrid) grid = nvr::kProbeMaxGrid;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const nvr::u32x4_t* p = static_cast<const nvr::u32x4_t*>(buf);
  if ((int64_t)bytes > nvr::kProbeStreamBytes)
    nvr::probe_read_kernel<true><<<(int)grid, nvr::kProbeThreads, 0, s>>>(p, nvec, sink);
  else
    nvr::probe_read_kernel<false><<<(int)grid, nvr::kProbeThreads, 0, s>>>(p, nvec, sink);
  return hipGetLastError() == hipSuccess ? ROUTER_OK : ROUTER_EHIP;
}
