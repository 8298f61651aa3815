// Runtime NVFP4 quantization of a bf16 tensor (gfx950).
//
// One global scale per call, computed on the device (commit df05289d,
// dsv4/layers/grouped_linear.py: one flattened quantize launch, no host
// sync for gsa): gsa = fp32(max|x|) / 2688 (commit 04cf8ca8,
// dsv4/layers/router.py, runtime-gsa paragraph). Rows are contiguous and D is
// a multiple of 16, so the tensor is a flat array of 16-element blocks: block
// b reads 32 bytes of x at 32 b and writes 8 code bytes at 8 b and one scale
// byte at b.
//
// Two shapes of launch:
//  * small tensors (<= kSingleBlocks blocks): one workgroup loads every block
//    into registers, reduces max|x|, derives gsa and quantizes from registers
//    (x read once, one launch);
//  * large tensors: amax_partial_kernel writes one max per workgroup, then
//    quant_kernel folds those partial maxima in every workgroup (a few KB from
//    L2), derives the same gsa everywhere and quantizes (x read twice: a
//    tensor-wide max has to be known before the first code is written; up to
//    160 MB the second read comes from the Infinity Cache).
#include "nvfp4_device.hpp"
#include "router_internal.hpp"

namespace nvr {

constexpr int kSingleThreads = 512;
constexpr int kSingleBlocksPerThread = 4;

__device__ __forceinline__ float gsa_from_absmax_bits(uint32_t m) {
  return __uint_as_float(m << 16) / kGsaDivisor;  // IEEE fp32 division
}

__device__ __forceinline__ void load_block(const u32x4_t* __restrict__ x, int64_t b, uint32_t* w) {
  const u32x4_t v0 = x[2 * b];
  const u32x4_t v1 = x[2 * b + 1];
  w[0] = v0[0]; w[1] = v0[1]; w[2] = v0[2]; w[3] = v0[3];
  w[4] = v1[0]; w[5] = v1[1]; w[6] = v1[2]; w[7] = v1[3];
}

__device__ __forceinline__ uint32_t vec_absmax(u32x4_t v) {
  return max(max(bf16_pair_absmax(v[0]), bf16_pair_absmax(v[1])), max(bf16_pair_absmax(v[2]), bf16_pair_absmax(v[3])));
}

__device__ __forceinline__ uint32_t block_absmax(const uint32_t* w) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, bf16_pair_absmax(w[i]));
  return m;
}

// The quantizer's common case: gsa in [2^-80, 2^100] (every tensor whose
// magnitude is not extreme), decided once per launch. The block scale and
// the codes then take block_scale's and encode8's fast path with no
// double-precision fallback in the loop (a per-block choice would have the
// compiler evaluate the fallback's division for every block). rcp6 is
// rcp(6 gsa), hoisted out of the loop.
__device__ __forceinline__ bool gsa_fast(float gsa) { return gsa >= 0x1p-80f && gsa <= 0x1p100f; }

__device__ __forceinline__ void quant_block16_fast(const uint32_t* w, float gsa, float rcp6, uint32_t& c0,
                                                   uint32_t& c1, uint32_t& sbyte) {
  const float bmax = __uint_as_float(bf16_block_absmax(w) << 16);
  const float p = bmax * rcp6;
  sbyte = near_scale_key(p) < kNearScaleLimit ? e4m3_byte_exact(bmax, p, gsa) : e4m3_from_f32(fminf(p, 448.0f));
  const float S = e4m3_value(sbyte);
  const float inv = S > 0.0f ? __builtin_amdgcn_rcpf(gsa * S) : 0.0f;
  c0 = fp4_exact8(w, inv, S, gsa);
  c1 = fp4_exact8(w + 4, inv, S, gsa);
}

// Workgroup-wide max of a per-thread value (blockDim.x threads, multiple of 64).
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  v = wave_max_u32(v);
  const int wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  uint32_t m = 0;
  for (int i = 0; i < nwaves; ++i) m = max(m, red[i]);
  return m;
}

__global__ __launch_bounds__(kSingleThreads) void quant_single_kernel(const u32x4_t* __restrict__ x, int64_t nblocks,
                                                                      const float* __restrict__ gsa_override,
                                                                      uint2* __restrict__ codes,
                                                                      uint8_t* __restrict__ scales,
                                                                      float* __restrict__ gsa_out) {
  __shared__ uint32_t red[kSingleThreads / 64];
  uint32_t w[kSingleBlocksPerThread][8];
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < kSingleBlocksPerThread; ++j) {
    const int64_t b = threadIdx.x + (int64_t)j * kSingleThreads;
    if (b < nblocks) {
      load_block(x, b, w[j]);
      m = max(m, block_absmax(w[j]));
    }
  }
  float gsa;
  if (gsa_override) {
    gsa = *gsa_override;
  } else {
    gsa = gsa_from_absmax_bits(block_max_u32(m, red));
  }
  if (threadIdx.x == 0) *gsa_out = gsa;
  const bool fast = gsa_fast(gsa);
  const float rcp6 = __builtin_amdgcn_rcpf(6.0f * gsa);
#pragma unroll
  for (int j = 0; j < kSingleBlocksPerThread; ++j) {
    const int64_t b = threadIdx.x + (int64_t)j * kSingleThreads;
    if (b < nblocks) {
      uint32_t c0, c1, s;
      if (fast) quant_block16_fast(w[j], gsa, rcp6, c0, c1, s);
      else quant_block16(w[j], gsa, c0, c1, s);
      codes[b] = make_uint2(c0, c1);
      scales[b] = (uint8_t)s;
    }
  }
}

constexpr int kAmaxThreads = 256;
// Loads in flight per thread in the max pass: two measured best (amax +
// quantize at T = 8192, D = 7168: 45.5-45.7 us against 46.2-46.5 with four
// and one; at T = 32768, streaming: 181.4-181.7 against 185.0 with three,
// 187.8-189.5 with four or one, 203 with eight).
constexpr int kAmaxUnroll = 2;

// Tensors up to this size are read by the max pass with ordinary loads, so
// that they stay in the 256 MB Infinity Cache for the quantize pass; larger
// ones would only evict each other there and stream with nontemporal loads.
constexpr int64_t kAmaxCachedBytes = 160ll << 20;

template <bool NT>
__device__ __forceinline__ u32x4_t amax_load(const u32x4_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}

template <bool NT>
__global__ __launch_bounds__(kAmaxThreads) void amax_partial_kernel(const u32x4_t* __restrict__ x, int64_t nvec,
                                                                    uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[kAmaxThreads / 64];
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * kAmaxThreads;
  int64_t i = (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x;
  for (; i + (kAmaxUnroll - 1) * stride < nvec; i += kAmaxUnroll * stride) {
    u32x4_t v[kAmaxUnroll];
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) v[u] = amax_load<NT>(x + i + u * stride);
#pragma unroll
    for (int u = 0; u < kAmaxUnroll; ++u) m = max(m, vec_absmax(v[u]));
  }
  for (; i < nvec; i += stride) {
    m = max(m, vec_absmax(amax_load<NT>(x + i)));
  }
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

constexpr int kQuantThreads = 512;

__global__ __launch_bounds__(kQuantThreads) void quant_kernel(const u32x4_t* __restrict__ x, int64_t nblocks,
                                                              const uint32_t* __restrict__ partial, int npartial,
                                                              const float* __restrict__ gsa_override,
                                                              uint2* __restrict__ codes,
                                                              uint8_t* __restrict__ scales,
                                                              float* __restrict__ gsa_out) {
  __shared__ uint32_t red[kQuantThreads / 64];
  float gsa;
  if (gsa_override) {
    gsa = *gsa_override;
  } else {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < npartial; i += kQuantThreads) m = max(m, partial[i]);
    gsa = gsa_from_absmax_bits(block_max_u32(m, red));
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *gsa_out = gsa;
  const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
  const int64_t b0 = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
  if (gsa_fast(gsa)) {  // uniform
    const float rcp6 = __builtin_amdgcn_rcpf(6.0f * gsa);
    for (int64_t b = b0; b < nblocks; b += stride) {
      uint32_t w[8];
      load_block(x, b, w);
      uint32_t c0, c1, s;
      quant_block16_fast(w, gsa, rcp6, c0, c1, s);
      codes[b] = make_uint2(c0, c1);
      scales[b] = (uint8_t)s;
    }
  } else {
    for (int64_t b = b0; b < nblocks; b += stride) {
      uint32_t w[8];
      load_block(x, b, w);
      uint32_t c0, c1, s;
      quant_block16(w, gsa, c0, c1, s);
      codes[b] = make_uint2(c0, c1);
      scales[b] = (uint8_t)s;
    }
  }
}

__global__ void fill_zero_kernel(uint32_t* __restrict__ p, int64_t nwords) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

size_t quantize_scratch_bytes() { return (size_t)kAmaxPartials * sizeof(uint32_t); }

hipError_t launch_quantize(const void* x, int64_t rows, int64_t D, const float* gsa_override, uint8_t* codes,
                           uint8_t* scales, float* gsa_out, void* scratch, hipStream_t stream) {
  const int64_t nblocks = rows * (D / 16);
  const u32x4_t* xv = static_cast<const u32x4_t*>(x);
  uint2* cv = reinterpret_cast<uint2*>(codes);
  static_assert(kSingleThreads * kSingleBlocksPerThread == kSingleWgMaxBlocks, "single-WG capacity");
  if (nblocks <= kSingleWgMaxBlocks) {
    quant_single_kernel<<<1, kSingleThreads, 0, stream>>>(xv, nblocks, gsa_override, cv, scales, gsa_out);
    return hipGetLastError();
  }
  uint32_t* partial = static_cast<uint32_t*>(scratch);
  int npartial = 0;
  if (!gsa_override) {
    const int64_t nvec = nblocks * 2;
    const int64_t want = (nvec + kAmaxThreads * 8 - 1) / (kAmaxThreads * 8);
    npartial = (int)(want < kAmaxPartials ? (want < 1 ? 1 : want) : kAmaxPartials);
    if (nvec * 16 <= kAmaxCachedBytes)
      amax_partial_kernel<false><<<npartial, kAmaxThreads, 0, stream>>>(xv, nvec, partial);
    else
      amax_partial_kernel<true><<<npartial, kAmaxThreads, 0, stream>>>(xv, nvec, partial);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // Equal grid-stride passes for every thread: a last pass that only part of
  // the threads take would cost the whole VALU issue of one. Workgroups of
  // 512 threads, each folding the partial maxima once. When x is small enough
  // to be re-read from the Infinity Cache, at most 2048 of them (four blocks
  // per thread at T = 8192, D = 7168: 48.7-49.6 us with 7168 workgroups of
  // 256, 47.1-47.4 with 3584, 46.3-47.2 with 1792 of 512); streaming x from
  // HBM, up to 8192 keep more loads in flight (T = 32768: 186.0-187.9 us
  // against 189.2-190.5 with 8192 of 256, 188.7-189.6 with 4096 of 512).
  const int64_t max_grid = nblocks * 32 <= kAmaxCachedBytes ? kQuantMaxGrid / 4 : kQuantMaxGrid;
  const int64_t want = (nblocks + kQuantThreads - 1) / kQuantThreads;
  const int64_t passes = (want + max_grid - 1) / max_grid;
  const int grid = (int)((want + passes - 1) / passes);
  quant_kernel<<<grid, kQuantThreads, 0, stream>>>(xv, nblocks, partial, npartial, gsa_override, cv, scales,
                                                   gsa_out);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream) {
  const int64_t nwords = (int64_t)(bytes / 4);
  if (nwords == 0) return hipSuccess;
  const int64_t want = (nwords + 255) / 256;
  fill_zero_kernel<<<(int)(want < 1024 ? want : 1024), 256, 0, stream>>>(static_cast<uint32_t*>(p), nwords);
  return hipGetLastError();
}

}  // namespace nvr
