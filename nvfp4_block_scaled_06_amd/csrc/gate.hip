// Block-scaled NVFP4 gate projection with the routing epilogue fused after it
// (gfx950).
//
// logits[t, e] = gsa * gsw * sum_d (q_x S_x)[t, d] * (q_w S_w)[e, d]: the gate
// GEMM on NVFP4 operands (commit 04cf8ca8, dsv4/layers/router.py, NVFP4 gate
// paragraph), followed by the six-step epilogue (commit e0f60b9f,
// dsv4/kernels/router/__init__.py) on the logits while they are still on
// chip, so they never make an HBM round trip unless logits_out asks for them.
//
// Operands: every 16-element block becomes fp16 values q * S, exact (at most
// 6 significant bits in [2^-10, 2688]), so the fp16 MFMA forms exact
// products and accumulates them in fp32. The scaled FP4 MFMA of gfx950 takes
// power-of-two scales per 32 elements and cannot carry an E4M3 scale per 16.
//
// Lane layout: in an MFMA each lane supplies 8 consecutive K values of one
// A row and of one B column, from one of 2 (32x32x16) or 4 (16x16x32) K
// groups. Each lane here loads 32 consecutive elements (16 code bytes, 2
// scale bytes) of its row and feeds them to four successive MFMAs, 8 at a
// time. Which real K index sits in which MFMA slot is a permutation of K
// that A and B share, so every product still meets its partner.
#include "nvfp4_device.hpp"
#include "router_internal.hpp"

#include <stdlib.h>

namespace nvr {

__device__ __forceinline__ f32x4_t mfma16(half8_t a, half8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32(half8_t a, half8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
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

// ---------------------------------------------------------------------------
// Split gate (small T): grid (expert groups of 64, K ranges, 16-row tiles).
// Each wave owns 16 experts x 16 rows over a K range and writes fp32 partial
// sums to the workspace; the last workgroup to arrive for a row tile (device
// arrival counter) adds the partials in a fixed order and runs the epilogue.
// ---------------------------------------------------------------------------
template <int JMAX>
__global__ __launch_bounds__(256) void gate_split_kernel(
    const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs, const float* __restrict__ gsa_p,
    const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws, const float* __restrict__ gsw_p,
    const float* __restrict__ bias, float routed_scale, int T, int D, int E, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ logits_out, float* __restrict__ part,
    uint32_t* __restrict__ counters, int ksplit, int nsteps) {
  extern __shared__ float lds[];  // [16][E] logits of this row tile
  __shared__ uint32_t s_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int e = (blockIdx.x * 4 + wave) * 16 + n;  // B column (expert) of this lane
  const int row0 = blockIdx.z * 16;
  const int arow = row0 + n;  // A row (token) of this lane
  const int ks = blockIdx.y;
  const int s0 = (int)((int64_t)nsteps * ks / ksplit);
  const int s1 = (int)((int64_t)nsteps * (ks + 1) / ksplit);
  const bool a_ok = arow < T, b_ok = e < E;

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = s0; s < s1; ++s) {
    const int64_t k0 = (int64_t)s * 128 + 32 * g;
    const bool k_ok = k0 < D;
    const Chunk32 a = load_chunk(xc, xs, arow, D, k0, a_ok && k_ok);
    const Chunk32 b = load_chunk(wc, ws, e, D, k0, b_ok && k_ok);
    const _Float16 sa0 = e4m3_f16(a.s & 0xFFu), sa1 = e4m3_f16(a.s >> 8);
    const _Float16 sb0 = e4m3_f16(b.s & 0xFFu), sb1 = e4m3_f16(b.s >> 8);
    acc = mfma16(fp4x8_to_f16(a.c[0], sa0), fp4x8_to_f16(b.c[0], sb0), acc);
    acc = mfma16(fp4x8_to_f16(a.c[1], sa0), fp4x8_to_f16(b.c[1], sb0), acc);
    acc = mfma16(fp4x8_to_f16(a.c[2], sa1), fp4x8_to_f16(b.c[2], sb1), acc);
    acc = mfma16(fp4x8_to_f16(a.c[3], sa1), fp4x8_to_f16(b.c[3], sb1), acc);
  }

  // 16x16 accumulator layout: lane holds rows 4g..4g+3 of column n.
  float* pp = part + (int64_t)ks * T * E;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r = row0 + 4 * g + v;
    if (r < T && b_ok) pp[(int64_t)r * E + e] = acc[v];
  }
  __threadfence();  // release the partials before arriving
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t total = gridDim.x * gridDim.y;
    const uint32_t prev = atomicAdd(&counters[blockIdx.z], 1u);
    s_last = (prev == total - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();  // acquire every other workgroup's partials

  const float scale = (*gsa_p) * (*gsw_p);
  const int nrows = min(16, T - row0);
  for (int i = threadIdx.x; i < nrows * E; i += 256) {
    const int m = i / E, ee = i - m * E;
    const float* src = part + (int64_t)(row0 + m) * E + ee;
    float sum = 0.0f;
    for (int q = 0; q < ksplit; ++q) sum += src[(int64_t)q * T * E];
    const float L = sum * scale;
    lds[i] = L;
    if (logits_out) logits_out[(int64_t)row0 * E + i] = L;
  }
  __syncthreads();
  for (int m = wave; m < nrows; m += 4) {
    const int64_t t = row0 + m;
    wave_route_row<JMAX>(lds + m * E, bias, E, k, routed_scale, topk_idx + t * k, topk_w + t * k);
  }
  if (threadIdx.x == 0) __hip_atomic_store(&counters[blockIdx.z], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Fused gate (large T): one workgroup per 32 tokens and all E experts. Wave w
// owns expert tiles w, w+4, ... (32 experts each); 32x32x16 MFMAs; the
// accumulators are scaled into LDS and each wave routes 8 of the 32 rows.
// ---------------------------------------------------------------------------
template <int NT, int JMAX>
__global__ __launch_bounds__(256) void gate_fused_kernel(
    const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs, const float* __restrict__ gsa_p,
    const uint8_t* __restrict__ wc, const uint8_t* __restrict__ ws, const float* __restrict__ gsw_p,
    const float* __restrict__ bias, float routed_scale, int T, int D, int E, int k, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, float* __restrict__ logits_out) {
  extern __shared__ float lds[];  // [32][E]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int row0 = blockIdx.x * 32;
  const int arow = row0 + r;
  const bool a_ok = arow < T;

  f32x16_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0.0f;

  for (int64_t kb = 0; kb < D; kb += 64) {
    const int64_t k0 = kb + 32 * h;
    const bool k_ok = k0 < D;
    const Chunk32 a = load_chunk(xc, xs, arow, D, k0, a_ok && k_ok);
    const _Float16 sa0 = e4m3_f16(a.s & 0xFFu), sa1 = e4m3_f16(a.s >> 8);
    const half8_t A0 = fp4x8_to_f16(a.c[0], sa0), A1 = fp4x8_to_f16(a.c[1], sa0);
    const half8_t A2 = fp4x8_to_f16(a.c[2], sa1), A3 = fp4x8_to_f16(a.c[3], sa1);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int e = (wave + 4 * t) * 32 + r;
      const Chunk32 b = load_chunk(wc, ws, e, D, k0, k_ok && e < E);
      const _Float16 sb0 = e4m3_f16(b.s & 0xFFu), sb1 = e4m3_f16(b.s >> 8);
      acc[t] = mfma32(A0, fp4x8_to_f16(b.c[0], sb0), acc[t]);
      acc[t] = mfma32(A1, fp4x8_to_f16(b.c[1], sb0), acc[t]);
      acc[t] = mfma32(A2, fp4x8_to_f16(b.c[2], sb1), acc[t]);
      acc[t] = mfma32(A3, fp4x8_to_f16(b.c[3], sb1), acc[t]);
    }
  }

  // 32x32 accumulator layout: value v of lane (r, h) is row 8(v/4) + 4h + v%4, column r.
  const float scale = (*gsa_p) * (*gsw_p);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int e = (wave + 4 * t) * 32 + r;
    if (e < E) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = 8 * (v >> 2) + 4 * h + (v & 3);
        lds[m * E + e] = acc[t][v] * scale;
      }
    }
  }
  __syncthreads();
  const int nrows = min(32, T - row0);
  for (int m = wave; m < nrows; m += 4) {
    const int64_t t = row0 + m;
    wave_route_row<JMAX>(lds + m * E, bias, E, k, routed_scale, topk_idx + t * k, topk_w + t * k);
  }
  if (logits_out) {
    for (int i = threadIdx.x; i < nrows * E; i += 256) logits_out[(int64_t)row0 * E + i] = lds[i];
  }
}

// ---------------------------------------------------------------------------
// Host side: planning and launch.
// ---------------------------------------------------------------------------
static GateTuning read_tuning() {
  GateTuning t;
  if (const char* v = getenv("NVR_SPLIT_MAX_T")) t.split_max_t = atoi(v);
  if (const char* v = getenv("NVR_SPLIT_TARGET_WGS")) t.split_target_wgs = atoi(v);
  if (const char* v = getenv("NVR_SPLIT_MAX_KSPLIT")) t.split_max_ksplit = atoi(v);
  if (t.split_max_t < 0) t.split_max_t = 0;
  if (t.split_max_t > 16 * kMaxCounters) t.split_max_t = 16 * kMaxCounters;
  if (t.split_target_wgs < 1) t.split_target_wgs = 1;
  if (t.split_max_ksplit < 1) t.split_max_ksplit = 1;
  return t;
}

const GateTuning& gate_tuning() {
  static const GateTuning t = read_tuning();
  return t;
}

bool use_split_gate(int64_t T) { return T <= gate_tuning().split_max_t; }

SplitPlan plan_split(int64_t T, int64_t D, int64_t E) {
  const GateTuning& tu = gate_tuning();
  SplitPlan p;
  p.col_groups = (int)((E + 63) / 64);
  p.row_tiles = (int)((T + 15) / 16);
  p.nsteps = (int)((D + 127) / 128);
  int64_t ks = tu.split_target_wgs / ((int64_t)p.col_groups * (p.row_tiles > 0 ? p.row_tiles : 1));
  if (ks > p.nsteps) ks = p.nsteps;
  if (ks > tu.split_max_ksplit) ks = tu.split_max_ksplit;
  if (ks < 1) ks = 1;
  p.ksplit = (int)ks;
  return p;
}

size_t gate_scratch_bytes(int64_t T, int64_t D, int64_t E) {
  if (!use_split_gate(T)) return 0;
  const SplitPlan p = plan_split(T, D, E);
  return (size_t)p.ksplit * (size_t)T * (size_t)E * sizeof(float);
}

template <int JMAX>
static hipError_t launch_split_j(const SplitPlan& p, const uint8_t* xc, const uint8_t* xs, const float* gsa,
                                 const uint8_t* wc, const uint8_t* ws, const float* gsw, const float* bias,
                                 float rs, int T, int D, int E, int k, int32_t* idx, float* w, float* lo,
                                 float* part, uint32_t* counters, hipStream_t stream) {
  const dim3 grid(p.col_groups, p.ksplit, p.row_tiles);
  const size_t lds = (size_t)16 * E * sizeof(float);
  gate_split_kernel<JMAX><<<grid, 256, lds, stream>>>(xc, xs, gsa, wc, ws, gsw, bias, rs, T, D, E, k, idx, w, lo,
                                                      part, counters, p.ksplit, p.nsteps);
  return hipGetLastError();
}

template <int NT, int JMAX>
static hipError_t launch_fused_j(const uint8_t* xc, const uint8_t* xs, const float* gsa, const uint8_t* wc,
                                 const uint8_t* ws, const float* gsw, const float* bias, float rs, int T, int D,
                                 int E, int k, int32_t* idx, float* w, float* lo, hipStream_t stream) {
  const int grid = (T + 31) / 32;
  const size_t lds = (size_t)32 * E * sizeof(float);
  gate_fused_kernel<NT, JMAX><<<grid, 256, lds, stream>>>(xc, xs, gsa, wc, ws, gsw, bias, rs, T, D, E, k, idx, w,
                                                          lo);
  return hipGetLastError();
}

hipError_t launch_gate(const uint8_t* xc, const uint8_t* xs, const float* gsa, const uint8_t* wc, const uint8_t* ws,
                       const float* gsw, const float* bias, float rs, int64_t T64, int64_t D64, int64_t E64,
                       int64_t k64, int32_t* idx, float* w, float* lo, uint32_t* counters, void* scratch,
                       hipStream_t stream) {
  const int T = (int)T64, D = (int)D64, E = (int)E64, k = (int)k64;
  if (T == 0) return hipSuccess;
  const int jneed = (E + 63) / 64;
  if (use_split_gate(T64)) {
    const SplitPlan p = plan_split(T64, D64, E64);
    float* part = static_cast<float*>(scratch);
    if (jneed <= 1) return launch_split_j<1>(p, xc, xs, gsa, wc, ws, gsw, bias, rs, T, D, E, k, idx, w, lo, part, counters, stream);
    if (jneed <= 2) return launch_split_j<2>(p, xc, xs, gsa, wc, ws, gsw, bias, rs, T, D, E, k, idx, w, lo, part, counters, stream);
    if (jneed <= 4) return launch_split_j<4>(p, xc, xs, gsa, wc, ws, gsw, bias, rs, T, D, E, k, idx, w, lo, part, counters, stream);
    if (jneed <= 6) return launch_split_j<6>(p, xc, xs, gsa, wc, ws, gsw, bias, rs, T, D, E, k, idx, w, lo, part, counters, stream);
    return launch_split_j<8>(p, xc, xs, gsa, wc, ws, gsw, bias, rs, T, D, E, k, idx, w, lo, part, counters, stream);
  }
  const int nt = (E + 127) / 128;
  if (nt <= 1) return launch_fused_j<1, 2>(xc, xs, gsa, wc, ws, gsw, bias, rs, T, D, E, k, idx, w, lo, stream);
  if (nt <= 2) return launch_fused_j<2, 4>(xc, xs, gsa, wc, ws, gsw, bias, rs, T, D, E, k, idx, w, lo, stream);
  if (nt <= 3) return launch_fused_j<3, 6>(xc, xs, gsa, wc, ws, gsw, bias, rs, T, D, E, k, idx, w, lo, stream);
  return launch_fused_j<4, 8>(xc, xs, gsa, wc, ws, gsw, bias, rs, T, D, E, k, idx, w, lo, stream);
}

}  // namespace nvr
