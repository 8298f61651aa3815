// Block-scaled NVFP4 gate projection with the routing epilogue fused after it
// (gfx950).
//
// logits[t, e] = gsa * gsw * sum_d (q_x S_x)[t, d] * (q_w S_w)[e, d]: the gate
// GEMM on NVFP4 operands (commit 04cf8ca8, dsv4/layers/router.py, NVFP4 gate
// paragraph), followed by the six-step epilogue (commit e0f60b9f,
// dsv4/kernels/router/__init__.py) while the logits are still on chip or in
// L2, so they never make an HBM round trip unless logits_out asks for them.
//
// Three kernels, by token count T:
//  * gemv (T <= 4, decode): one workgroup per 4 experts, K split over its
//    threads (one 16-element block each), dot products of exact fp16 code
//    values on the VALU, a fixed-order workgroup sum; the last workgroup to
//    arrive (device arrival counter) routes every token. A variant also
//    quantizes x itself (router_forward: one launch per router call).
//  * tile (T <= 256): 16x16 output tiles on 16x16x32 f16 MFMAs, the four
//    waves of a workgroup splitting K and summing through LDS; the last
//    workgroup of each 16-row tile routes it.
//  * fused (larger T): one workgroup per 32 tokens and all experts on
//    32x32x16 f16 MFMAs; the accumulators go through LDS straight into the
//    epilogue.
//
// MFMA operands: every 16-element block becomes fp16 values q * S, exact (at
// most 6 significant bits in [2^-10, 2688]), so products are exact and only
// the fp32 accumulation rounds. The scaled FP4 MFMA of gfx950 takes
// power-of-two scales per 32 elements and cannot carry an E4M3 scale per 16.
//
// MFMA lane layout: each lane supplies 8 consecutive K values of one A row
// and of one B column, from one of 2 (32x32x16) or 4 (16x16x32) K groups. A
// lane here loads 32 consecutive elements (16 code bytes, 2 scale bytes) of
// its row and feeds them to four successive MFMAs, 8 at a time: a
// permutation of K that A and B share, so every product meets its partner.
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

__device__ __forceinline__ void release_counter(uint32_t* counter) {
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// gemv: decode-size T.
// ---------------------------------------------------------------------------
struct GemvArgs {
  const u32x4_t* x;           // bf16 x [T, D] (quantizing variant only)
  const float* gsa_override;  // quantizing variant only; NULL = runtime gsa
  uint8_t* xc;                // x codes [T, D/2]: written by workgroup 0 (quantizing) or read
  uint8_t* xs;                // x scales [T, D/16]: likewise
  float* gsa;                 // [1]: written by workgroup 0 (quantizing) or read
  const uint8_t* wc;
  const uint8_t* ws;
  const float* gsw;
  const float* bias;
  float routed_scale;
  int T, D, E, k;
  int32_t* idx;
  float* w;
  float* logits_out;
  float* lbuf;  // [T, E] workspace
  uint32_t* counter;
};

constexpr int kGemvMaxT = 4;
constexpr int kGemvMaxThreads = 512;
constexpr int kGemvExperts = 4;  // experts per workgroup: E/4 arrivals on the counter

template <int TMAX, int BPT, int JMAX, bool QUANT>
__global__ __launch_bounds__(kGemvMaxThreads) void gate_gemv_kernel(GemvArgs a) {
  constexpr int EPW = kGemvExperts;
  __shared__ float red[kGemvMaxThreads / 64][EPW][TMAX];
  __shared__ uint32_t ured[kGemvMaxThreads / 64];
  __shared__ float lg[TMAX * 512];
  __shared__ uint32_t s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int e0 = blockIdx.x * EPW;
  const int nb = a.D >> 4;
  const int T = a.T;

  // Gate-weight blocks of this workgroup's experts (8 code bytes + 1 scale
  // byte each), issued first so their latency overlaps the activation work.
  uint32_t wq[EPW][BPT][2], wsb[EPW][BPT];
#pragma unroll
  for (int p = 0; p < EPW; ++p)
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const int j = tid + b * blockDim.x, e = e0 + p;
      wq[p][b][0] = wq[p][b][1] = 0u;
      wsb[p][b] = 0u;
      if (j < nb && e < a.E) {
        const uint2 v = *reinterpret_cast<const uint2*>(a.wc + (int64_t)e * (a.D / 2) + 8 * j);
        wq[p][b][0] = v.x;
        wq[p][b][1] = v.y;
        wsb[p][b] = a.ws[(int64_t)e * nb + j];
      }
    }

  uint32_t xq[TMAX][BPT][2], xsb[TMAX][BPT];
  float gsa;
  if constexpr (QUANT) {
    // Every workgroup reads all of x (T*D*2 bytes, from L2 after the first)
    // and derives the same gsa; each thread quantizes the blocks it owns.
    uint32_t raw[TMAX][BPT][8];
    uint32_t m = 0;
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
#pragma unroll
      for (int b = 0; b < BPT; ++b) {
        const int j = tid + b * blockDim.x;
#pragma unroll
        for (int i = 0; i < 8; ++i) raw[t][b][i] = 0u;
        if (t < T && j < nb) {
          const u32x4_t v0 = a.x[2 * ((int64_t)t * nb + j)];
          const u32x4_t v1 = a.x[2 * ((int64_t)t * nb + j) + 1];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            raw[t][b][i] = v0[i];
            raw[t][b][4 + i] = v1[i];
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) m = max(m, bf16_pair_absmax(raw[t][b][i]));
        }
      }
    if (a.gsa_override) {
      gsa = *a.gsa_override;
    } else {
      m = wave_max_u32(m);
      if (lane == 0) ured[wave] = m;
      __syncthreads();
      uint32_t mm = 0;
      for (int i = 0; i < nwaves; ++i) mm = max(mm, ured[i]);
      gsa = __uint_as_float(mm << 16) / kGsaDivisor;
    }
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
#pragma unroll
      for (int b = 0; b < BPT; ++b) {
        const int j = tid + b * blockDim.x;
        uint32_t s = 0u;
        xq[t][b][0] = xq[t][b][1] = 0u;
        if (t < T) quant_block16(raw[t][b], gsa, xq[t][b][0], xq[t][b][1], s);
        xsb[t][b] = s;
        if (blockIdx.x == 0 && t < T && j < nb) {
          *reinterpret_cast<uint2*>(a.xc + ((int64_t)t * nb + j) * 8) = make_uint2(xq[t][b][0], xq[t][b][1]);
          a.xs[(int64_t)t * nb + j] = (uint8_t)s;
        }
      }
    if (blockIdx.x == 0 && tid == 0) *a.gsa = gsa;
  } else {
    gsa = *a.gsa;
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
#pragma unroll
      for (int b = 0; b < BPT; ++b) {
        const int j = tid + b * blockDim.x;
        xq[t][b][0] = xq[t][b][1] = 0u;
        xsb[t][b] = 0u;
        if (t < T && j < nb) {
          const uint2 v = *reinterpret_cast<const uint2*>(a.xc + ((int64_t)t * nb + j) * 8);
          xq[t][b][0] = v.x;
          xq[t][b][1] = v.y;
          xsb[t][b] = a.xs[(int64_t)t * nb + j];
        }
      }
  }

  // Per-block dot products of exact code values, scaled by S_x * S_w (exact).
  float acc[EPW][TMAX];
#pragma unroll
  for (int p = 0; p < EPW; ++p)
#pragma unroll
    for (int t = 0; t < TMAX; ++t) acc[p][t] = 0.0f;
#pragma unroll
  for (int b = 0; b < BPT; ++b) {
    const int j = tid + b * blockDim.x;
    if (j < nb) {
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        if (t < T) {
          const half8_t x0 = fp4x8_q(xq[t][b][0]), x1 = fp4x8_q(xq[t][b][1]);
          const float sx = e4m3_value(xsb[t][b]);
#pragma unroll
          for (int p = 0; p < EPW; ++p) {
            float d = dot8(x0, fp4x8_q(wq[p][b][0]), 0.0f);
            d = dot8(x1, fp4x8_q(wq[p][b][1]), d);
            acc[p][t] = fmaf(d, sx * e4m3_value(wsb[p][b]), acc[p][t]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    if (t < T) {
#pragma unroll
      for (int p = 0; p < EPW; ++p) {
        const float v = wave_sum(acc[p][t]);
        if (lane == 0) red[wave][p][t] = v;
      }
    }
  }
  __syncthreads();
  const float scale = gsa * (*a.gsw);
  if (tid < EPW * TMAX) {
    const int p = tid % EPW, t = tid / EPW, e = e0 + p;
    if (t < T && e < a.E) {
      float s = 0.0f;
      for (int i = 0; i < nwaves; ++i) s += red[i][p][t];
      const float L = s * scale;
      store_coherent(a.lbuf + (int64_t)t * a.E + e, L);
      if (a.logits_out) a.logits_out[(int64_t)t * a.E + e] = L;
    }
  }

  if (!arrive_last(a.counter, gridDim.x, &s_last)) return;
  for (int i = tid; i < T * a.E; i += blockDim.x) lg[i] = load_coherent(a.lbuf + i);
  __syncthreads();
  if (wave < T) wave_route_row<JMAX>(lg + wave * a.E, a.bias, a.E, a.k, a.routed_scale, a.idx + wave * a.k,
                                     a.w + wave * a.k);
  release_counter(a.counter);
}

// ---------------------------------------------------------------------------
// tile: T up to a few hundred.
// ---------------------------------------------------------------------------
struct TileArgs {
  const uint8_t* xc;
  const uint8_t* xs;
  const float* gsa;
  const uint8_t* wc;
  const uint8_t* ws;
  const float* gsw;
  const float* bias;
  float routed_scale;
  int T, D, E, k;
  int32_t* idx;
  float* w;
  float* logits_out;
  float* lbuf;  // [T, E] workspace
  uint32_t* counters;
  int nsteps;  // 128-element K steps
};

template <int JMAX>
__global__ __launch_bounds__(256) void gate_tile_kernel(TileArgs a) {
  __shared__ float part[4][16][17];
  __shared__ uint32_t s_last;
  extern __shared__ float lg[];  // [16][E]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int col0 = blockIdx.x * 16, row0 = blockIdx.y * 16;
  const int arow = row0 + n, e = col0 + n;
  const bool a_ok = arow < a.T, b_ok = e < a.E;
  const int s0 = a.nsteps * wave / 4, s1 = a.nsteps * (wave + 1) / 4;

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  Chunk32 an = {}, bn = {};
  if (s0 < s1) {
    const int64_t k0 = (int64_t)s0 * 128 + 32 * g;
    an = load_chunk(a.xc, a.xs, arow, a.D, k0, a_ok && k0 < a.D);
    bn = load_chunk(a.wc, a.ws, e, a.D, k0, b_ok && k0 < a.D);
  }
  for (int s = s0; s < s1; ++s) {
    const Chunk32 ac = an, bc = bn;
    if (s + 1 < s1) {
      const int64_t k0 = (int64_t)(s + 1) * 128 + 32 * g;
      an = load_chunk(a.xc, a.xs, arow, a.D, k0, a_ok && k0 < a.D);
      bn = load_chunk(a.wc, a.ws, e, a.D, k0, b_ok && k0 < a.D);
    }
    const _Float16 sa0 = e4m3_f16(ac.s & 0xFFu), sa1 = e4m3_f16(ac.s >> 8);
    const _Float16 sb0 = e4m3_f16(bc.s & 0xFFu), sb1 = e4m3_f16(bc.s >> 8);
    acc = mfma16(fp4x8_to_f16(ac.c[0], sa0), fp4x8_to_f16(bc.c[0], sb0), acc);
    acc = mfma16(fp4x8_to_f16(ac.c[1], sa0), fp4x8_to_f16(bc.c[1], sb0), acc);
    acc = mfma16(fp4x8_to_f16(ac.c[2], sa1), fp4x8_to_f16(bc.c[2], sb1), acc);
    acc = mfma16(fp4x8_to_f16(ac.c[3], sa1), fp4x8_to_f16(bc.c[3], sb1), acc);
  }
  // 16x16 accumulator layout: lane holds rows 4g..4g+3 of column n.
#pragma unroll
  for (int v = 0; v < 4; ++v) part[wave][4 * g + v][n] = acc[v];
  __syncthreads();
  if (wave == 0) {
    const float scale = (*a.gsa) * (*a.gsw);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g + v, r = row0 + m;
      const float L = ((part[0][m][n] + part[1][m][n]) + (part[2][m][n] + part[3][m][n])) * scale;
      if (r < a.T && b_ok) {
        store_coherent(a.lbuf + (int64_t)r * a.E + e, L);
        if (a.logits_out) a.logits_out[(int64_t)r * a.E + e] = L;
      }
    }
  }
  if (!arrive_last(&a.counters[blockIdx.y], gridDim.x, &s_last)) return;
  const int nrows = min(16, a.T - row0);
  for (int i = threadIdx.x; i < nrows * a.E; i += 256) lg[i] = load_coherent(a.lbuf + (int64_t)row0 * a.E + i);
  __syncthreads();
  for (int m = wave; m < nrows; m += 4) {
    const int64_t t = row0 + m;
    wave_route_row<JMAX>(lg + m * a.E, a.bias, a.E, a.k, a.routed_scale, a.idx + t * a.k, a.w + t * a.k);
  }
  release_counter(&a.counters[blockIdx.y]);
}

// ---------------------------------------------------------------------------
// fused: prefill-size T. One workgroup per 32 tokens and all E experts. Wave
// w owns expert tiles w, w+4, ... (32 experts each).
// ---------------------------------------------------------------------------
template <int NT, int JMAX>
__global__ __launch_bounds__(256) void gate_fused_kernel(TileArgs a) {
  extern __shared__ float lds[];  // [32][E]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int row0 = blockIdx.x * 32;
  const int arow = row0 + r;
  const bool a_ok = arow < a.T;
  const int D = a.D, E = a.E;

  f32x16_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0.0f;

  for (int64_t kb = 0; kb < D; kb += 64) {
    const int64_t k0 = kb + 32 * h;
    const bool k_ok = k0 < D;
    const Chunk32 ca = load_chunk(a.xc, a.xs, arow, D, k0, a_ok && k_ok);
    const _Float16 sa0 = e4m3_f16(ca.s & 0xFFu), sa1 = e4m3_f16(ca.s >> 8);
    const half8_t A0 = fp4x8_to_f16(ca.c[0], sa0), A1 = fp4x8_to_f16(ca.c[1], sa0);
    const half8_t A2 = fp4x8_to_f16(ca.c[2], sa1), A3 = fp4x8_to_f16(ca.c[3], sa1);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int e = (wave + 4 * t) * 32 + r;
      const Chunk32 cb = load_chunk(a.wc, a.ws, e, D, k0, k_ok && e < E);
      const _Float16 sb0 = e4m3_f16(cb.s & 0xFFu), sb1 = e4m3_f16(cb.s >> 8);
      acc[t] = mfma32(A0, fp4x8_to_f16(cb.c[0], sb0), acc[t]);
      acc[t] = mfma32(A1, fp4x8_to_f16(cb.c[1], sb0), acc[t]);
      acc[t] = mfma32(A2, fp4x8_to_f16(cb.c[2], sb1), acc[t]);
      acc[t] = mfma32(A3, fp4x8_to_f16(cb.c[3], sb1), acc[t]);
    }
  }

  // 32x32 accumulator layout: value v of lane (r, h) is row 8(v/4) + 4h + v%4, column r.
  const float scale = (*a.gsa) * (*a.gsw);
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
  const int nrows = min(32, a.T - row0);
  for (int m = wave; m < nrows; m += 4) {
    const int64_t t = row0 + m;
    wave_route_row<JMAX>(lds + m * E, a.bias, E, a.k, a.routed_scale, a.idx + t * a.k, a.w + t * a.k);
  }
  if (a.logits_out) {
    for (int i = threadIdx.x; i < nrows * E; i += 256) a.logits_out[(int64_t)row0 * E + i] = lds[i];
  }
}

// ---------------------------------------------------------------------------
// Host side: planning and launch.
// ---------------------------------------------------------------------------
static GateTuning read_tuning() {
  GateTuning t;
  if (const char* v = getenv("NVR_SPLIT_MAX_T")) t.split_max_t = atoi(v);
  if (t.split_max_t < 0) t.split_max_t = 0;
  if (t.split_max_t > 16 * kMaxCounters) t.split_max_t = 16 * kMaxCounters;
  return t;
}

const GateTuning& gate_tuning() {
  static const GateTuning t = read_tuning();
  return t;
}

// Blocks per thread of the gemv kernel (0 if D is too large for it).
static int gemv_bpt(int64_t D) {
  const int64_t nb = D / 16;
  for (int bpt : {1, 2, 4})
    if ((nb + bpt - 1) / bpt <= kGemvMaxThreads) return bpt;
  return 0;
}

GateKind gate_kind(int64_t T, int64_t D) {
  if (T <= kGemvMaxT && gemv_bpt(D) > 0) return GateKind::kGemv;
  if (T <= gate_tuning().split_max_t) return GateKind::kTile;
  return GateKind::kFused;
}

size_t gate_scratch_bytes(int64_t T, int64_t D, int64_t E) {
  return gate_kind(T, D) == GateKind::kFused ? 0 : (size_t)T * (size_t)E * sizeof(float);
}

template <int TMAX, int BPT, bool QUANT>
static hipError_t launch_gemv_b(const GemvArgs& a, int threads, hipStream_t stream) {
  const int j = (a.E + 63) / 64;
  const int grid = (a.E + kGemvExperts - 1) / kGemvExperts;
  if (j <= 1) gate_gemv_kernel<TMAX, BPT, 1, QUANT><<<grid, threads, 0, stream>>>(a);
  else if (j <= 2) gate_gemv_kernel<TMAX, BPT, 2, QUANT><<<grid, threads, 0, stream>>>(a);
  else if (j <= 4) gate_gemv_kernel<TMAX, BPT, 4, QUANT><<<grid, threads, 0, stream>>>(a);
  else if (j <= 6) gate_gemv_kernel<TMAX, BPT, 6, QUANT><<<grid, threads, 0, stream>>>(a);
  else gate_gemv_kernel<TMAX, BPT, 8, QUANT><<<grid, threads, 0, stream>>>(a);
  return hipGetLastError();
}

template <bool QUANT>
static hipError_t launch_gemv(const GemvArgs& a, hipStream_t stream) {
  const int bpt = gemv_bpt(a.D);
  const int nb = a.D / 16;
  int threads = ((nb + bpt - 1) / bpt + 63) / 64 * 64;
  if (threads < 64 * kGemvMaxT) threads = 64 * kGemvMaxT;
  if constexpr (QUANT) {
    if (bpt == 1) return launch_gemv_b<kGemvMaxT, 1, true>(a, threads, stream);
    return launch_gemv_b<kGemvMaxT, 2, true>(a, threads, stream);
  }
  switch (bpt) {
    case 1: return launch_gemv_b<kGemvMaxT, 1, QUANT>(a, threads, stream);
    case 2: return launch_gemv_b<kGemvMaxT, 2, QUANT>(a, threads, stream);
    default: return launch_gemv_b<kGemvMaxT, 4, QUANT>(a, threads, stream);
  }
}

static hipError_t launch_tile(const TileArgs& a, hipStream_t stream) {
  const dim3 grid((a.E + 15) / 16, (a.T + 15) / 16);
  const size_t lds = (size_t)16 * a.E * sizeof(float);
  const int j = (a.E + 63) / 64;
  if (j <= 1) gate_tile_kernel<1><<<grid, 256, lds, stream>>>(a);
  else if (j <= 2) gate_tile_kernel<2><<<grid, 256, lds, stream>>>(a);
  else if (j <= 4) gate_tile_kernel<4><<<grid, 256, lds, stream>>>(a);
  else if (j <= 6) gate_tile_kernel<6><<<grid, 256, lds, stream>>>(a);
  else gate_tile_kernel<8><<<grid, 256, lds, stream>>>(a);
  return hipGetLastError();
}

static hipError_t launch_fused(const TileArgs& a, hipStream_t stream) {
  const int grid = (a.T + 31) / 32;
  const size_t lds = (size_t)32 * a.E * sizeof(float);
  const int nt = (a.E + 127) / 128;
  if (nt <= 1) gate_fused_kernel<1, 2><<<grid, 256, lds, stream>>>(a);
  else if (nt <= 2) gate_fused_kernel<2, 4><<<grid, 256, lds, stream>>>(a);
  else if (nt <= 3) gate_fused_kernel<3, 6><<<grid, 256, lds, stream>>>(a);
  else gate_fused_kernel<4, 8><<<grid, 256, lds, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_gate(const uint8_t* xc, const uint8_t* xs, const float* gsa, const uint8_t* wc, const uint8_t* ws,
                       const float* gsw, const float* bias, float rs, int64_t T, int64_t D, int64_t E, int64_t k,
                       int32_t* idx, float* w, float* lo, uint32_t* counters, void* scratch, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const GateKind kind = gate_kind(T, D);
  float* lbuf = static_cast<float*>(scratch);
  if (kind == GateKind::kGemv) {
    GemvArgs a{nullptr, nullptr, const_cast<uint8_t*>(xc), const_cast<uint8_t*>(xs), const_cast<float*>(gsa),
               wc, ws, gsw, bias, rs, (int)T, (int)D, (int)E, (int)k, idx, w, lo, lbuf, counters};
    return launch_gemv<false>(a, stream);
  }
  TileArgs a{xc, xs, gsa, wc, ws, gsw, bias, rs, (int)T, (int)D, (int)E, (int)k, idx, w, lo, lbuf, counters,
             (int)((D + 127) / 128)};
  return kind == GateKind::kTile ? launch_tile(a, stream) : launch_fused(a, stream);
}

// The quantizing gemv keeps every raw x block of a thread in registers: at
// most two blocks per thread.
bool forward_single_launch(int64_t T, int64_t D) {
  const int bpt = gemv_bpt(D);
  return gate_kind(T, D) == GateKind::kGemv && bpt > 0 && bpt <= 2;
}

hipError_t launch_forward_fused(const void* x, const float* gsa_override, uint8_t* xc, uint8_t* xs, float* gsa_out,
                                const uint8_t* wc, const uint8_t* ws, const float* gsw, const float* bias, float rs,
                                int64_t T, int64_t D, int64_t E, int64_t k, int32_t* idx, float* w, float* lo,
                                uint32_t* counters, void* scratch, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  GemvArgs a{static_cast<const u32x4_t*>(x), gsa_override, xc, xs, gsa_out, wc, ws, gsw, bias, rs, (int)T, (int)D,
             (int)E, (int)k, idx, w, lo, static_cast<float*>(scratch), counters};
  return launch_gemv<true>(a, stream);
}

}  // namespace nvr
