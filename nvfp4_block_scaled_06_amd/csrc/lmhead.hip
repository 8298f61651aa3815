// lm_head-shaped NVFP4 GEMV with a greedy (top-1) epilogue (gfx950).
//
// logits[t, n] = gsa * gsw * sum_d (q_x S_x)[t, d] * (q_w S_w)[n, d] over a
// vocabulary-sized weight matrix (the NVFP4 lm_head of commit df05289d,
// dsv4/layers/grouped_linear.py, weights paragraph: the BF16 copy it replaces
// is 1.8 GB), then the largest logit of each token, an exact tie going to the
// lower row. With T <= 4 tokens this is a stream of the packed weights
// (E x D / 2 code bytes and E x D / 16 scale bytes), so the roofline is HBM
// bandwidth: the same GEMV design as the router's decode gate at a size where
// the bandwidth, not the launch and handoff latency, sets the time.
//
//  * Workgroup: 64 rows, four wavefronts of 16 rows, 2 rows in flight per
//    wavefront at all times (a rolling ring: a row's loads are issued as soon
//    as the row two before it is summed; two measured faster than one,
//    three or four: 89.9-92.6 against 94.9-96.7 us per call with four at
//    N = 129280, D = 7168); lane l takes the 32-element chunks l, l + 64,
//    ... of a row (16 code bytes and 2 scale bytes each, coalesced
//    1 KB per wavefront).
//    The weights are read once per call, with nontemporal loads (measured:
//    110 us against 115 us with cached loads at 129,280 x 7168; 8 rows in
//    flight or 8 rows per wavefront were no faster).
//  * x: the tokens' chunks are converted once per workgroup into LDS as
//    exact fp16 q S values, the weight chunks in registers; block products
//    are exact in fp32 and the per-lane sums and the wavefront sum run in a
//    fixed order (bit-reproducible).
//  * Epilogue: each workgroup's best (logit key, row) per token goes to the
//    workspace with a device-coherent store; the last workgroup to arrive
//    (arrival counter) takes the maximum over them.
#include "../../include/nvfp4_router.h"
#include "mma_tile.hpp"  // gate_common.hpp, raw buffer descriptors

namespace nvr {

constexpr int kLmWaves = 4;
constexpr int kLmThreads = 64 * kLmWaves;
constexpr int kLmRowsPerWave = 16;
constexpr int kLmRows = kLmWaves * kLmRowsPerWave;  // rows per workgroup
constexpr int kLmInFlight = 2;                       // rows per wavefront whose loads are in flight
constexpr int kLmMaxT = 4;
constexpr int kLmMaxD = 16384;

struct LmArgs {
  const uint8_t* xc;
  const uint8_t* xs;
  const float* gsa;
  const uint8_t* wc;
  const uint8_t* ws;
  const float* gsw;
  int T, D, N;
  int32_t* idx;
  float* logit;
  float* logits_out;
  uint64_t* cand;  // [T, nwg] per-workgroup best (key << 32 | ~row)
  uint32_t* counter;
  int nwg;
};

// Largest 64-bit value over the wavefront (every lane gets it).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o);
    const uint64_t u = ((uint64_t)hi << 32) | lo;
    v = u > v ? u : v;
  }
  return v;
}

// The fp32 value whose score_key is k (k > 0).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// CPL: 32-element chunks per lane, D / 32 / 64 rounded up.
template <int CPL>
__global__ __launch_bounds__(kLmThreads) void lmhead_argmax_kernel(LmArgs a) {
  extern __shared__ half8_t xl[];  // [T][D / 8]: x chunks as fp16 q S, 4 half8 per 32-element chunk
  __shared__ uint64_t wbest[kLmWaves][kLmMaxT];
  __shared__ uint32_t s_last;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int T = a.T, nch = a.D >> 5;
  const int64_t rowc = a.D / 2, rows = a.D / 16;
  const float gsa = load_early(a.gsa), gsw = load_early(a.gsw);

  // x into LDS: thread i converts chunk i of the flattened [T, D / 32] chunks.
  for (int i = threadIdx.x; i < T * nch; i += kLmThreads) {
    const int t = i / nch, c = i - t * nch;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(a.xc + (int64_t)t * rowc + 16 * c);
    const uint32_t sb = *reinterpret_cast<const uint16_t*>(a.xs + (int64_t)t * rows + 2 * c);
    const _Float16 s0 = e4m3_f16(sb & 0xFFu), s1 = e4m3_f16(sb >> 8);
    half8_t* d = xl + (int64_t)t * (nch * 4) + 4 * c;
    d[0] = fp4x8_to_f16(v[0], s0);
    d[1] = fp4x8_to_f16(v[1], s0);
    d[2] = fp4x8_to_f16(v[2], s1);
    d[3] = fp4x8_to_f16(v[3], s1);
  }
  __syncthreads();

  const double scale = (double)gsa * (double)gsw;
  uint64_t best[kLmMaxT];
#pragma unroll
  for (int t = 0; t < kLmMaxT; ++t) best[t] = 0ull;
  const int row_base = blockIdx.x * kLmRows + wave * kLmRowsPerWave;
  // Raw buffer loads: rows past N read zeros, and chunks
  // past D get an offset past the range (zeros, no branch), so the loads are
  // unconditional and complete in issue order. A ring of kLmInFlight rows:
  // row u + kLmInFlight is loaded into row u's registers as soon as row u is
  // summed, so that many rows stay in flight throughout (summing row u waits
  // for its own loads only). Rows past N and chunks past D contribute
  // nothing (their x chunk index is clamped).
  // Descriptors over this workgroup's rows only (from its first row): 32-bit
  // ranges and offsets then hold for any N.
  const int64_t wg_row0 = (int64_t)blockIdx.x * kLmRows;
  const int64_t wg_rows = min((int64_t)kLmRows, (int64_t)a.N - wg_row0);
  const __amdgpu_buffer_rsrc_t wcr = make_rsrc(a.wc + wg_row0 * rowc, wg_rows * rowc);
  const __amdgpu_buffer_rsrc_t wsr = make_rsrc(a.ws + wg_row0 * rows, wg_rows * rows);
  uint32_t oc[CPL], os[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    oc[i] = c < nch ? (uint32_t)(16 * c) : kMmaOob;
    os[i] = c < nch ? (uint32_t)(2 * c) : kMmaOob;
  }
  u32x4_t wv[kLmInFlight][CPL];
  uint32_t wsv[kLmInFlight][CPL];
  auto load_row = [&](int slot, int u) {
    const int lr = wave * kLmRowsPerWave + u;  // row within the workgroup
    const uint32_t rc = (uint32_t)lr * (uint32_t)rowc, rs = (uint32_t)lr * (uint32_t)rows;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      wv[slot][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wcr, oc[i] + rc, 0, kNtAux));
      wsv[slot][i] = __builtin_amdgcn_raw_buffer_load_b16(wsr, os[i] + rs, 0, kNtAux);
    }
  };
#pragma unroll
  for (int u = 0; u < kLmInFlight; ++u) load_row(u, u);
#pragma unroll
  for (int u = 0; u < kLmRowsPerWave; ++u) {
    const int slot = u % kLmInFlight, row = row_base + u;
    float acc[kLmMaxT];
#pragma unroll
    for (int t = 0; t < kLmMaxT; ++t) acc[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = min(lane + 64 * i, nch - 1);
      const _Float16 s0 = e4m3_f16(wsv[slot][i] & 0xFFu), s1 = e4m3_f16(wsv[slot][i] >> 8);
      const half8_t w0 = fp4x8_to_f16(wv[slot][i][0], s0), w1 = fp4x8_to_f16(wv[slot][i][1], s0);
      const half8_t w2 = fp4x8_to_f16(wv[slot][i][2], s1), w3 = fp4x8_to_f16(wv[slot][i][3], s1);
#pragma unroll
      for (int t = 0; t < kLmMaxT; ++t) {
        if (t < T) {
          const half8_t* xp = xl + (int64_t)t * (nch * 4) + 4 * c;
          // One block (two halves) at a time: exact block sums, then fp32 accumulation.
          acc[t] += dot8(xp[1], w1, dot8(xp[0], w0, 0.0f));
          acc[t] += dot8(xp[3], w3, dot8(xp[2], w2, 0.0f));
        }
      }
    }
    if (u + kLmInFlight < kLmRowsPerWave) load_row(slot, u + kLmInFlight);
#pragma unroll
    for (int t = 0; t < kLmMaxT; ++t) {
      if (t < T) {
        const float L = (float)((double)wave_sum(acc[t]) * scale);
        if (row < a.N) {
          const uint64_t key = ((uint64_t)score_key(L) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)row);
          best[t] = key > best[t] ? key : best[t];
          if (a.logits_out && lane == 0) a.logits_out[(int64_t)t * a.N + row] = L;
        }
      }
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < kLmMaxT; ++t) wbest[wave][t] = best[t];
  }
  __syncthreads();
  if ((int)threadIdx.x < T) {
    const int t = threadIdx.x;
    uint64_t b = wbest[0][t];
#pragma unroll
    for (int w = 1; w < kLmWaves; ++w) b = wbest[w][t] > b ? wbest[w][t] : b;
    __hip_atomic_store(a.cand + (int64_t)t * a.nwg + blockIdx.x, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!arrive_last(a.counter, a.nwg, &s_last)) return;

  // Last workgroup: the maximum over every workgroup's best, per token.
  for (int t = 0; t < T; ++t) {
    uint64_t b = 0ull;
    for (int i = threadIdx.x; i < a.nwg; i += kLmThreads) {
      const uint64_t v = __hip_atomic_load(a.cand + (int64_t)t * a.nwg + i, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
      b = v > b ? v : b;
    }
    b = wave_max_u64(b);
    __syncthreads();  // wbest is reused
    if (lane == 0) wbest[wave][0] = b;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint64_t m = wbest[0][0];
#pragma unroll
      for (int w = 1; w < kLmWaves; ++w) m = wbest[w][0] > m ? wbest[w][0] : m;
      a.idx[t] = (int32_t)(0xFFFFFFFFu - (uint32_t)m);
      a.logit[t] = key_value((uint32_t)(m >> 32));
    }
  }
  release_counter(a.counter);
}

static int lm_nwg(int64_t N) { return (int)((N + kLmRows - 1) / kLmRows); }

size_t lmhead_scratch_bytes(int64_t T, int64_t N) { return (size_t)T * (size_t)lm_nwg(N) * sizeof(uint64_t); }

template <int CPL>
static hipError_t launch_lm(const LmArgs& a, hipStream_t stream) {
  const size_t lds = (size_t)a.T * (size_t)a.D * sizeof(_Float16);
  lmhead_argmax_kernel<CPL><<<a.nwg, kLmThreads, lds, stream>>>(a);
  return hipGetLastError();
}

}  // namespace nvr

namespace {

bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool lm_shape_ok(int64_t T, int64_t D, int64_t N) {
  // T * D <= 32768 keeps the tokens' fp16 copy within 64 KB of LDS.
  return T >= 0 && T <= nvr::kLmMaxT && D >= 32 && D <= nvr::kLmMaxD && D % 32 == 0 && T * D <= 32768 && N >= 1 &&
         N <= (int64_t(1) << 30);
}

}  // namespace

extern "C" size_t lmhead_workspace_bytes(int64_t T, int64_t D, int64_t N) {
  if (!lm_shape_ok(T, D, N)) return 0;
  return nvr::kScratchOffset + nvr::lmhead_scratch_bytes(T, N);
}

extern "C" int lmhead_argmax(const uint8_t* x_codes, const uint8_t* x_scales, const float* gsa,
                             const uint8_t* w_codes, const uint8_t* w_scales, const float* gsw, int64_t T, int64_t D,
                             int64_t N, int32_t* out_idx, float* out_logit, float* logits_out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!lm_shape_ok(T, D, N)) return ROUTER_EINVAL;
  if (T == 0) return ROUTER_OK;
  if (!x_codes || !x_scales || !gsa || !w_codes || !w_scales || !gsw || !out_idx || !out_logit || !workspace)
    return ROUTER_EINVAL;
  if (!aligned_to(x_codes, 16) || !aligned_to(w_codes, 16) || !aligned_to(x_scales, 2) || !aligned_to(w_scales, 2) ||
      !aligned_to(workspace, 256) || !aligned_to(out_idx, 4) || !aligned_to(out_logit, 4) ||
      (logits_out && !aligned_to(logits_out, 4)))
    return ROUTER_EINVAL;
  if (workspace_bytes < lmhead_workspace_bytes(T, D, N)) return ROUTER_EINVAL;
  char* base = static_cast<char*>(workspace);
  nvr::LmArgs a{x_codes, x_scales, gsa, w_codes, w_scales, gsw, (int)T, (int)D, (int)N, out_idx, out_logit,
                logits_out, reinterpret_cast<uint64_t*>(base + nvr::kScratchOffset),
                reinterpret_cast<uint32_t*>(base), nvr::lm_nwg(N)};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int cpl = (int)((D / 32 + 63) / 64);
  hipError_t e;
  if (cpl <= 1) e = nvr::launch_lm<1>(a, s);
  else if (cpl <= 2) e = nvr::launch_lm<2>(a, s);
  else if (cpl <= 4) e = nvr::launch_lm<4>(a, s);
  else e = nvr::launch_lm<8>(a, s);
  return e == hipSuccess ? ROUTER_OK : ROUTER_EHIP;
}
