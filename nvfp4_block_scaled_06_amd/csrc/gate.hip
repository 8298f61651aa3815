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
//  * decode (T <= 4): one workgroup per 128-element K slice; dot products of
//    exact fp16 code values on the VALU, slice partials through the
//    workspace, and the last workgroup to arrive (device arrival counter)
//    adds them and routes every token. A variant also quantizes x itself
//    (router_forward: one launch per router call).
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

// A uniform fp32 operand in device memory, read with a vector load where the
// call stands: the compiler would otherwise sink a scalar load of it to its
// first use and expose a whole memory round trip there.
__device__ __forceinline__ float load_early(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void release_counter(uint32_t* counter) {
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// decode: T <= 4 and D <= 16384. Workgroup (g, s) owns the 16 experts of
// group g and K slice s (64 blocks, one per lane); each of its 8 wavefronts
// owns 2 of the experts over the whole slice. Per expert row a workgroup
// reads 512 code bytes (four whole 128-byte lines) and 64 scale bytes, and
// the slices of one group run on one XCD, so no weight line is fetched into
// two L2s except at group boundaries. The quantizing variant reads all of x
// for the global max (every workgroup, from L2), then wavefront t quantizes
// token t's 64 slice blocks; group 0 stores the codes. Each wavefront sums
// its exact block products over the slice and stores one partial per
// (token, expert) with a device-coherent store; the last workgroup to arrive
// adds the slice partials in slice order and routes every token.
// ---------------------------------------------------------------------------
struct DecodeArgs {
  const u32x4_t* x;           // bf16 x [T, D] (quantizing variant only)
  const float* gsa_override;  // quantizing variant only; NULL = runtime gsa
  uint8_t* xc;                // x codes [T, D/2]: written by group 0 (quantizing) or read
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
  float* part;  // [nslices, T, E] slice partials (workspace scratch)
  uint32_t* counter;
  int nslices;  // K slices of 64 blocks
  int nwg;      // workgroups: expert groups * nslices
};

constexpr int kDecMaxT = 4;
constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecEpw = 2;                         // experts per wavefront
constexpr int kDecGroup = kDecWaves * kDecEpw;     // experts per workgroup
constexpr int kDecSlice = 64;                      // K blocks per slice
constexpr int kDecMaxSlices = 16;
constexpr int kDecAmaxChunks = 4;                  // 16-byte chunks of x per thread in the first max pass

template <int EP, bool QUANT>
__global__ __launch_bounds__(kDecThreads) void gate_decode_kernel(DecodeArgs a) {
  constexpr int TM = kDecMaxT;
  __shared__ uint32_t ured[kDecWaves];
  __shared__ uint32_t xq_lds[TM][kDecSlice][2];
  __shared__ uint32_t xs_lds[TM][kDecSlice];
  __shared__ WaveRouteScratch<EP> rsc[TM];
  __shared__ uint32_t s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, E = a.E, nb = a.D >> 4;
  // Workgroup ids go to the 8 XCDs in turn; number them so that consecutive
  // (group, slice) pairs land on one XCD: XCD x runs pairs [x q + min(x, r),
  // ...) of nwg = 8 q + r.
  const int nq = a.nwg >> 3, nr = a.nwg & 7, bx = blockIdx.x & 7;
  const int n = bx * nq + min(bx, nr) + (blockIdx.x >> 3);
  const int g = n / a.nslices, s = n - g * a.nslices;
  const int j = s * kDecSlice + lane;  // this lane's K block
  const bool jok = j < nb;
  const int64_t rowc = a.D / 2;

  // Every global load is issued before the first use (predicated by lane,
  // not by uniform branches).
  float bv[EP];  // bias of experts lane + 64 j, for the routing wavefronts
#pragma unroll
  for (int jj = 0; jj < EP; ++jj) bv[jj] = a.bias[min(lane + 64 * jj, E - 1)];
  const float gsw = load_early(a.gsw);
  uint32_t wq[kDecEpw][2], wsb[kDecEpw];
#pragma unroll
  for (int p = 0; p < kDecEpw; ++p) {
    const int e = g * kDecGroup + wave * kDecEpw + p;
    wq[p][0] = wq[p][1] = wsb[p] = 0u;
    if (e < E && jok) {
      const uint2 v = *reinterpret_cast<const uint2*>(a.wc + (int64_t)e * rowc + 8 * j);
      wq[p][0] = v.x;
      wq[p][1] = v.y;
      wsb[p] = a.ws[(int64_t)e * nb + j];
    }
  }

  float gsa;
  uint32_t xq[TM][2], xsb[TM];
  if constexpr (QUANT) {
    const float ov = a.gsa_override ? load_early(a.gsa_override) : 0.0f;
    // Wavefronts 2t and 2t + 1 quantize token t's 64 slice blocks, a lane
    // pair per block (8 elements each; the block max through one DPP
    // exchange). All lanes stride over x for the global max.
    const int qt = wave >> 1, qb = ((wave & 1) << 5) | (lane >> 1), qh = lane & 1;
    const bool quantizer = qt < T && s * kDecSlice + qb < nb;
    const int64_t qblk = (int64_t)qt * nb + s * kDecSlice + qb;
    u32x4_t v0 = {0u, 0u, 0u, 0u};
    if (quantizer) v0 = a.x[2 * qblk + qh];
    const int n16 = T * nb * 2;
    u32x4_t xv[kDecAmaxChunks];
#pragma unroll
    for (int c = 0; c < kDecAmaxChunks; ++c) {
      const int i = tid + c * kDecThreads;
      xv[c] = i < n16 ? a.x[i] : u32x4_t{0u, 0u, 0u, 0u};
    }
    uint32_t m = 0;
#pragma unroll
    for (int c = 0; c < kDecAmaxChunks; ++c)
      m = max(m, max(max(bf16_pair_absmax(xv[c][0]), bf16_pair_absmax(xv[c][1])),
                     max(bf16_pair_absmax(xv[c][2]), bf16_pair_absmax(xv[c][3]))));
    for (int i = tid + kDecAmaxChunks * kDecThreads; i < n16; i += kDecThreads) {  // T * D > 8192 only
      const u32x4_t v = a.x[i];
      m = max(m, max(max(bf16_pair_absmax(v[0]), bf16_pair_absmax(v[1])),
                     max(bf16_pair_absmax(v[2]), bf16_pair_absmax(v[3]))));
    }
    m = wave_max_u32(m);
    if (lane == 0) ured[wave] = m;
    __syncthreads();
    uint32_t mm = 0;
#pragma unroll
    for (int i = 0; i < kDecWaves; ++i) mm = max(mm, ured[i]);
    gsa = a.gsa_override ? ov : __uint_as_float(mm << 16) / kGsaDivisor;
    if (qt < T) {  // lanes past the end of K hold zero codes
      const uint32_t raw[4] = {v0[0], v0[1], v0[2], v0[3]};
      const uint32_t hm = bf16_words_absmax<4>(raw);
      const BlockScale bs = block_scale(max(hm, dpp_u<kDppXor1>(hm)), gsa);
      uint32_t c = 0u, sb = 0u;
      if (quantizer) {
        c = encode8(raw, bs, gsa);
        sb = bs.sbyte;
        if (g == 0) {
          *reinterpret_cast<uint32_t*>(a.xc + qblk * 8 + 4 * qh) = c;
          if (qh == 0) a.xs[qblk] = (uint8_t)sb;
        }
      }
      xq_lds[qt][qb][qh] = c;
      if (qh == 0) xs_lds[qt][qb] = sb;
    }
    if (n == 0 && tid == 0) *a.gsa = gsa;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      xq[t][0] = xq_lds[t][lane][0];
      xq[t][1] = xq_lds[t][lane][1];
      xsb[t] = xs_lds[t][lane];
    }
  } else {
    gsa = load_early(a.gsa);
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const int64_t blk = (int64_t)t * nb + j;
      xq[t][0] = xq[t][1] = xsb[t] = 0u;
      if (t < T && jok) {
        const uint2 v = *reinterpret_cast<const uint2*>(a.xc + blk * 8);
        xq[t][0] = v.x;
        xq[t][1] = v.y;
        xsb[t] = a.xs[blk];
      }
    }
  }

  // Block products: with both operands as fp16 values q * S (exact), a
  // block's 16 products and their sum are exact in fp32 (at most 12
  // significant bits between the smallest product and the largest sum), so
  // rounding starts only in the fixed-order sums over blocks and slices.
  // Lanes past the end of K hold zero codes and add nothing.
  half8_t w0[kDecEpw], w1[kDecEpw];
#pragma unroll
  for (int p = 0; p < kDecEpw; ++p) {
    const _Float16 sw = e4m3_f16(wsb[p]);
    w0[p] = fp4x8_to_f16(wq[p][0], sw);
    w1[p] = fp4x8_to_f16(wq[p][1], sw);
  }
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    if (t < T) {
      const _Float16 sx = e4m3_f16(xsb[t]);
      const half8_t x0 = fp4x8_to_f16(xq[t][0], sx), x1 = fp4x8_to_f16(xq[t][1], sx);
#pragma unroll
      for (int p = 0; p < kDecEpw; ++p) {
        const float sum = wave_sum(dot8(x1, w1[p], dot8(x0, w0[p], 0.0f)));
        const int e = g * kDecGroup + wave * kDecEpw + p;
        if (lane == 0 && e < E) store_coherent(a.part + ((int64_t)s * T + t) * E + e, sum);
      }
    }
  }

  if (!arrive_last(a.counter, a.nwg, &s_last)) return;

  // Wavefront t routes token t; it reads token t's slice partials in the
  // router's layout (lane l: experts l, l + 64, ...) and adds them in slice
  // order, times gsa * gsw (double, one final rounding to fp32). Partial
  // (q, t, e) sits at (q T + t) E + e. The loads of 8 slices are issued
  // together; slice indexes past the last one repeat it (not added).
  if (wave < T) {
    const int t = wave, ns = a.nslices;
    const double scale = (double)gsa * (double)gsw;
    float sum[EP];
#pragma unroll
    for (int jj = 0; jj < EP; ++jj) sum[jj] = 0.0f;
    for (int q0 = 0; q0 < ns; q0 += 8) {
      float v[8][EP];
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int jj = 0; jj < EP; ++jj)
          v[q][jj] = load_coherent(a.part + (min(q0 + q, ns - 1) * T + t) * E + min(lane + 64 * jj, E - 1));
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int jj = 0; jj < EP; ++jj) sum[jj] += q0 + q < ns ? v[q][jj] : 0.0f;
    }
    float L[EP];
#pragma unroll
    for (int jj = 0; jj < EP; ++jj) {
      L[jj] = (float)((double)sum[jj] * scale);
      const int e = lane + 64 * jj;
      if (a.logits_out && e < E) a.logits_out[t * E + e] = L[jj];
    }
    wave_route_regs<EP>(L, bv, E, a.k, a.routed_scale, a.idx + t * a.k, a.w + t * a.k, rsc[t]);
  }
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
  __shared__ float bias_s[512];
  __shared__ WaveRouteScratch<JMAX> rsc[4];
  __shared__ uint32_t s_last;
  extern __shared__ float lg[];  // [16][E]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float bias0 = (int)threadIdx.x < a.E ? a.bias[threadIdx.x] : 0.0f;
  const float bias1 = (int)threadIdx.x + 256 < a.E ? a.bias[threadIdx.x + 256] : 0.0f;
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
  if ((int)threadIdx.x < a.E) bias_s[threadIdx.x] = bias0;
  if ((int)threadIdx.x + 256 < a.E) bias_s[threadIdx.x + 256] = bias1;
  __syncthreads();
  for (int m = wave; m < nrows; m += 4) {
    const int64_t t = row0 + m;
    wave_route_row<JMAX>(lg + m * a.E, bias_s, a.E, a.k, a.routed_scale, a.idx + t * a.k, a.w + t * a.k,
                         rsc[wave]);
  }
  release_counter(&a.counters[blockIdx.y]);
}

// ---------------------------------------------------------------------------
// fused (prefill): one workgroup per BM tokens and all E experts, 4 waves.
//  * B (gate weights): wave w owns expert tiles w, w+4, ... (32 experts each,
//    NT per wave); each lane loads its 16 code bytes + 2 scale bytes per
//    64-element K step straight into registers and converts them to the
//    32x32x16 MFMA operand layout itself (no sharing needed, no LDS).
//  * A (tokens): the BM x 64 tile of each K step is converted once, by the
//    whole workgroup (one 16-byte chunk per thread), into an LDS buffer of fp16
//    values that every wave reads with ds_read_b128.
//  * Software pipeline: code bytes for step s+2 are loaded while step s runs
//    its MFMAs, then step s+1 is converted behind them; two LDS buffers.
//  * Epilogue: 32 rows at a time, scaled accumulators into LDS, then the
//    16-lanes-per-token router (four tokens per wavefront at once).
// ---------------------------------------------------------------------------
constexpr int kPrefillThreads = 256;
constexpr int kARowHalves = 72;  // LDS row stride of the A tile (64 values + 8 pad: fewer bank conflicts)

struct StepRegs {
  u32x4_t a;          // this thread's A chunk (16 code bytes)
  uint32_t as;        // its 2 scale bytes
  u32x4_t b[4];       // this lane's B chunk per expert tile
  uint32_t bs[4];
};

template <int BM, int NT>
__device__ __forceinline__ void prefill_load(StepRegs& R, const TileArgs& a, int row0, int wave, int lane, int step,
                                             int nsteps) {
  const int st = min(step, nsteps - 1);  // clamped: loads past the end re-read the last step (unused)
  const int tid = threadIdx.x;
  // A: thread t -> row t/2 of the tile, 32-element half t%2 of the step.
  {
    const int r = tid >> 1, hh = tid & 1;
    const int64_t row = row0 + r;
    const int64_t k0 = (int64_t)st * 64 + 32 * hh;
    const bool ok = tid < 2 * BM && row < a.T && k0 < a.D;
    R.a = u32x4_t{0u, 0u, 0u, 0u};
    R.as = 0u;
    if (ok) {
      R.a = *reinterpret_cast<const u32x4_t*>(a.xc + row * (a.D / 2) + k0 / 2);
      R.as = *reinterpret_cast<const uint16_t*>(a.xs + row * (a.D / 16) + k0 / 16);
    }
  }
  const int r = lane & 31, h = lane >> 5;
  const int64_t k0 = (int64_t)st * 64 + 32 * h;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t e = (int64_t)(wave + 4 * t) * 32 + r;
    R.b[t] = u32x4_t{0u, 0u, 0u, 0u};
    R.bs[t] = 0u;
    if (e < a.E && k0 < a.D) {
      R.b[t] = *reinterpret_cast<const u32x4_t*>(a.wc + e * (a.D / 2) + k0 / 2);
      R.bs[t] = *reinterpret_cast<const uint16_t*>(a.ws + e * (a.D / 16) + k0 / 16);
    }
  }
}

// The thread's A chunk, converted and stored in the LDS tile.
template <int BM>
__device__ __forceinline__ void prefill_store_a(const StepRegs& R, _Float16* abuf) {
  const int tid = threadIdx.x;
  if (tid < 2 * BM) {
    const int r = tid >> 1, hh = tid & 1;
    const _Float16 s0 = e4m3_f16(R.as & 0xFFu), s1 = e4m3_f16(R.as >> 8);
    half8_t* dst = reinterpret_cast<half8_t*>(abuf + r * kARowHalves + 32 * hh);
    dst[0] = fp4x8_to_f16(R.a[0], s0);
    dst[1] = fp4x8_to_f16(R.a[1], s0);
    dst[2] = fp4x8_to_f16(R.a[2], s1);
    dst[3] = fp4x8_to_f16(R.a[3], s1);
  }
}

template <int NT>
__device__ __forceinline__ void prefill_convert_b(const StepRegs& R, half8_t (&B)[NT][4]) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const _Float16 s0 = e4m3_f16(R.bs[t] & 0xFFu), s1 = e4m3_f16(R.bs[t] >> 8);
    B[t][0] = fp4x8_to_f16(R.b[t][0], s0);
    B[t][1] = fp4x8_to_f16(R.b[t][1], s0);
    B[t][2] = fp4x8_to_f16(R.b[t][2], s1);
    B[t][3] = fp4x8_to_f16(R.b[t][3], s1);
  }
}

template <int BM, int NT>
__device__ __forceinline__ void prefill_mfma(const _Float16* abuf, const half8_t (&B)[NT][4], int lane,
                                             f32x16_t (&acc)[BM / 32][NT]) {
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int rt = 0; rt < BM / 32; ++rt) {
    const half8_t* src = reinterpret_cast<const half8_t*>(abuf + (rt * 32 + r) * kARowHalves + 32 * h);
    half8_t A[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) A[j] = src[j];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[rt][t] = mfma32(A[j], B[t][j], acc[rt][t]);
  }
}

template <int BM, int NT, int J16>
union PrefillLds {
  _Float16 abuf[2][BM * kARowHalves];  // K loop: the converted A tiles
  Row16Scratch<J16> rsc[4];            // epilogue: one router scratch per wave
};

template <int BM, int NT, int J16>
__global__ __launch_bounds__(kPrefillThreads) void gate_fused_kernel(TileArgs a) {
  __shared__ __attribute__((aligned(16))) PrefillLds<BM, NT, J16> u;
  __shared__ float bias_s[512];
  extern __shared__ float lg[];  // [32][E + 16]
  _Float16 (&abuf)[2][BM * kARowHalves] = u.abuf;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row0 = blockIdx.x * BM;
  const int E = a.E;
  const int nsteps = (a.D + 63) / 64;
  const float bias0 = (int)threadIdx.x < E ? a.bias[threadIdx.x] : 0.0f;
  const float bias1 = (int)threadIdx.x + 256 < E ? a.bias[threadIdx.x + 256] : 0.0f;

  f32x16_t acc[BM / 32][NT];
#pragma unroll
  for (int rt = 0; rt < BM / 32; ++rt)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rt][t][v] = 0.0f;

  StepRegs R0, R1;
  half8_t B[NT][4];
  prefill_load<BM, NT>(R0, a, row0, wave, lane, 0, nsteps);
  prefill_load<BM, NT>(R1, a, row0, wave, lane, 1, nsteps);
  prefill_store_a<BM>(R0, abuf[0]);
  prefill_convert_b<NT>(R0, B);
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {
    // Even step s: LDS buffer 0, B from R0; R0 reloads step s+2.
    prefill_load<BM, NT>(R0, a, row0, wave, lane, s + 2, nsteps);
    prefill_mfma<BM, NT>(abuf[0], B, lane, acc);
    if (s + 1 >= nsteps) break;
    prefill_store_a<BM>(R1, abuf[1]);
    prefill_convert_b<NT>(R1, B);
    __syncthreads();
    // Odd step s+1: LDS buffer 1, B from R1; R1 reloads step s+3.
    prefill_load<BM, NT>(R1, a, row0, wave, lane, s + 3, nsteps);
    prefill_mfma<BM, NT>(abuf[1], B, lane, acc);
    if (s + 2 >= nsteps) break;
    prefill_store_a<BM>(R0, abuf[0]);
    prefill_convert_b<NT>(R0, B);
    __syncthreads();
  }

  // Epilogue, 32 rows at a time. 32x32 accumulator layout: value v of lane
  // (r, h) is row 8(v/4) + 4h + v%4, column r.
  const float scale = (*a.gsa) * (*a.gsw);
  const int ldE = E + 16;
  if ((int)threadIdx.x < E) bias_s[threadIdx.x] = bias0;
  if ((int)threadIdx.x + 256 < E) bias_s[threadIdx.x + 256] = bias1;
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int rt = 0; rt < BM / 32; ++rt) {
    if (row0 + rt * 32 >= a.T) break;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int e = (wave + 4 * t) * 32 + r;
      if (e < E) {
#pragma unroll
        for (int v = 0; v < 16; ++v) lg[(8 * (v >> 2) + 4 * h + (v & 3)) * ldE + e] = acc[rt][t][v] * scale;
      }
    }
    __syncthreads();
    const int base = row0 + rt * 32;
    // 32 rows: wave w routes rows 8w .. 8w+7, four at a time.
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int m = wave * 8 + half * 4 + (lane >> 4);
      const int64_t t = base + m;
      row16_route<J16>(lg + m * ldE, bias_s, E, a.k, a.routed_scale, t < a.T, a.idx + t * a.k, a.w + t * a.k,
                       u.rsc[wave]);
    }
    if (a.logits_out) {
      const int nrows = min(32, a.T - base);
      for (int i = threadIdx.x; i < nrows * E; i += kPrefillThreads) {
        const int m = i / E, e = i - m * E;
        a.logits_out[(int64_t)(base + m) * E + e] = lg[m * ldE + e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side: planning and launch.
// ---------------------------------------------------------------------------
static GateTuning read_tuning() {
  GateTuning t;
  if (const char* v = getenv("NVR_SPLIT_MAX_T")) t.split_max_t = atoi(v);
  if (const char* v = getenv("NVR_FUSED_BM")) t.fused_bm = atoi(v);
  if (t.split_max_t < 0) t.split_max_t = 0;
  if (t.split_max_t > 16 * kMaxCounters) t.split_max_t = 16 * kMaxCounters;
  return t;
}

const GateTuning& gate_tuning() {
  static const GateTuning t = read_tuning();
  return t;
}

static int decode_slices(int64_t D) { return (int)((D / 16 + kDecSlice - 1) / kDecSlice); }

GateKind gate_kind(int64_t T, int64_t D) {
  if (T <= kDecMaxT && decode_slices(D) <= kDecMaxSlices) return GateKind::kDecode;
  if (T <= gate_tuning().split_max_t) return GateKind::kTile;
  return GateKind::kFused;
}

size_t gate_scratch_bytes(int64_t T, int64_t D, int64_t E) {
  switch (gate_kind(T, D)) {
    case GateKind::kDecode: return (size_t)decode_slices(D) * (size_t)T * (size_t)E * sizeof(float);
    case GateKind::kTile: return (size_t)T * (size_t)E * sizeof(float);
    default: return 0;
  }
}

template <bool QUANT>
static hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  DecodeArgs b = a;
  b.nslices = decode_slices(a.D);
  b.nwg = (a.E + kDecGroup - 1) / kDecGroup * b.nslices;
  const int ep = (a.E + 63) / 64;
  if (ep <= 1) gate_decode_kernel<1, QUANT><<<b.nwg, kDecThreads, 0, stream>>>(b);
  else if (ep <= 2) gate_decode_kernel<2, QUANT><<<b.nwg, kDecThreads, 0, stream>>>(b);
  else if (ep <= 4) gate_decode_kernel<4, QUANT><<<b.nwg, kDecThreads, 0, stream>>>(b);
  else gate_decode_kernel<8, QUANT><<<b.nwg, kDecThreads, 0, stream>>>(b);
  return hipGetLastError();
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

template <int BM, int NT, int J16>
static hipError_t launch_fused_t(const TileArgs& a, hipStream_t stream) {
  const int grid = (a.T + BM - 1) / BM;
  const size_t lds = (size_t)32 * (a.E + 16) * sizeof(float);
  gate_fused_kernel<BM, NT, J16><<<grid, kPrefillThreads, lds, stream>>>(a);
  return hipGetLastError();
}

template <int BM>
static hipError_t launch_fused_bm(const TileArgs& a, hipStream_t stream) {
  const int nt = (a.E + 127) / 128;
  if (nt <= 1) return a.E <= 64 ? launch_fused_t<BM, 1, 4>(a, stream) : launch_fused_t<BM, 1, 8>(a, stream);
  if (nt <= 2) return launch_fused_t<BM, 2, 16>(a, stream);
  if (nt <= 3) return launch_fused_t<BM, 3, 24>(a, stream);
  return launch_fused_t<BM, 4, 32>(a, stream);
}

static hipError_t launch_fused(const TileArgs& a, hipStream_t stream) {
  // Row tile: the largest of 128 / 64 / 32 that still gives every compute
  // unit a workgroup (taller tiles reuse each converted weight for more rows).
  // 128-row tiles only for E <= 256 (their accumulators, 16 x (E/32) fp32
  // per lane, must stay in registers).
  const int bm = gate_tuning().fused_bm > 0 ? gate_tuning().fused_bm
                 : (a.T >= 128 * 256 && a.E <= 256 ? 128 : (a.T >= 64 * 256 ? 64 : 32));
  if (bm >= 128) return launch_fused_bm<128>(a, stream);
  if (bm >= 64) return launch_fused_bm<64>(a, stream);
  return launch_fused_bm<32>(a, stream);
}

hipError_t launch_gate(const uint8_t* xc, const uint8_t* xs, const float* gsa, const uint8_t* wc, const uint8_t* ws,
                       const float* gsw, const float* bias, float rs, int64_t T, int64_t D, int64_t E, int64_t k,
                       int32_t* idx, float* w, float* lo, uint32_t* counters, void* scratch, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const GateKind kind = gate_kind(T, D);
  float* lbuf = static_cast<float*>(scratch);
  if (kind == GateKind::kDecode) {
    DecodeArgs a{nullptr, nullptr, const_cast<uint8_t*>(xc), const_cast<uint8_t*>(xs), const_cast<float*>(gsa),
                 wc, ws, gsw, bias, rs, (int)T, (int)D, (int)E, (int)k, idx, w, lo,
                 lbuf, counters, 0, 0};
    return launch_decode<false>(a, stream);
  }
  TileArgs a{xc, xs, gsa, wc, ws, gsw, bias, rs, (int)T, (int)D, (int)E, (int)k, idx, w, lo, lbuf, counters,
             (int)((D + 127) / 128)};
  return kind == GateKind::kTile ? launch_tile(a, stream) : launch_fused(a, stream);
}

bool forward_single_launch(int64_t T, int64_t D) { return gate_kind(T, D) == GateKind::kDecode; }

hipError_t launch_forward_fused(const void* x, const float* gsa_override, uint8_t* xc, uint8_t* xs, float* gsa_out,
                                const uint8_t* wc, const uint8_t* ws, const float* gsw, const float* bias, float rs,
                                int64_t T, int64_t D, int64_t E, int64_t k, int32_t* idx, float* w, float* lo,
                                uint32_t* counters, void* scratch, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  DecodeArgs a{static_cast<const u32x4_t*>(x), gsa_override, xc, xs, gsa_out, wc, ws, gsw, bias, rs, (int)T, (int)D,
               (int)E, (int)k, idx, w, lo, static_cast<float*>(scratch), counters, 0, 0};
  return launch_decode<true>(a, stream);
}

}  // namespace nvr
