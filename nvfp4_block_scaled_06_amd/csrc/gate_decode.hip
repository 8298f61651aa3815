// Decode-size gate (T <= 4 tokens) with the routing epilogue fused after it
// (gfx950), and the single-launch router call that also quantizes x.
//
// logits[t, e] = gsa * gsw * sum_d (q_x S_x)[t, d] * (q_w S_w)[e, d]: the gate
// GEMM on NVFP4 operands (commit 04cf8ca8, dsv4/layers/router.py, NVFP4 gate
// paragraph), followed by the six-step epilogue (commit e0f60b9f,
// dsv4/kernels/router/__init__.py). At this size the projection is a GEMV
// that streams the packed weights: dot products of exact fp16 code values
// on the VALU, no MFMA.
#include "gate_common.hpp"

namespace nvr {

// ---------------------------------------------------------------------------
// decode: T <= 4 and D <= 16384. Workgroup (g, s) owns the 16 experts of
// group g and K slice s (64 blocks, one per lane); each of its 8 wavefronts
// owns 2 of the experts over the whole slice. Per expert row a workgroup
// reads 512 code bytes (four whole 128-byte lines) and 64 scale bytes, and
// the slices of one group run on one XCD, so no weight line is fetched into
// two L2s except at group boundaries.
//
// Quantizing variant: every workgroup reads all of x for the global max
// (from L2 after the first workgroup of its XCD), then all 512 threads
// quantize the T x 64 blocks of the slice, LPB = 512 / (64 T') lanes per
// block (T' = T rounded up to a power of two): 8 lanes of 2 elements each at
// T = 1. Group 0 stores the codes and scales, workgroup 0 stores gsa.
//
// Handoff without counters or waits: each wavefront sums its exact block
// products over the slice and stores one partial per (token, expert) as a
// flagged 32-bit word (below) with a device-coherent store, and does not wait
// for it. The workgroup dispatched last (the highest id) is also the
// consumer: after its own partials, wavefront t polls token t's partials
// until every flag is set and adds them in slice order; then the other
// wavefronts store zero over every word of the call while wavefront t routes
// token t. The flagged words live in a
// workspace region that no other kernel writes and that every call leaves
// zero, so a set flag is always this call's. The consumer waits only for
// workgroups that never wait, so the poll ends once they have stored; it is
// bounded all the same (kDecPollCap rounds, seconds).
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
  uint32_t* part;  // [nslices, T, E] flagged partials (the workspace's decode region, zero between calls)
  int nslices;     // K slices of 64 blocks
  int nwg;         // workgroups: expert groups * nslices
};

constexpr int kDecMaxT = 4;
constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecEpw = 2;                         // experts per wavefront
constexpr int kDecGroup = kDecWaves * kDecEpw;     // experts per workgroup
constexpr int kDecSlice = 64;                      // K blocks per slice
constexpr int kDecMaxSlices = 16;
constexpr int kDecAmaxChunks = 4;                  // 16-byte chunks of x per thread in the first max pass
constexpr int kDecPollCap = 1 << 22;
static_assert((size_t)kDecMaxSlices * kDecMaxT * 512 * sizeof(uint32_t) <= kDecodeRegionBytes,
              "the decode region holds every partial of the largest decode call");

// A flagged word is the partial's fp32 bits XOR kFlagXor, so 0 means "not
// written yet". It is nonzero for every partial: a partial equal to the
// pattern kFlagXor (a NaN whose lowest payload bit is set) would need a NaN
// input with that payload bit, and the only NaNs that can enter these sums
// come from fp16 operands (out-of-range scale bytes), whose payloads have
// their low 13 bits clear once in fp32.
constexpr uint32_t kFlagXor = 0x7FC00001u;

__device__ __forceinline__ void store_flagged(uint32_t* p, float v) {
  __hip_atomic_store(p, __float_as_uint(v) ^ kFlagXor, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t load_flagged(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void clear_flagged(uint32_t* p) {
  __hip_atomic_store(p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Codes of NW bf16 pairs under block scale b, packed two per byte (the even
// element in the low nibble): NW bytes.
template <int NW>
__device__ __forceinline__ uint32_t encode_pairs(const uint32_t* w, const BlockScale& b, float gsa) {
  if (b.fast) {
    uint32_t o = fp4_exact_pair<0>(0u, w[0], b.inv, b.S, gsa);
    if constexpr (NW > 1) o = fp4_exact_pair<1>(o, w[1], b.inv, b.S, gsa);
    if constexpr (NW > 2) o = fp4_exact_pair<2>(o, w[2], b.inv, b.S, gsa);
    if constexpr (NW > 3) o = fp4_exact_pair<3>(o, w[3], b.inv, b.S, gsa);
    return o;
  }
  uint32_t out = 0u;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    uint32_t lo = (w[i] >> 12) & 0x8u, hi = (w[i] >> 28) & 0x8u;  // sign bits: a zero scale leaves only these
    if (b.S != 0.0f) {
      lo |= e2m1_round(fabs((double)bf16_lo(w[i])) / b.G64);
      hi |= e2m1_round(fabs((double)bf16_hi(w[i])) / b.G64);
    }
    out |= (lo | (hi << 4)) << (8 * i);
  }
  return out;
}

// Largest 15-bit magnitude pattern over aligned groups of G lanes (G = 2, 4
// or 8): every lane of a group gets it.
template <int G>
__device__ __forceinline__ uint32_t lanes_max(uint32_t v) {
  if constexpr (G >= 2) v = max(v, dpp_u<kDppXor1>(v));
  if constexpr (G >= 4) v = max(v, dpp_u<kDppXor2>(v));
  if constexpr (G >= 8) v = max(v, dpp_u<kDppHalfMirror>(v));
  return v;
}

// gsa of the call: max|x| over all of x (every thread of the workgroup
// strides over it; the 15-bit magnitude patterns order like the values),
// divided by 2688 in fp32. Every workgroup derives it this same way, so all
// of them hold the same bits. The loads are issued first (decode_x_load), the
// reduction comes later (decode_gsa).
struct XChunks {
  u32x4_t v[kDecAmaxChunks];
};

__device__ __forceinline__ XChunks decode_x_load(const DecodeArgs& a) {
  XChunks c;
  const int n16 = a.T * (a.D >> 4) * 2;
#pragma unroll
  for (int i = 0; i < kDecAmaxChunks; ++i) {
    const int idx = threadIdx.x + i * kDecThreads;
    c.v[i] = idx < n16 ? a.x[idx] : u32x4_t{0u, 0u, 0u, 0u};
  }
  return c;
}

__device__ __forceinline__ float decode_gsa(const DecodeArgs& a, const XChunks& c, uint32_t* ured) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = a.T * (a.D >> 4) * 2;
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < kDecAmaxChunks; ++i)
    m = max(m, max(max(bf16_pair_absmax(c.v[i][0]), bf16_pair_absmax(c.v[i][1])),
                   max(bf16_pair_absmax(c.v[i][2]), bf16_pair_absmax(c.v[i][3]))));
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
  return __uint_as_float(mm << 16) / kGsaDivisor;
}

// The consumer workgroup, all its wavefronts: wavefront t < T takes token t.
// Lane l holds experts l, l + 64, ... (bias bv) and adds their slice
// partials in slice order, times gsa * gsw (double, one final rounding to
// fp32). Partial (q, t, e) sits at (q T + t) E + e. A round loads QC slices;
// slice indexes past the last one repeat it (not added), experts past E
// repeat the last one (not routed). Once every token's partials are in (a
// workgroup barrier), the other wavefronts clear the whole region of this
// call while the first T route.
template <int EP>
__device__ __forceinline__ void decode_consume(const DecodeArgs& a, float gsa, float gsw, const float (&bv)[EP],
                                               WaveRouteScratch<EP>* rsc) {
  const int lane = threadIdx.x & 63, t = threadIdx.x >> 6;
  const int T = a.T, E = a.E, ns = a.nslices;
  constexpr int QC = EP >= 8 ? 4 : 8;
  float sum[EP];
#pragma unroll
  for (int jj = 0; jj < EP; ++jj) sum[jj] = 0.0f;
  if (t < T) {
    for (int q0 = 0; q0 < ns; q0 += QC) {
      uint32_t v[QC][EP];
      // One round at a time: a second round in flight would still be loading
      // into registers when the first one completes, and the routing that
      // follows would wait for it.
      for (int spin = 0; spin < kDecPollCap; ++spin) {
#pragma unroll
        for (int q = 0; q < QC; ++q)
#pragma unroll
          for (int jj = 0; jj < EP; ++jj)
            v[q][jj] =
                load_flagged(a.part + (int64_t)(min(q0 + q, ns - 1) * T + t) * E + min(lane + 64 * jj, E - 1));
        bool ready = true;
#pragma unroll
        for (int q = 0; q < QC; ++q)
#pragma unroll
          for (int jj = 0; jj < EP; ++jj) ready = ready && v[q][jj] != 0u;
        if (__all(ready)) break;
      }
#pragma unroll
      for (int q = 0; q < QC; ++q)
#pragma unroll
        for (int jj = 0; jj < EP; ++jj) sum[jj] += q0 + q < ns ? __uint_as_float(v[q][jj] ^ kFlagXor) : 0.0f;
    }
  }
  __syncthreads();
  if (t >= T) {
    // Every word this call wrote has been read: clear them for the next
    // call, 16 bytes per store (the region is 16-byte aligned).
    const int nwords = ns * T * E, n16 = nwords >> 2;
    const int i0 = threadIdx.x - 64 * T, stride = kDecThreads - 64 * T;
    u32x4_t* p16 = reinterpret_cast<u32x4_t*>(a.part);
    for (int i = i0; i < n16; i += stride) p16[i] = u32x4_t{0u, 0u, 0u, 0u};
    if (i0 < (nwords & 3)) a.part[4 * n16 + i0] = 0u;
    return;
  }
  const double scale = (double)gsa * (double)gsw;
  float L[EP];
#pragma unroll
  for (int jj = 0; jj < EP; ++jj) {
    L[jj] = (float)((double)sum[jj] * scale);
    const int e = lane + 64 * jj;
    if (a.logits_out && e < E) a.logits_out[t * E + e] = L[jj];
  }
  wave_route_regs<EP>(L, bv, E, a.k, a.routed_scale, a.idx + t * a.k, a.w + t * a.k, rsc[t]);
}

template <int EP, bool QUANT, int LPB>
__global__ __launch_bounds__(kDecThreads) void gate_decode_kernel(DecodeArgs a) {
  constexpr int TM = kDecMaxT;
  constexpr int NW = 8 / LPB;  // bf16 pairs each quantizing lane holds
  __shared__ uint32_t ured[kDecWaves];
  __shared__ __attribute__((aligned(8))) uint8_t xq_lds[TM][kDecSlice][8];
  __shared__ uint8_t xs_lds[TM][kDecSlice];
  __shared__ WaveRouteScratch<EP> rsc[TM];
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
  const bool consumer = blockIdx.x == gridDim.x - 1;

  // Every global load is issued before the first use (predicated by lane,
  // not by uniform branches), x first: the global max waits for it, the
  // weights are needed only after the quantization.
  XChunks xall;
  // Thread tid quantizes NW pairs of block qb of token qt's slice; the LPB
  // lanes of a block are adjacent and take its dwords in order.
  const int qt = tid / (64 * LPB), qb = (tid / LPB) & 63, qh = tid & (LPB - 1);
  const bool quantizer = qt < T && s * kDecSlice + qb < nb;
  const int64_t qblk = (int64_t)qt * nb + s * kDecSlice + qb;
  uint32_t xw[NW];
  if constexpr (QUANT) {
    xall = decode_x_load(a);
    const uint32_t* src = reinterpret_cast<const uint32_t*>(a.x) + qblk * 8 + qh * NW;
    if constexpr (NW == 4) {
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (quantizer) v = *reinterpret_cast<const u32x4_t*>(src);
      xw[0] = v[0]; xw[1] = v[1]; xw[2] = v[2]; xw[3] = v[3];
    } else if constexpr (NW == 2) {
      uint2 v = make_uint2(0u, 0u);
      if (quantizer) v = *reinterpret_cast<const uint2*>(src);
      xw[0] = v.x; xw[1] = v.y;
    } else {
      xw[0] = quantizer ? *src : 0u;
    }
  }
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

  float bv[EP];  // the consumer's bias of experts lane + 64 jj
#pragma unroll
  for (int jj = 0; jj < EP; ++jj) bv[jj] = consumer ? a.bias[min(lane + 64 * jj, E - 1)] : 0.0f;
  const float gsw = consumer ? load_early(a.gsw) : 0.0f;

  float gsa;
  uint32_t xq[TM][2], xsb[TM];
  if constexpr (QUANT) {
    const float ov = a.gsa_override ? load_early(a.gsa_override) : 0.0f;
    const float runtime_gsa = decode_gsa(a, xall, ured);
    gsa = a.gsa_override ? ov : runtime_gsa;
    if (qt < T) {  // lanes past the end of K hold zero codes
      const BlockScale bs = block_scale(lanes_max<LPB>(bf16_words_absmax<NW>(xw)), gsa);
      uint32_t c = 0u, sb = 0u;
      if (quantizer) {
        c = encode_pairs<NW>(xw, bs, gsa);
        sb = bs.sbyte;
        if (g == 0) {
          uint8_t* dst = a.xc + qblk * 8 + qh * NW;
          if constexpr (NW == 4) *reinterpret_cast<uint32_t*>(dst) = c;
          else if constexpr (NW == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)c;
          else *dst = (uint8_t)c;
          if (qh == 0) a.xs[qblk] = (uint8_t)sb;
        }
      }
      uint8_t* l = &xq_lds[qt][qb][qh * NW];
      if constexpr (NW == 4) *reinterpret_cast<uint32_t*>(l) = c;
      else if constexpr (NW == 2) *reinterpret_cast<uint16_t*>(l) = (uint16_t)c;
      else *l = (uint8_t)c;
      if (qh == 0) xs_lds[qt][qb] = (uint8_t)sb;
    }
    if (n == 0 && tid == 0) *a.gsa = gsa;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const uint2 v = *reinterpret_cast<const uint2*>(xq_lds[t][lane]);
      xq[t][0] = v.x;
      xq[t][1] = v.y;
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
        if (lane == 0 && e < E) store_flagged(a.part + ((int64_t)s * T + t) * E + e, sum);
      }
    }
  }
  if (consumer) decode_consume<EP>(a, gsa, gsw, bv, rsc);
}

int decode_slices(int64_t D) { return (int)((D / 16 + kDecSlice - 1) / kDecSlice); }

bool decode_fits(int64_t T, int64_t D) { return T <= kDecMaxT && decode_slices(D) <= kDecMaxSlices; }

// Lanes per quantized block: 512 threads over the T' x 64 blocks of a slice.
template <int EP, bool QUANT>
static void launch_decode_ep(const DecodeArgs& b, hipStream_t stream) {
  if constexpr (QUANT) {
    if (b.T == 1) gate_decode_kernel<EP, true, 8><<<b.nwg, kDecThreads, 0, stream>>>(b);
    else if (b.T == 2) gate_decode_kernel<EP, true, 4><<<b.nwg, kDecThreads, 0, stream>>>(b);
    else gate_decode_kernel<EP, true, 2><<<b.nwg, kDecThreads, 0, stream>>>(b);
  } else {
    gate_decode_kernel<EP, false, 2><<<b.nwg, kDecThreads, 0, stream>>>(b);
  }
}

template <bool QUANT>
static hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  DecodeArgs b = a;
  b.nslices = decode_slices(a.D);
  b.nwg = (a.E + kDecGroup - 1) / kDecGroup * b.nslices;
  const int ep = (a.E + 63) / 64;
  if (ep <= 1) launch_decode_ep<1, QUANT>(b, stream);
  else if (ep <= 2) launch_decode_ep<2, QUANT>(b, stream);
  else if (ep <= 4) launch_decode_ep<4, QUANT>(b, stream);
  else launch_decode_ep<8, QUANT>(b, stream);
  return hipGetLastError();
}

hipError_t launch_decode_gate(const uint8_t* xc, const uint8_t* xs, const float* gsa, const uint8_t* wc,
                              const uint8_t* ws, const float* gsw, const float* bias, float rs, int64_t T, int64_t D,
                              int64_t E, int64_t k, int32_t* idx, float* w, float* lo, void* workspace,
                              hipStream_t stream) {
  DecodeArgs a{nullptr, nullptr, const_cast<uint8_t*>(xc), const_cast<uint8_t*>(xs), const_cast<float*>(gsa),
               wc, ws, gsw, bias, rs, (int)T, (int)D, (int)E, (int)k, idx, w, lo,
               reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + kDecodeRegionOffset), 0, 0};
  return launch_decode<false>(a, stream);
}

hipError_t launch_forward_fused(const void* x, const float* gsa_override, uint8_t* xc, uint8_t* xs, float* gsa_out,
                                const uint8_t* wc, const uint8_t* ws, const float* gsw, const float* bias, float rs,
                                int64_t T, int64_t D, int64_t E, int64_t k, int32_t* idx, float* w, float* lo,
                                void* workspace, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  DecodeArgs a{static_cast<const u32x4_t*>(x), gsa_override, xc, xs, gsa_out, wc, ws, gsw, bias, rs, (int)T, (int)D,
               (int)E, (int)k, idx, w, lo,
               reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + kDecodeRegionOffset), 0, 0};
  return launch_decode<true>(a, stream);
}

}  // namespace nvr
