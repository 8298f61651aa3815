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

int decode_slices(int64_t D) { return (int)((D / 16 + kDecSlice - 1) / kDecSlice); }

bool decode_fits(int64_t T, int64_t D) { return T <= kDecMaxT && decode_slices(D) <= kDecMaxSlices; }

size_t decode_scratch_bytes(int64_t T, int64_t D, int64_t E) {
  return (size_t)decode_slices(D) * (size_t)T * (size_t)E * sizeof(float);
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

hipError_t launch_decode_gate(const uint8_t* xc, const uint8_t* xs, const float* gsa, const uint8_t* wc,
                              const uint8_t* ws, const float* gsw, const float* bias, float rs, int64_t T, int64_t D,
                              int64_t E, int64_t k, int32_t* idx, float* w, float* lo, float* lbuf,
                              uint32_t* counters, hipStream_t stream) {
  DecodeArgs a{nullptr, nullptr, const_cast<uint8_t*>(xc), const_cast<uint8_t*>(xs), const_cast<float*>(gsa),
               wc, ws, gsw, bias, rs, (int)T, (int)D, (int)E, (int)k, idx, w, lo, lbuf, counters, 0, 0};
  return launch_decode<false>(a, stream);
}

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
