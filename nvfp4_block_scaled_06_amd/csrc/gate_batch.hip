// Batched-decode router (4 < T <= 256 tokens, D <= 16384) in two launches
// (gfx950): runtime NVFP4 quantization of x, the block-scaled gate
// projection and the six-step routing epilogue (commit 04cf8ca8,
// dsv4/layers/router.py; commit e0f60b9f, dsv4/kernels/router/__init__.py).
//
//  1. batch_amax_zero_kernel: every workgroup takes the largest |x| of its
//     share of x (one partial maximum each) and zeroes its share of this
//     call's flag region (the kernel boundary orders both before launch 2).
//  2. gate_batch_kernel: workgroup (token tile, K slice, expert block) =
//     16 tokens x 256 elements x 128 experts, 8 wavefronts (the slice is
//     short so that the quantization and operand conversion, which bound a
//     workgroup's time, are spread over as many compute units as the
//     batch-decode sizes fill).
//     - Loads first, in the order they are needed: the partial maxima, this
//       thread's half block of x, its weight chunks.
//     - gsa from the partial maxima (every workgroup the same bits); each
//       lane pair quantizes one block of the 16 x 256 x tile (exact
//       rounding) into an LDS tile of fp16 q S values; the workgroups of
//       expert block 0 also store the codes and scales.
//     - 16x16x32 f16 MFMAs: wavefront w takes experts 16 w .. 16 w + 15 of
//       the block over the whole slice; each lane loads 32 consecutive K of
//       its weight row and feeds four MFMAs with them, the A tile giving the
//       same K values (a K permutation that A and B share).
//     - Each (token, expert) slice partial goes out as a flagged word with a
//       device-coherent store, without waiting.
//     - The ceil(T / 2) workgroups dispatched last are also consumers:
//       consumer c takes tokens 2 c and 2 c + 1 (then every 2 ncons-th pair
//       after them); four wavefronts per token each poll and add the
//       partials of a quarter of the slices, and the first of them adds the
//       other quarters' sums (through LDS, in quarter order) and routes the
//       token.
//
// The partial values are exact block sums added in fp32; a flagged word is
// the partial's bits XOR kBatchFlagXor (a NaN pattern no sum takes), so the
// zeroed region tells unwritten words apart. The consumers run last in
// dispatch order and every producer finishes without waiting, so their
// polls always end (a cap bounds them regardless).
#include <algorithm>

#include "gate_common.hpp"

namespace nvr {

constexpr int kBatchRows = 16;       // tokens per workgroup tile
constexpr int kBatchSlice = 256;     // K elements per slice (16 blocks)
constexpr int kBatchSteps = kBatchSlice / 128;  // 32-element chunks per lane
constexpr int kBatchExperts = 128;   // experts per workgroup (16 per wavefront)
constexpr int kBatchThreads = 512;   // 8 wavefronts
constexpr int kBatchMaxSlices = 64;  // D <= 16384
constexpr int kBatchMaxTokens = 256;
constexpr int kBatchConsTokens = 2;  // tokens per consumer workgroup
constexpr int kBatchConsSplit = 4;   // wavefronts per token, each adding a part of the slices
constexpr int kBatchALd = kBatchSlice + 8;  // LDS row stride of the A tile in halves
constexpr int kBatchPollCap = 1 << 22;
constexpr uint32_t kBatchFlagXor = 0x7FC00001u;

struct BatchArgs {
  const u32x4_t* x;           // bf16 [T, D]
  const float* gsa_override;  // NULL = runtime gsa
  const uint32_t* partial;    // partial maxima of launch 1 (15-bit magnitude patterns)
  int npartial;
  uint8_t* xc;  // [T, D/2] out
  uint8_t* xs;  // [T, D/16] out
  float* gsa_out;
  const uint8_t* wc;
  const uint8_t* ws;
  const float* gsw;
  const float* bias;
  float routed_scale;
  int T, D, E, k;
  int32_t* idx;
  float* w;
  float* logits_out;
  uint32_t* part;  // [ns, T, E] flagged partials, zeroed by launch 1
  int ns, ntt, neb, nwg, ncons;
};

// 32 elements of weight row e from element kk (load_chunk's layout), read
// without a branch: a chunk past E or D reads a clamped in-bounds chunk and
// is zeroed afterwards (no conditional block in front of later loads).
__device__ __forceinline__ Chunk32 load_chunk_clamped(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales, int e, int E, int64_t kk,
                                                      int64_t D) {
  const bool ok = e < E && kk < D;
  const int64_t row = min(e, E - 1), k0 = min(kk, D - 32);
  Chunk32 ch;
  ch.c = *reinterpret_cast<const u32x4_t*>(codes + row * (D / 2) + k0 / 2);
  ch.s = *reinterpret_cast<const uint16_t*>(scales + row * (D / 16) + k0 / 16);
  if (!ok) {
    ch.c = u32x4_t{0u, 0u, 0u, 0u};
    ch.s = 0u;
  }
  return ch;
}

__device__ __forceinline__ uint32_t u32x4_absmax(u32x4_t v) {
  return max(max(bf16_pair_absmax(v[0]), bf16_pair_absmax(v[1])), max(bf16_pair_absmax(v[2]), bf16_pair_absmax(v[3])));
}

// Launch 1: one partial maximum per workgroup over a grid-stride share of x
// (nvec 16-byte vectors; none when the scale is given), and zeros over
// nzero16 16-byte words of the flag region.
__global__ __launch_bounds__(kBatchThreads) void batch_amax_zero_kernel(const u32x4_t* __restrict__ x, int64_t nvec,
                                                                        uint32_t* __restrict__ partial,
                                                                        u32x4_t* __restrict__ zero, int64_t nzero16) {
  __shared__ uint32_t red[kBatchThreads / 64];
  const int64_t stride = (int64_t)gridDim.x * kBatchThreads;
  const int64_t i0 = (int64_t)blockIdx.x * kBatchThreads + threadIdx.x;
  uint32_t m = 0;
  for (int64_t i = i0; i < nvec; i += stride) m = max(m, u32x4_absmax(x[i]));
  for (int64_t i = i0; i < nzero16; i += stride) zero[i] = u32x4_t{0u, 0u, 0u, 0u};
  if (nvec == 0) return;
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t mm = 0;
#pragma unroll
    for (int i = 0; i < kBatchThreads / 64; ++i) mm = max(mm, red[i]);
    partial[blockIdx.x] = mm;
  }
}

template <int EP>
__global__ __launch_bounds__(kBatchThreads) void gate_batch_kernel(BatchArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 atile[kBatchRows * kBatchALd];
  __shared__ uint32_t ured[kBatchThreads / 64];
  __shared__ float comb[kBatchConsTokens][kBatchConsSplit - 1][EP][64];
  __shared__ WaveRouteScratch<EP> rsc[kBatchConsTokens];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, E = a.E, D = a.D, nb = D >> 4;
  // Workgroup ids go to the 8 XCDs in turn; consecutive numbers run on one
  // XCD: the token tiles of one (slice, expert block) first (they share its
  // weight tile), then the expert blocks (they share the x tile).
  const int nq = a.nwg >> 3, nr = a.nwg & 7, bx = blockIdx.x & 7;
  const int n = bx * nq + min(bx, nr) + (blockIdx.x >> 3);
  const int tt = n % a.ntt, rest = n / a.ntt;
  const int eb = rest % a.neb, s = rest / a.neb;
  const int row0 = tt * kBatchRows, e0 = eb * kBatchExperts;

  // Loads, all issued before the first wait and in the order they are
  // needed: the scale override (read from a valid address either way, and
  // first: the runtime branch reuses its register, which waits for it), the
  // partial maxima (two per thread; clamped indexes repeat a value, which a
  // maximum ignores), this thread's half block of x (half qh of block qb of
  // the slice, row qr of the tile), two 32-element weight chunks. Addresses
  // out of range are clamped and the values zeroed, so no load sits in a
  // conditional block (the compiler waits for every load in flight at such
  // a block's end).
  const bool runtime = a.gsa_override == nullptr;
  const float ov = load_early(runtime ? a.gsw : a.gsa_override);
  const int np = max(a.npartial, 1);  // launch 1 wrote npartial >= 1 values when runtime
  const uint32_t pm0 = a.partial[min(tid, np - 1)];
  const uint32_t pm1 = a.partial[min(tid + kBatchThreads, np - 1)];
  const int qr = tid >> 5, qb = (tid >> 1) & 15, qh = tid & 1;
  const int qt = row0 + qr, blk = s * (kBatchSlice / 16) + qb;
  const bool qok = qt < T && blk < nb;
  u32x4_t xv = a.x[qok ? ((int64_t)qt * nb + blk) * 2 + qh : 0];
  const int col = lane & 15, g = lane >> 4;
  const int e = e0 + 16 * wave + col;
  Chunk32 bc[kBatchSteps];
#pragma unroll
  for (int st = 0; st < kBatchSteps; ++st)
    bc[st] = load_chunk_clamped(a.wc, a.ws, e, E, (int64_t)s * kBatchSlice + st * 128 + 32 * g, D);
  if (!qok) xv = u32x4_t{0u, 0u, 0u, 0u};

  float gsa;
  if (runtime) {
    const uint32_t pm = wave_max_u32(max(pm0, pm1));
    if (lane == 0) ured[wave] = pm;
    __syncthreads();
    uint32_t mm = 0;
#pragma unroll
    for (int i = 0; i < kBatchThreads / 64; ++i) mm = max(mm, ured[i]);
    gsa = __uint_as_float(mm << 16) / kGsaDivisor;
  } else {
    gsa = ov;
  }

  // Quantize: the two lanes of a block share its maximum (one DPP step) and
  // each encodes its 8 elements; the A tile gets their fp16 q S values (zeros
  // past T or D: code 0, scale 0).
  {
    const uint32_t wv[4] = {xv[0], xv[1], xv[2], xv[3]};
    const BlockScale bs = block_scale(group_max_u32<2>(bf16_words_absmax<4>(wv)), gsa);
    uint32_t c = encode8(wv, bs, gsa), sb = bs.sbyte;
    if (!qok) c = sb = 0u;
    if (eb == 0 && qok) {
      const int64_t b = (int64_t)qt * nb + blk;
      *reinterpret_cast<uint32_t*>(a.xc + b * 8 + qh * 4) = c;
      if (qh == 0) a.xs[b] = (uint8_t)sb;
    }
    *reinterpret_cast<half8_t*>(atile + qr * kBatchALd + 16 * qb + 8 * qh) = fp4x8_to_f16(c, e4m3_f16(sb));
  }
  if (n == 0 && tid == 0) *a.gsa_out = gsa;
  __syncthreads();

  // MFMAs: lane (col, g) gives K values kl + 8 j .. + 7 of token row col (A)
  // and of expert e (B) to MFMA j.
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < kBatchSteps; ++st) {
    const int kl = st * 128 + 32 * g;
    const half8_t* ap = reinterpret_cast<const half8_t*>(atile + col * kBatchALd + kl);
    const _Float16 sb0 = e4m3_f16(bc[st].s & 0xFFu), sb1 = e4m3_f16(bc[st].s >> 8);
    acc = mfma16(ap[0], fp4x8_to_f16(bc[st].c[0], sb0), acc);
    acc = mfma16(ap[1], fp4x8_to_f16(bc[st].c[1], sb0), acc);
    acc = mfma16(ap[2], fp4x8_to_f16(bc[st].c[2], sb1), acc);
    acc = mfma16(ap[3], fp4x8_to_f16(bc[st].c[3], sb1), acc);
  }
  // 16x16 accumulator layout: lane (col, g) holds token rows 4 g .. 4 g + 3
  // of expert column col.
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int t = row0 + 4 * g + v;
    if (t < T && e < E)
      __hip_atomic_store(a.part + ((int64_t)s * T + t) * E + e, __float_as_uint(acc[v]) ^ kBatchFlagXor,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  const int cons = a.nwg - 1 - (int)blockIdx.x;
  if (cons >= a.ncons) return;
  // Consumer: wavefront w takes token p = w % 2 of this workgroup's pair and
  // part h = w / 2 of the slices. Lane l holds experts l, l + 64, ...; a wave
  // adds slices h qs .. min(ns, (h + 1) qs) - 1 in order, QC per polling
  // round (indexes past its last slice repeat it and are not added; experts
  // past E repeat the last one and are not routed). The first part's wave
  // adds the other parts' sums in part order and routes the token.
  const int p = wave % kBatchConsTokens, h = wave / kBatchConsTokens;
  const int ns = a.ns, qs = (ns + kBatchConsSplit - 1) / kBatchConsSplit;
  const int q_begin = min(ns, h * qs), q_end = min(ns, q_begin + qs);
  const float gsw = load_early(a.gsw);
  float bv[EP];
#pragma unroll
  for (int jj = 0; jj < EP; ++jj) bv[jj] = h == 0 ? a.bias[min(lane + 64 * jj, E - 1)] : 0.0f;
  const double scale = (double)gsa * (double)gsw;
  constexpr int QC = EP >= 8 ? 4 : 8;
  for (int base = kBatchConsTokens * cons; base < T; base += kBatchConsTokens * a.ncons) {
    const int t = base + p;
    float sum[EP];
#pragma unroll
    for (int jj = 0; jj < EP; ++jj) sum[jj] = 0.0f;
    if (t < T) {
      for (int q0 = q_begin; q0 < q_end; q0 += QC) {
        uint32_t v[QC][EP];
        for (int spin = 0; spin < kBatchPollCap; ++spin) {
#pragma unroll
          for (int q = 0; q < QC; ++q)
#pragma unroll
            for (int jj = 0; jj < EP; ++jj)
              v[q][jj] = __hip_atomic_load(
                  a.part + ((int64_t)min(q0 + q, q_end - 1) * T + t) * E + min(lane + 64 * jj, E - 1),
                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
          for (int jj = 0; jj < EP; ++jj)
            sum[jj] += q0 + q < q_end ? __uint_as_float(v[q][jj] ^ kBatchFlagXor) : 0.0f;
      }
      if (h > 0) {
#pragma unroll
        for (int jj = 0; jj < EP; ++jj) comb[p][h - 1][jj][lane] = sum[jj];
      }
    }
    __syncthreads();
    if (h == 0 && t < T) {
      float L[EP];
#pragma unroll
      for (int jj = 0; jj < EP; ++jj) {
        float tot = sum[jj];
#pragma unroll
        for (int o = 0; o < kBatchConsSplit - 1; ++o) tot += comb[p][o][jj][lane];
        L[jj] = (float)((double)tot * scale);
        const int ex = lane + 64 * jj;
        if (a.logits_out && ex < E) a.logits_out[(int64_t)t * E + ex] = L[jj];
      }
      wave_route_regs<EP>(L, bv, E, a.k, a.routed_scale, a.idx + (int64_t)t * a.k, a.w + (int64_t)t * a.k, rsc[p]);
    }
    __syncthreads();  // comb is rewritten by the next token pair
  }
}

static int batch_slices(int64_t D) { return (int)((D + kBatchSlice - 1) / kBatchSlice); }

bool batch_fits(int64_t T, int64_t D) {
  return T >= 1 && T <= kBatchMaxTokens && !decode_fits(T, D) && batch_slices(D) <= kBatchMaxSlices;
}

size_t batch_scratch_bytes(int64_t T, int64_t D, int64_t E) {
  // The flag region is zeroed in whole 16-byte words.
  const size_t words = (size_t)batch_slices(D) * (size_t)T * (size_t)E;
  return (size_t)kAmaxPartials * sizeof(uint32_t) + (words + 3) / 4 * 16;
}

template <int EP>
static void launch_batch_ep(const BatchArgs& b, hipStream_t stream) {
  gate_batch_kernel<EP><<<b.nwg, kBatchThreads, 0, stream>>>(b);
}

hipError_t launch_forward_batch(const void* x, const float* gsa_override, uint8_t* xc, uint8_t* xs, float* gsa_out,
                                const uint8_t* wc, const uint8_t* ws, const float* gsw, const float* bias, float rs,
                                int64_t T, int64_t D, int64_t E, int64_t k, int32_t* idx, float* w, float* lo,
                                void* scratch, hipStream_t stream) {
  BatchArgs a{};
  a.x = static_cast<const u32x4_t*>(x);
  a.gsa_override = gsa_override;
  a.xc = xc;
  a.xs = xs;
  a.gsa_out = gsa_out;
  a.wc = wc;
  a.ws = ws;
  a.gsw = gsw;
  a.bias = bias;
  a.routed_scale = rs;
  a.T = (int)T;
  a.D = (int)D;
  a.E = (int)E;
  a.k = (int)k;
  a.idx = idx;
  a.w = w;
  a.logits_out = lo;
  a.ns = batch_slices(D);
  a.ntt = (int)((T + kBatchRows - 1) / kBatchRows);
  a.neb = (int)((E + kBatchExperts - 1) / kBatchExperts);
  a.nwg = a.ntt * a.ns * a.neb;
  a.ncons = (int)std::min<int64_t>((T + kBatchConsTokens - 1) / kBatchConsTokens, a.nwg);
  uint32_t* partial = static_cast<uint32_t*>(scratch);
  a.part = partial + kAmaxPartials;  // 16-byte aligned: the scratch is, and kAmaxPartials words are 4096 bytes
  a.partial = partial;
  // Launch 1: partial maxima (unless the scale is given) and the flag region's zeros.
  const int64_t nvec = gsa_override ? 0 : T * D / 8;
  const int64_t nzero16 = ((int64_t)a.ns * T * E + 3) / 4;
  const int64_t want = (std::max(nvec, nzero16) + kBatchThreads - 1) / kBatchThreads;
  const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(want, kAmaxPartials));
  a.npartial = gsa_override ? 0 : grid;
  batch_amax_zero_kernel<<<grid, kBatchThreads, 0, stream>>>(a.x, nvec, partial, reinterpret_cast<u32x4_t*>(a.part),
                                                              nzero16);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int ep = (int)((E + 63) / 64);
  if (ep <= 1) launch_batch_ep<1>(a, stream);
  else if (ep <= 2) launch_batch_ep<2>(a, stream);
  else if (ep <= 4) launch_batch_ep<4>(a, stream);
  else launch_batch_ep<8>(a, stream);
  return hipGetLastError();
}

}  // namespace nvr
