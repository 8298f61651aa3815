// Prefill gate on MFMA tiles (gfx950), shared by the translation units that
// instantiate it, one per bucket of expert counts (gate_mfma_e*.hip), so the
// many tile shapes compile in parallel.
#pragma once

#include "mma_tile.hpp"
#include "route16.hpp"

namespace nvr {

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

// ---------------------------------------------------------------------------
// mfma (prefill, T > 256): workgroup tile BM tokens x 128 NTW experts, four
// wavefronts; wavefront w owns the 32-expert tiles w, w + 4, ... of the
// tile's expert block. K advances 128 elements per step.
//  * A (tokens): each step's BM x 128 tile is converted once per workgroup
//    (32 elements per thread and row) into an LDS tile of fp16 q S values,
//    double-buffered, which every wavefront reads with ds_read_b128.
//  * B (gate weights): each lane loads two 32-element chunks of its expert
//    row per step (16 code bytes + 2 scale bytes each) and converts them in
//    registers; no other wavefront needs them.
//  * K permutation: lane (r, h) of a 32x32x16 MFMA supplies 8 K values of
//    row/column r from group h; in step-relative K, MFMA j (0..7) takes
//    [32h + 8j, +8) for j < 4 and [64 + 32h + 8(j - 4), +8) for j >= 4, on A
//    and on B alike, so every product meets its partner and each K value is
//    used once.
//  * Loads run mma_ring() steps ahead in a register ring; both operands of a
//    step are converted during the step before it, between its MFMAs.
//  * Epilogue: when the tile holds every expert, scaled accumulators go
//    through LDS, 32 or 64 tokens at a time, into the 16-lanes-per-token
//    router.
//    When E is split over NCB workgroups, each stores its logits to the
//    workspace (device-coherent) and the last of the token block's NCB
//    workgroups to arrive loads them all and routes the block.
// Workgroups are numbered so that the NCB expert blocks of a token block run
// on one XCD (x fetched from HBM once, shared in its L2).
// ---------------------------------------------------------------------------
struct MmaArgs {
  TileArgs t;
  int ncb;     // expert blocks (workgroups per token block)
  int nwg;     // workgroups
  int nsteps;  // 128-element K steps, rounded up to whole scale windows
};

// Epilogue rows per pass: 64 when the tile has them and their logits rows
// fit the LDS (up to 384 experts), else 32 (fewer passes: measured 2-3 %
// of the large-prefill gate with one K group). Each wavefront routes
// LR / (4 KS) rows per pass, as sets of four. One K group: two sets per
// call (interleaved, for latency hiding: with one wavefront per SIMD this
// was worth ~6 % of the large-prefill gate). Two K groups: one set per call,
// the SIMD's other wavefront hiding the latency (the prefill gate at
// T = 8192, E = 256: 47.2-47.8 -> 46.2-46.9 us against two sets, same run,
// bit-identical outputs).
template <int BM, int J16, int KS>
constexpr int epi_rows() { return BM >= 64 && J16 <= 24 ? 64 : 32; }
template <int BM, int J16, int KS>
constexpr int epi_sets() { return KS == 2 ? 1 : 2; }

// LDS row stride of the epilogue's logits, in floats: the router reads 16 J16
// entries per row (16 bytes at a time), and the accumulators of a whole
// expert block (128 NTW columns, zeros past E) are written there, so the row
// holds the wider of the two.
template <int NTW, int J16>
constexpr int epi_ld() { return (16 * J16 > 128 * NTW ? 16 * J16 : 128 * NTW) + 4; }

template <int BM, int NTW, int J16, int KS>
union MmaLds {
  struct {
    _Float16 abuf[KS][2][BM * kMmaARow];   // each K group's converted A tiles, double-buffered
    uint8_t swin[mma_win_bytes<BM, NTW>()];  // two scale windows
  } k;                                       // K loop
  struct {
    float lg[epi_rows<BM, J16, KS>() * epi_ld<NTW, J16>()];       // epilogue: one pass's logits
    Row16Scratch<J16, epi_sets<BM, J16, KS>()> rsc[4 * KS];        // one router scratch per wavefront
  } epi;
};

// Routing epilogue of a BM-token workgroup tile run by kMmaThreads * KS
// threads: fill(IntC<rt>{}, lr0) leaves row tile rt's scaled logits in lg
// rows lr0 .. lr0 + 31 (columns local to the workgroup's expert block, zeros
// past E). With split experts (ncb > 1) each workgroup stores its block's
// logits to the workspace (device-coherent) and the last of the token
// block's ncb workgroups to arrive loads them all and routes the block;
// otherwise the tile is routed straight from LDS, LR tokens per pass.
template <int BM, int NTW, int J16, int KS, class Fill>
__device__ __forceinline__ void route_tile(const TileArgs& a, int ncb, int rb, int row0, int col0, float* lg,
                                           Row16Scratch<J16, epi_sets<BM, J16, KS>()>* rsc, const float* bias_s,
                                           uint32_t* s_last, Fill&& tile_to_lds) {
  constexpr int ldE = epi_ld<NTW, J16>();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int E = a.E;
  if (ncb > 1) {
    // Split experts: this block's logits to the workspace, then the last
    // block of the token block routes it.
    auto store_pass = [&](auto rtc) {
      constexpr int rt = decltype(rtc)::value;
      const int base = row0 + rt * 32;
      if (base >= a.T) return;  // uniform
      __syncthreads();
      tile_to_lds(rtc, 0);
      __syncthreads();
      const int nrows = min(32, a.T - base);
      // Every LDS read of the pass first, then the stores: one element per
      // loop trip waited for each read in turn.
      constexpr int PER = 32 * 128 * NTW / (kMmaThreads * KS);  // elements per thread
      static_assert(32 * 128 * NTW % (kMmaThreads * KS) == 0, "whole elements per thread");
      float L[PER];
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int i = threadIdx.x + u * kMmaThreads * KS, mm = i / (128 * NTW), c = i - mm * (128 * NTW);
        L[u] = lg[mm * ldE + c];
      }
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int i = threadIdx.x + u * kMmaThreads * KS, mm = i / (128 * NTW), c = i - mm * (128 * NTW);
        const int e = col0 + c;
        if (mm < nrows && e < E) {
          store_coherent(a.lbuf + (int64_t)(base + mm) * E + e, L[u]);
          if (a.logits_out) a.logits_out[(int64_t)(base + mm) * E + e] = L[u];
        }
      }
    };
    static_for<0, BM / 32>(store_pass);
    if (!arrive_last(&a.counters[rb], ncb, s_last)) return;
  }
  // Passes of LR tokens, as a runtime loop so that the routing code exists
  // once: unrolled per pass and per call it made the largest kernels several
  // times the instruction cache, and their routing ran from misses. Filling
  // a pass from the accumulators takes compile-time row tile indexes (runtime
  // ones would put them in scratch), so each pass's fill has its own branch.
  constexpr int LR = epi_rows<BM, J16, KS>(), NSET = epi_sets<BM, J16, KS>();
#pragma unroll 1
  for (int p = 0; p < BM / LR; ++p) {
    const int base = row0 + p * LR;
    if (base >= a.T) break;  // uniform
    const int nrows = min(LR, a.T - base);
    __syncthreads();
    if (ncb > 1) {
      // Gather the token block's logits from every expert block: wavefront w
      // takes rows w, w + 4KS, ...; lane l columns l, l + 64, ...; all loads
      // are issued before the first store. Rows past T and experts past E
      // read a clamped (valid) address; the router masks both.
      constexpr int RR = LR / (4 * KS);
      const float* src = a.lbuf + (int64_t)base * E;
      float v[RR][J16 / 4];
#pragma unroll
      for (int rr = 0; rr < RR; ++rr)
#pragma unroll
        for (int cc = 0; cc < J16 / 4; ++cc) {
          const int mm = min(wave + 4 * KS * rr, nrows - 1), e = min(lane + 64 * cc, E - 1);
          v[rr][cc] = load_coherent(src + mm * E + e);
        }
#pragma unroll
      for (int rr = 0; rr < RR; ++rr)
#pragma unroll
        for (int cc = 0; cc < J16 / 4; ++cc) lg[(wave + 4 * KS * rr) * ldE + lane + 64 * cc] = v[rr][cc];
    } else {
      static_for<0, BM / LR>([&](auto pc) {
        constexpr int pp = decltype(pc)::value;
        if (p == pp)
          static_for<0, LR / 32>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            tile_to_lds(IntC<pp * (LR / 32) + i>{}, 32 * i);
          });
      });
    }
    __syncthreads();
    // Wavefront w routes rows RW w .. RW w + RW - 1 (RW = LR / 4KS), in calls
    // of NSET interleaved sets of four.
    constexpr int RW = LR / (4 * KS);
#pragma unroll 1
    for (int c0 = 0; c0 < RW / 4; c0 += NSET) {
      const float* Lr[NSET];
      bool vr[NSET];
      int32_t* oi[NSET];
      float* ow[NSET];
#pragma unroll
      for (int q = 0; q < NSET; ++q) {
        const int mm = wave * RW + 4 * (c0 + q) + (lane >> 4);
        const int64_t t = base + mm;
        Lr[q] = lg + mm * ldE;
        vr[q] = t < a.T;
        oi[q] = a.idx + t * a.k;
        ow[q] = a.w + t * a.k;
      }
      row16_route<J16, NSET>(Lr, bias_s, E, a.k, a.routed_scale, vr, oi, ow, rsc[wave]);
    }
    if (a.logits_out && ncb == 1) {
      for (int i = threadIdx.x; i < nrows * E; i += kMmaThreads * KS) {
        const int mm = i / E, e = i - mm * E;
        a.logits_out[(int64_t)(base + mm) * E + e] = lg[mm * ldE + e];
      }
    }
  }
  if (ncb > 1) release_counter(&a.counters[rb]);
}

// KS K groups of four wavefronts: group g takes K steps g, g + KS, ... and
// both groups hold the same output tiles (wavefront w and w + 4 on one
// SIMD), so one group's conversion work overlaps the other's MFMAs; their
// accumulators are added in the epilogue. One wavefront per SIMD otherwise
// (KS = 1), the register file then allowing the widest tiles.
template <int BM, int NTW, int J16, int KS, bool STAGED>
__global__ __launch_bounds__(kMmaThreads * KS) __attribute__((amdgpu_waves_per_eu(KS, KS))) void gate_mfma_kernel(
    MmaArgs m) {
  constexpr int ldE = epi_ld<NTW, J16>();
  static_assert(sizeof(MmaLds<BM, NTW, J16, KS>) + 512 * sizeof(float) + 16 <= 160 * 1024,
                "LDS of one workgroup must fit a compute unit");
  const TileArgs& a = m.t;
  __shared__ __attribute__((aligned(16))) MmaLds<BM, NTW, J16, KS> u;
  __shared__ __attribute__((aligned(16))) float bias_s[512];
  __shared__ uint32_t s_last;
  float* lg = u.epi.lg;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wt = wave & 3, grp = wave >> 2;
  const int E = a.E;
  // Token block / expert block of this workgroup (XCD-grouped numbering).
  const int nq = m.nwg >> 3, nr = m.nwg & 7, bx = blockIdx.x & 7;
  const int n = bx * nq + min(bx, nr) + (blockIdx.x >> 3);
  const int rb = n / m.ncb, cb = n - rb * m.ncb;
  const int row0 = rb * BM, col0 = cb * 128 * NTW;
  const int nsteps = m.nsteps;
  const float bias0 = (int)threadIdx.x < E ? a.bias[threadIdx.x] : 0.0f;
  const float bias1 = KS == 1 && (int)threadIdx.x + 256 < E ? a.bias[threadIdx.x + 256] : 0.0f;
  const float gsa = load_early(a.gsa), gsw = load_early(a.gsw);

  constexpr int NS = mma_sets<BM, NTW>();
  f32x16_t acc[NS][BM / 32][NTW];
  const int64_t rowc = a.D / 2, rows = a.D / 16;
  const MmaPtrs<BM, NTW> P = mma_ptrs<BM, NTW>(
      a.xc + row0 * rowc, a.xs + row0 * rows, min((int64_t)BM, (int64_t)a.T - row0), a.wc + col0 * rowc,
      a.ws + col0 * rows, min((int64_t)128 * NTW, (int64_t)a.E - col0), a.D, wt, lane);
  mma_mainloop<BM, NTW, KS, STAGED>(P, a.D, nsteps, &u.k.abuf[0][0][0], u.k.swin, lane, acc);

  // Epilogue. 32x32 accumulator layout: value v of lane (r, h) is row
  // 8(v/4) + 4h + v%4, column r of its tile. With two K groups, group 1
  // leaves its sums in LDS and group 0 adds them (a fixed order).
  const float scale = gsa * gsw;
  const int r = lane & 31, h = lane >> 5;
  if ((int)threadIdx.x < E) bias_s[threadIdx.x] = bias0;
  if (KS == 1 && (int)threadIdx.x + 256 < E) bias_s[threadIdx.x + 256] = bias1;
  // This K group's scaled sums of row tile rt into lg rows lr0 .. lr0 + 31
  // (group 1 first, then group 0 adds); columns are local to the workgroup's
  // expert block under split experts, else expert indexes (the same when
  // there is one expert block).
  auto tile_to_lds = [&](auto rtc, int lr0) {
    constexpr int rt = decltype(rtc)::value;
    float* out = lg + lr0 * ldE;
    if (KS == 2 && grp == 1) {
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const int c = (wt + 4 * t) * 32 + r;
#pragma unroll
        for (int v = 0; v < 16; ++v) out[(8 * (v >> 2) + 4 * h + (v & 3)) * ldE + c] = acc[0][rt][t][v];
      }
    }
    if (KS == 2) __syncthreads();
    if (grp == 0) {
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        const int c = (wt + 4 * t) * 32 + r;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float* d = &out[(8 * (v >> 2) + 4 * h + (v & 3)) * ldE + c];
          *d = (KS == 2 ? acc[0][rt][t][v] + *d : acc[0][rt][t][v]) * scale;
        }
      }
    }
  };
  route_tile<BM, NTW, J16, KS>(a, m.ncb, rb, row0, col0, lg, u.epi.rsc, bias_s, &s_last, tile_to_lds);
}

// Launch of the prefill gate with BM tokens x 128 NTW experts per workgroup
// (a plan of plan_mma()), for E <= 16 J16 experts; m.nsteps is set here.
template <int BM, int NTW, int J16>
static hipError_t launch_mma_t(const MmaArgs& m0, hipStream_t stream) {
  constexpr int KS = mma_ksplit<BM, NTW>();
  MmaArgs m = m0;
  m.nsteps = mma_padded_steps<BM, NTW>(m0.t.D);
  // Scale windows take 16-byte loads: rows of D / 16 scale bytes must keep
  // them aligned.
  if (m.t.D % 256 == 0) gate_mfma_kernel<BM, NTW, J16, KS, true><<<m.nwg, kMmaThreads * KS, 0, stream>>>(m);
  else gate_mfma_kernel<BM, NTW, J16, KS, false><<<m.nwg, kMmaThreads * KS, 0, stream>>>(m);
  return hipGetLastError();
}

template <int J16>
hipError_t launch_mma_e(const MmaArgs& m, int bm, int ntw, hipStream_t stream) {
  switch (bm * 8 + ntw) {
    case 128 * 8 + 1: return launch_mma_t<128, 1, J16>(m, stream);
    case 128 * 8 + 2: return launch_mma_t<128, 2, J16>(m, stream);
    case 128 * 8 + 3: return launch_mma_t<128, 3, J16>(m, stream);
    case 64 * 8 + 1: return launch_mma_t<64, 1, J16>(m, stream);
    case 64 * 8 + 2: return launch_mma_t<64, 2, J16>(m, stream);
    case 64 * 8 + 3: return launch_mma_t<64, 3, J16>(m, stream);
    case 64 * 8 + 4: return launch_mma_t<64, 4, J16>(m, stream);
    case 32 * 8 + 1: return launch_mma_t<32, 1, J16>(m, stream);
    case 32 * 8 + 2: return launch_mma_t<32, 2, J16>(m, stream);
    case 32 * 8 + 3: return launch_mma_t<32, 3, J16>(m, stream);
    default: return launch_mma_t<32, 4, J16>(m, stream);
  }
}

extern template hipError_t launch_mma_e<4>(const MmaArgs&, int, int, hipStream_t);
extern template hipError_t launch_mma_e<8>(const MmaArgs&, int, int, hipStream_t);
extern template hipError_t launch_mma_e<16>(const MmaArgs&, int, int, hipStream_t);
extern template hipError_t launch_mma_e<24>(const MmaArgs&, int, int, hipStream_t);
extern template hipError_t launch_mma_e<32>(const MmaArgs&, int, int, hipStream_t);

}  // namespace nvr
