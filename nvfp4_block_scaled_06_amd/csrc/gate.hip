// Block-scaled NVFP4 gate projection with the routing epilogue fused after it
// (gfx950).
//
// logits[t, e] = gsa * gsw * sum_d (q_x S_x)[t, d] * (q_w S_w)[e, d]: the gate
// GEMM on NVFP4 operands (commit 04cf8ca8, dsv4/layers/router.py, NVFP4 gate
// paragraph), followed by the six-step epilogue (commit e0f60b9f,
// dsv4/kernels/router/__init__.py) while the logits are still on chip or in
// L2, so they never make an HBM round trip unless logits_out asks for them.
//
// Two kernels here, by token count T (T <= 4 takes the decode GEMV in
// gate_decode.hip):
//  * tile (T <= 256): 16x16 output tiles on 16x16x32 f16 MFMAs, the
//    sixteen waves of a workgroup splitting K and summing through LDS; the
//    last workgroup of each 16-row tile routes it.
//  * mfma (larger T): BM tokens x 128 NTW experts per workgroup on 32x32x16
//    f16 MFMAs; the accumulators go through LDS straight into the epilogue.
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
#include "mma_tile.hpp"

#include <stdlib.h>

#include <algorithm>

namespace nvr {


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

// Sixteen wavefronts split a tile's K range, so each has only a few steps,
// and issue the loads of up to four steps before their first MFMA; at the
// end each routes one of the tile's rows. The K partial sums and the router
// scratch share LDS (the partials are dead once the tile's logits are out).
constexpr int kTileWaves = 16;
constexpr int kTileThreads = 64 * kTileWaves;
constexpr int kTileBatch = 4;  // K steps whose loads are in flight together

template <int JMAX>
union TileLds {
  float part[kTileWaves][16][17];
  WaveRouteScratch<JMAX> rsc[kTileWaves];
};

template <int JMAX>
__global__ __launch_bounds__(kTileThreads) void gate_tile_kernel(TileArgs a) {
  __shared__ TileLds<JMAX> u;
  __shared__ float bias_s[512];
  __shared__ uint32_t s_last;
  extern __shared__ float lg[];  // [16][E]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float bias0 = (int)threadIdx.x < a.E ? a.bias[threadIdx.x] : 0.0f;
  const float gsa = load_early(a.gsa), gsw = load_early(a.gsw);
  const int n = lane & 15, g = lane >> 4;
  const int col0 = blockIdx.x * 16, row0 = blockIdx.y * 16;
  const int arow = row0 + n, e = col0 + n;
  const bool a_ok = arow < a.T, b_ok = e < a.E;
  const int s0 = a.nsteps * wave / kTileWaves, s1 = a.nsteps * (wave + 1) / kTileWaves;

  // Chunks past this wavefront's steps or past D load as zeros and add
  // nothing.
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int sb = s0; sb < s1; sb += kTileBatch) {
    Chunk32 ac[kTileBatch], bc[kTileBatch];
#pragma unroll
    for (int u = 0; u < kTileBatch; ++u) {
      const int64_t k0 = (int64_t)(sb + u) * 128 + 32 * g;
      const bool ok = sb + u < s1 && k0 < a.D;
      ac[u] = load_chunk(a.xc, a.xs, arow, a.D, k0, a_ok && ok);
      bc[u] = load_chunk(a.wc, a.ws, e, a.D, k0, b_ok && ok);
    }
#pragma unroll
    for (int u = 0; u < kTileBatch; ++u) {
      const _Float16 sa0 = e4m3_f16(ac[u].s & 0xFFu), sa1 = e4m3_f16(ac[u].s >> 8);
      const _Float16 sb0 = e4m3_f16(bc[u].s & 0xFFu), sb1 = e4m3_f16(bc[u].s >> 8);
      acc = mfma16(fp4x8_to_f16(ac[u].c[0], sa0), fp4x8_to_f16(bc[u].c[0], sb0), acc);
      acc = mfma16(fp4x8_to_f16(ac[u].c[1], sa0), fp4x8_to_f16(bc[u].c[1], sb0), acc);
      acc = mfma16(fp4x8_to_f16(ac[u].c[2], sa1), fp4x8_to_f16(bc[u].c[2], sb1), acc);
      acc = mfma16(fp4x8_to_f16(ac[u].c[3], sa1), fp4x8_to_f16(bc[u].c[3], sb1), acc);
    }
  }
  // 16x16 accumulator layout: lane holds rows 4g..4g+3 of column n. The
  // sixteen partial sums are added as a fixed pairwise tree.
#pragma unroll
  for (int v = 0; v < 4; ++v) u.part[wave][4 * g + v][n] = acc[v];
  __syncthreads();
  if (wave == 0) {
    const float scale = gsa * gsw;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g + v, r = row0 + m;
      float q[kTileWaves];
#pragma unroll
      for (int w = 0; w < kTileWaves; ++w) q[w] = u.part[w][m][n];
#pragma unroll
      for (int h = kTileWaves / 2; h >= 1; h >>= 1)
#pragma unroll
        for (int w = 0; w < h; ++w) q[w] = q[w] + q[w + h];
      const float L = q[0] * scale;
      if (r < a.T && b_ok) {
        store_coherent(a.lbuf + (int64_t)r * a.E + e, L);
        if (a.logits_out) a.logits_out[(int64_t)r * a.E + e] = L;
      }
    }
  }
  if (!arrive_last(&a.counters[blockIdx.y], gridDim.x, &s_last)) return;
  const int nrows = min(16, a.T - row0);
  for (int i = threadIdx.x; i < nrows * a.E; i += kTileThreads)
    lg[i] = load_coherent(a.lbuf + (int64_t)row0 * a.E + i);
  if ((int)threadIdx.x < a.E) bias_s[threadIdx.x] = bias0;
  __syncthreads();
  if (wave < nrows) {  // 16 rows at most: one per wavefront
    const int64_t t = row0 + wave;
    wave_route_row<JMAX>(lg + wave * a.E, bias_s, a.E, a.k, a.routed_scale, a.idx + t * a.k, a.w + t * a.k,
                         u.rsc[wave]);
  }
  release_counter(&a.counters[blockIdx.y]);
}

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
//  * Loads run mma_ring() steps ahead in a register ring.
//  * Epilogue: when the tile holds every expert, scaled accumulators go
//    through LDS, 32 tokens at a time, into the 16-lanes-per-token router.
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
  int nsteps;  // 128-element K steps, rounded up to a multiple of K groups times the ring depth
};

// Epilogue rows per pass: 64 when two K groups share the work and the rows
// fit the LDS, else 32. Each wavefront routes LR / (4 KS) rows per pass, as
// sets of four.
template <int BM, int J16, int KS>
constexpr int epi_rows() { return KS == 2 && BM >= 64 && J16 <= 24 ? 64 : 32; }
template <int BM, int J16, int KS>
constexpr int epi_sets() { return KS == 2 ? epi_rows<BM, J16, KS>() / 32 : 1; }

// LDS row stride of the epilogue's logits, in floats: the router reads 16 J16
// entries per row (16 bytes at a time), and the accumulators of a whole
// expert block (128 NTW columns, zeros past E) are written there, so the row
// holds the wider of the two.
template <int NTW, int J16>
constexpr int epi_ld() { return (16 * J16 > 128 * NTW ? 16 * J16 : 128 * NTW) + 4; }

template <int BM, int NTW, int J16, int KS>
union MmaLds {
  _Float16 abuf[KS][2][BM * kMmaARow];  // K loop: each K group's converted A tiles, double-buffered
  struct {
    float lg[epi_rows<BM, J16, KS>() * epi_ld<NTW, J16>()];       // epilogue: one pass's logits
    Row16Scratch<J16, epi_sets<BM, J16, KS>()> rsc[4 * KS];        // one router scratch per wavefront
  } epi;
};

// KS K groups of four wavefronts: group g takes K steps g, g + KS, ... and
// both groups hold the same output tiles (wavefront w and w + 4 on one
// SIMD), so one group's conversion work overlaps the other's MFMAs; their
// accumulators are added in the epilogue. One wavefront per SIMD otherwise
// (KS = 1), the register file then allowing the widest tiles.
template <int BM, int NTW, int J16, int KS>
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
  mma_mainloop<BM, NTW, KS>(P, a.D, nsteps, &u.abuf[0][0][0], lane, acc);

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
  if (m.ncb > 1) {
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
      for (int i = threadIdx.x; i < 32 * 128 * NTW; i += kMmaThreads * KS) {
        const int mm = i / (128 * NTW), c = i - mm * (128 * NTW), e = col0 + c;
        if (mm < nrows && e < E) {
          const float L = lg[mm * ldE + c];
          store_coherent(a.lbuf + (int64_t)(base + mm) * E + e, L);
          if (a.logits_out) a.logits_out[(int64_t)(base + mm) * E + e] = L;
        }
      }
    };
    static_for<0, BM / 32>(store_pass);
    if (!arrive_last(&a.counters[rb], m.ncb, &s_last)) return;
  }
  // Passes of LR tokens; compile-time row tile indexes keep the accumulator
  // indexes static (a runtime loop over this body would put them in scratch).
  constexpr int LR = epi_rows<BM, J16, KS>(), NSET = epi_sets<BM, J16, KS>();
  auto pass = [&](auto pc) {
    constexpr int p = decltype(pc)::value;
    const int base = row0 + p * LR;
    if (base >= a.T) return;  // uniform
    const int nrows = min(LR, a.T - base);
    __syncthreads();
    if (m.ncb > 1) {
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
      static_for<0, LR / 32>([&](auto ic) {
        constexpr int i = decltype(ic)::value;
        tile_to_lds(IntC<p * (LR / 32) + i>{}, 32 * i);
      });
    }
    __syncthreads();
    // Wavefront w routes rows RW w .. RW w + RW - 1 (RW = LR / 4KS), in calls
    // of NSET interleaved sets of four.
    constexpr int RW = LR / (4 * KS);
#pragma unroll
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
      row16_route<J16, NSET>(Lr, bias_s, E, a.k, a.routed_scale, vr, oi, ow, u.epi.rsc[wave]);
    }
    if (a.logits_out && m.ncb == 1) {
      for (int i = threadIdx.x; i < nrows * E; i += kMmaThreads * KS) {
        const int mm = i / E, e = i - mm * E;
        a.logits_out[(int64_t)(base + mm) * E + e] = lg[mm * ldE + e];
      }
    }
  };
  static_for<0, BM / LR>(pass);
  if (m.ncb > 1) release_counter(&a.counters[rb]);
}

// ---------------------------------------------------------------------------
// Host side: planning and launch.
// ---------------------------------------------------------------------------
static GateTuning read_tuning() {
  GateTuning t;
  if (const char* v = getenv("NVR_SPLIT_MAX_T")) t.split_max_t = atoi(v);
  if (const char* v = getenv("NVR_MMA_BM")) t.mma_bm = atoi(v);
  if (const char* v = getenv("NVR_MMA_NTW")) t.mma_ntw = atoi(v);
  if (t.mma_bm != 32 && t.mma_bm != 64 && t.mma_bm != 128) t.mma_bm = 0;
  if (t.mma_ntw < 1 || t.mma_ntw > 4 || (t.mma_bm / 32) * t.mma_ntw * 16 > 192) t.mma_ntw = 0;
  if (t.split_max_t < 0) t.split_max_t = 0;
  if (t.split_max_t > 16 * kMaxCounters) t.split_max_t = 16 * kMaxCounters;
  return t;
}

const GateTuning& gate_tuning() {
  static const GateTuning t = read_tuning();
  return t;
}

GateKind gate_kind(int64_t T, int64_t D) {
  if (decode_fits(T, D)) return GateKind::kDecode;
  if (T <= gate_tuning().split_max_t) return GateKind::kTile;
  return GateKind::kMma;
}

static hipError_t launch_tile(const TileArgs& a, hipStream_t stream) {
  const dim3 grid((a.E + 15) / 16, (a.T + 15) / 16);
  const size_t lds = (size_t)16 * a.E * sizeof(float);
  const int j = (a.E + 63) / 64;
  if (j <= 1) gate_tile_kernel<1><<<grid, kTileThreads, lds, stream>>>(a);
  else if (j <= 2) gate_tile_kernel<2><<<grid, kTileThreads, lds, stream>>>(a);
  else if (j <= 4) gate_tile_kernel<4><<<grid, kTileThreads, lds, stream>>>(a);
  else if (j <= 6) gate_tile_kernel<6><<<grid, kTileThreads, lds, stream>>>(a);
  else gate_tile_kernel<8><<<grid, kTileThreads, lds, stream>>>(a);
  return hipGetLastError();
}

// Prefill plan: BM tokens x 128 NTW experts per workgroup, NCB expert blocks
// per token block. Among the layouts whose accumulators fit in registers,
// prefer those that give every compute unit a workgroup, then the least
// operand conversion per FLOP, (BM + 128 NTW) / (BM * 128 NTW): every
// workgroup converts its BM x D token tile and its 128 NTW x D weight tile.
struct MmaPlan {
  int bm, ntw, ncb;
};

static MmaPlan plan_mma(int64_t T, int64_t E) {
  const int tiles = (int)((E + 127) / 128);
  const MmaPlan forced = {gate_tuning().mma_bm, gate_tuning().mma_ntw, 0};
  if (forced.bm > 0 && forced.ntw > 0 && forced.ntw <= tiles) {
    const int ncb = (tiles + forced.ntw - 1) / forced.ntw;
    if (ncb == 1 || (T + forced.bm - 1) / forced.bm <= kMaxCounters) return {forced.bm, forced.ntw, ncb};
  }
  MmaPlan best = {32, tiles, 1};
  double best_cost = 1e30;
  int64_t best_wg = 0;
  for (int ntw = 1; ntw <= tiles; ++ntw) {
    if (tiles % ntw) continue;
    const int ncb = tiles / ntw;
    for (int bm : {128, 64, 32}) {
      if ((bm / 32) * ntw * 16 > 192) continue;  // accumulator registers
      const int64_t nrb = (T + bm - 1) / bm;
      if (ncb > 1 && nrb > kMaxCounters) continue;
      const int64_t wg = std::min<int64_t>(nrb * ncb, 256);
      const double cost = (double)(bm + 128 * ntw) / ((double)bm * 128 * ntw);
      if (wg > best_wg || (wg == best_wg && cost < best_cost)) {
        best = {bm, ntw, ncb};
        best_wg = wg;
        best_cost = cost;
      }
    }
  }
  return best;
}

template <int BM, int NTW, int J16>
static hipError_t launch_mma_t(const MmaArgs& m0, hipStream_t stream) {
  constexpr int KS = mma_ksplit<BM, NTW>(), G = KS * mma_ring<BM, NTW>();
  MmaArgs m = m0;
  m.nsteps = (m0.nsteps + G - 1) / G * G;
  gate_mfma_kernel<BM, NTW, J16, KS><<<m.nwg, kMmaThreads * KS, 0, stream>>>(m);
  return hipGetLastError();
}

template <int BM, int NTW>
static hipError_t launch_mma_j(const MmaArgs& m, hipStream_t stream) {
  const int E = m.t.E;
  if (E <= 64) return launch_mma_t<BM, NTW, 4>(m, stream);
  if (E <= 128) return launch_mma_t<BM, NTW, 8>(m, stream);
  if (E <= 256) return launch_mma_t<BM, NTW, 16>(m, stream);
  if (E <= 384) return launch_mma_t<BM, NTW, 24>(m, stream);
  return launch_mma_t<BM, NTW, 32>(m, stream);
}

static hipError_t launch_mma(const TileArgs& a, hipStream_t stream) {
  const MmaPlan p = plan_mma(a.T, a.E);
  MmaArgs m{a, p.ncb, 0, (int)((a.D + 127) / 128)};
  m.nwg = (int)((a.T + p.bm - 1) / p.bm) * p.ncb;
  switch (p.bm * 8 + p.ntw) {
    case 128 * 8 + 1: return launch_mma_j<128, 1>(m, stream);
    case 128 * 8 + 2: return launch_mma_j<128, 2>(m, stream);
    case 128 * 8 + 3: return launch_mma_j<128, 3>(m, stream);
    case 64 * 8 + 1: return launch_mma_j<64, 1>(m, stream);
    case 64 * 8 + 2: return launch_mma_j<64, 2>(m, stream);
    case 64 * 8 + 3: return launch_mma_j<64, 3>(m, stream);
    case 64 * 8 + 4: return launch_mma_j<64, 4>(m, stream);
    case 32 * 8 + 1: return launch_mma_j<32, 1>(m, stream);
    case 32 * 8 + 2: return launch_mma_j<32, 2>(m, stream);
    case 32 * 8 + 3: return launch_mma_j<32, 3>(m, stream);
    default: return launch_mma_j<32, 4>(m, stream);
  }
}

size_t gate_scratch_bytes(int64_t T, int64_t D, int64_t E) {
  switch (gate_kind(T, D)) {
    case GateKind::kDecode: return 0;  // the decode region below kScratchOffset
    case GateKind::kTile: return (size_t)T * (size_t)E * sizeof(float);
    default: return plan_mma(T, E).ncb > 1 ? (size_t)T * (size_t)E * sizeof(float) : 0;
  }
}

hipError_t launch_gate(const uint8_t* xc, const uint8_t* xs, const float* gsa, const uint8_t* wc, const uint8_t* ws,
                       const float* gsw, const float* bias, float rs, int64_t T, int64_t D, int64_t E, int64_t k,
                       int32_t* idx, float* w, float* lo, void* workspace, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const GateKind kind = gate_kind(T, D);
  if (kind == GateKind::kDecode)
    return launch_decode_gate(xc, xs, gsa, wc, ws, gsw, bias, rs, T, D, E, k, idx, w, lo, workspace, stream);
  uint32_t* counters = static_cast<uint32_t*>(workspace);
  float* lbuf = workspace ? reinterpret_cast<float*>(static_cast<char*>(workspace) + kScratchOffset) : nullptr;
  TileArgs a{xc, xs, gsa, wc, ws, gsw, bias, rs, (int)T, (int)D, (int)E, (int)k, idx, w, lo, lbuf, counters,
             (int)((D + 127) / 128)};
  return kind == GateKind::kTile ? launch_tile(a, stream) : launch_mma(a, stream);
}

bool forward_single_launch(int64_t T, int64_t D) { return gate_kind(T, D) == GateKind::kDecode; }

}  // namespace nvr
