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
//  * mfma (larger T, in gate_mfma.hpp): BM tokens x 128 NTW experts per
//    workgroup on 32x32x16 f16 MFMAs; the accumulators go through LDS
//    straight into the epilogue. This file plans it and dispatches to the
//    instantiations in gate_mfma_e*.hip.
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
#include "gate_mfma.hpp"

#include <stdlib.h>

#include <algorithm>

namespace nvr {


// ---------------------------------------------------------------------------
// tile: T up to a few hundred.
// ---------------------------------------------------------------------------

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

static hipError_t launch_mma(const TileArgs& a, hipStream_t stream) {
  const MmaPlan p = plan_mma(a.T, a.E);
  MmaArgs m{a, p.ncb, 0, 0};
  m.nwg = (int)((a.T + p.bm - 1) / p.bm) * p.ncb;
  if (a.E <= 64) return launch_mma_e<4>(m, p.bm, p.ntw, stream);
  if (a.E <= 128) return launch_mma_e<8>(m, p.bm, p.ntw, stream);
  if (a.E <= 256) return launch_mma_e<16>(m, p.bm, p.ntw, stream);
  if (a.E <= 384) return launch_mma_e<24>(m, p.bm, p.ntw, stream);
  return launch_mma_e<32>(m, p.bm, p.ntw, stream);
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
