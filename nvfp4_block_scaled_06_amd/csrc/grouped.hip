// Grouped NVFP4 GEMM (gfx950): the grouped linear layer's product over
// groups of rows (commit df05289d, dsv4/layers/grouped_linear.py).
//
//   Y[r, n] = gsa * gsw[g] * sum_d (q_x S_x)[r, d] * (q_w S_w)[g, n, d]
//
// for every row r of group g, rows offsets[g] .. offsets[g + 1] - 1 of the
// flattened activations. The activations of all groups are one tensor
// quantized by one router_quantize launch (one global scale gsa, on the
// device); each group's weight is its own NVFP4 [N, D] tensor with its own
// global scale gsw[g], kept in the checkpoint's row-major (N, K_packed)
// layout: the MFMA B operand reads K-contiguous rows, so the pages' transpose
// to (K_packed, N) is not needed here. The group offsets are read on the
// device, so the host never learns the group sizes (no host sync); they come
// from grouped_offsets, the element-wise product of a caller-allocated range
// buffer with padded_rows.
//
// Decode-size groups (at most 4 rows each) take a GEMV kernel (below); larger
// groups take workgroup (g, row tile, column tile): BM rows of group g times
// 128 NTW weight rows, on the shared MFMA tile machinery (exact fp16 operands, fp32
// accumulation). Row tiles past a group's end exit at once; rows past it
// inside a tile read zeros through the buffer descriptors and are not
// stored. Epilogue: with two K groups, group 1 leaves its sums in LDS and
// group 0 adds them (a fixed order), scales and stores.
#include "../../include/nvfp4_router.h"
#include "mma_tile.hpp"
#include "router_internal.hpp"

namespace nvr {

struct GroupedArgs {
  const uint8_t* xc;  // [R, D/2]
  const uint8_t* xs;  // [R, D/16]
  const float* gsa;   // [1]
  const uint8_t* wc;  // [G, N, D/2]
  const uint8_t* ws;  // [G, N, D/16]
  const float* gsw;   // [G]
  const int32_t* offsets;  // [G + 1]
  float* out;              // [R, N]
  int G, R, N, D;
  int row_tiles;  // row tiles per group (grid), from the caller's bound on rows per group
  int col_tiles;
  int nsteps;
  int nwg;
};

template <int BM, int NTW, int KS, bool STAGED>
__global__ __launch_bounds__(kMmaThreads * KS) __attribute__((amdgpu_waves_per_eu(KS, KS))) void grouped_mfma_kernel(
    GroupedArgs a) {
  static_assert(KS == mma_ksplit<BM, NTW>(), "K groups as the main loop has them");
  constexpr int BN = 128 * NTW;
  static_assert(KS == 1 || BM * BN * sizeof(float) <= sizeof(_Float16) * KS * 2 * BM * kMmaARow,
                "the epilogue's partial sums fit in the A tiles' LDS");
  __shared__ __attribute__((aligned(16))) _Float16 abuf[KS][2][BM * kMmaARow];
  __shared__ __attribute__((aligned(16))) uint8_t swin[STAGED ? mma_win_bytes<BM, NTW>() : 16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wt = wave & 3, grp = wave >> 2;
  // Workgroup ids go to the 8 XCDs in turn; consecutive tiles (the column
  // tiles of one row tile first) are numbered onto one XCD, so a row tile's
  // activations are fetched into one L2.
  const int nq = a.nwg >> 3, nrm = a.nwg & 7, bx = blockIdx.x & 7;
  const int n = bx * nq + min(bx, nrm) + (blockIdx.x >> 3);
  const int ct = n % a.col_tiles, rest = n / a.col_tiles;
  const int rt = rest % a.row_tiles, g = rest / a.row_tiles;
  // Offsets outside [0, R] or decreasing (a precondition violation) are
  // clamped, so no access leaves the caller's buffers.
  const int r_begin = min(max(a.offsets[g], 0), a.R), r_end = min(max(a.offsets[g + 1], r_begin), a.R);
  const int row0 = r_begin + rt * BM;
  if (row0 >= r_end) return;  // uniform: this group has fewer rows
  const int nr = min(BM, r_end - row0);
  const int col0 = ct * BN, nc = min(BN, a.N - col0);
  const float gsa = load_early(a.gsa), gsw = load_early(a.gsw + g);

  const int64_t rowc = a.D / 2, rows = a.D / 16;
  const int64_t wrow0 = (int64_t)g * a.N + col0;
  const MmaPtrs<BM, NTW> P = mma_ptrs<BM, NTW>(a.xc + row0 * rowc, a.xs + row0 * rows, nr, a.wc + wrow0 * rowc,
                                                 a.ws + wrow0 * rows, nc, a.D, wt, lane);
  constexpr int NS = mma_sets<BM, NTW>();
  f32x16_t acc[NS][BM / 32][NTW];
  mma_mainloop<BM, NTW, KS, STAGED>(P, a.D, a.nsteps, &abuf[0][0][0], swin, lane, acc);

  // 32x32 accumulator layout: value v of lane (r, h) is row 8(v/4) + 4h +
  // v%4, column r of its tile; wavefront wt holds the column tiles wt + 4t.
  const float scale = gsa * gsw;
  const int r = lane & 31, h = lane >> 5;
  float* part = reinterpret_cast<float*>(&abuf[0][0][0]);  // [BM][BN], K group 1's sums
  if (KS == 2 && grp == 1) {
#pragma unroll
    for (int rt2 = 0; rt2 < BM / 32; ++rt2)
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          part[(rt2 * 32 + 8 * (v >> 2) + 4 * h + (v & 3)) * BN + (wt + 4 * t) * 32 + r] = acc[0][rt2][t][v];
  }
  if (KS == 2) __syncthreads();
  if (grp != 0) return;
#pragma unroll
  for (int rt2 = 0; rt2 < BM / 32; ++rt2)
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const int c = (wt + 4 * t) * 32 + r;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rr = rt2 * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        float y = acc[0][rt2][t][v];
        if (KS == 2) y += part[rr * BN + c];
        if (rr < nr && c < nc) a.out[(int64_t)(row0 + rr) * a.N + col0 + c] = y * scale;
      }
    }
}

// Decode-size groups (at most kGvMaxRows rows per group): the layer is a
// stream of the packed expert weights, so it takes the lm_head GEMV's
// shape rather than MFMA tiles (which would multiply mostly zero rows).
// Workgroup (g, column tile) = 64 weight rows of group g, four wavefronts
// of 16 rows with 2 rows' loads in flight (as in the lm_head GEMV; GEMM
// 24.2-24.8 against 25.8-26.1 us with 4, 28.5-30.0 with 1, at G = 8, N =
// 4096, D = 7168); lane l takes the 32-element
// chunks l, l + 64, ... of a row (coalesced 1 KB per wavefront load,
// nontemporal: every weight byte is read once). The group's rows of x are
// converted once per workgroup into LDS as exact fp16 q S values; block
// products are exact in fp32, per-lane sums and the wavefront sum run in a
// fixed order, and the result is scaled by gsa * gsw[g] as in the tile path.
constexpr int kGvWaves = 4;
constexpr int kGvThreads = 64 * kGvWaves;
constexpr int kGvRowsPerWave = 16;
constexpr int kGvCols = kGvWaves * kGvRowsPerWave;  // weight rows (output columns) per workgroup
constexpr int kGvInFlight = 2;
constexpr int kGvMaxRows = 4;
constexpr int kGvMaxXHalves = 32768;  // rows x D of the fp16 x copy in LDS (64 KB)

template <int CPL>
__global__ __launch_bounds__(kGvThreads) void grouped_gemv_kernel(GroupedArgs a, int max_rows) {
  extern __shared__ half8_t xg[];  // [nr][D / 8]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nct = (a.N + kGvCols - 1) / kGvCols;
  const int g = blockIdx.x / nct, ct = blockIdx.x - g * nct;
  // Offsets outside [0, R] or decreasing are clamped, as in the tile path.
  const int r_begin = min(max(a.offsets[g], 0), a.R), r_end = min(max(a.offsets[g + 1], r_begin), a.R);
  const int nr = min(r_end - r_begin, max_rows);
  if (nr <= 0) return;  // uniform
  const int nch = a.D >> 5;
  const int64_t rowc = a.D / 2, rows = a.D / 16;
  const float gsa = load_early(a.gsa), gsw = load_early(a.gsw + g);

  for (int i = threadIdx.x; i < nr * nch; i += kGvThreads) {
    const int t = i / nch, c = i - t * nch;
    const int64_t r = r_begin + t;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(a.xc + r * rowc + 16 * c);
    const uint32_t sb = *reinterpret_cast<const uint16_t*>(a.xs + r * rows + 2 * c);
    const _Float16 s0 = e4m3_f16(sb & 0xFFu), s1 = e4m3_f16(sb >> 8);
    half8_t* d = xg + (int64_t)t * (nch * 4) + 4 * c;
    d[0] = fp4x8_to_f16(v[0], s0);
    d[1] = fp4x8_to_f16(v[1], s0);
    d[2] = fp4x8_to_f16(v[2], s1);
    d[3] = fp4x8_to_f16(v[3], s1);
  }
  __syncthreads();

  const float scale = gsa * gsw;
  const int col_base = ct * kGvCols + wave * kGvRowsPerWave;
  // Raw buffer loads over this workgroup's weight rows of group g (32-bit
  // ranges and offsets then hold for any N): a row past N reads zeros, and a
  // chunk past D gets an offset past the range (zeros, no branch), so the
  // loads are unconditional and complete in issue order.
  const int64_t wg_row0 = (int64_t)g * a.N + (int64_t)ct * kGvCols;
  const int64_t wg_rows = min((int64_t)kGvCols, (int64_t)a.N - (int64_t)ct * kGvCols);
  const __amdgpu_buffer_rsrc_t wcr = make_rsrc(a.wc + wg_row0 * rowc, wg_rows * rowc);
  const __amdgpu_buffer_rsrc_t wsr = make_rsrc(a.ws + wg_row0 * rows, wg_rows * rows);
  uint32_t oc[CPL], os[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    oc[i] = c < nch ? (uint32_t)(16 * c) : kMmaOob;
    os[i] = c < nch ? (uint32_t)(2 * c) : kMmaOob;
  }
  u32x4_t wv[kGvInFlight][CPL];
  uint32_t wsv[kGvInFlight][CPL];
  auto load_row = [&](int slot, int u) {
    const int lr = wave * kGvRowsPerWave + u;  // weight row within the workgroup
    const uint32_t rc = (uint32_t)lr * (uint32_t)rowc, rs = (uint32_t)lr * (uint32_t)rows;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      wv[slot][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wcr, oc[i] + rc, 0, kNtAux));
      wsv[slot][i] = __builtin_amdgcn_raw_buffer_load_b16(wsr, os[i] + rs, 0, kNtAux);
    }
  };
  // A ring of kGvInFlight rows: row u + kGvInFlight is loaded into row u's
  // registers as soon as row u is summed, so that many rows stay in flight
  // throughout (loads complete in order: summing row u waits for its own).
#pragma unroll
  for (int u = 0; u < kGvInFlight; ++u) load_row(u, u);
#pragma unroll
  for (int u = 0; u < kGvRowsPerWave; ++u) {
    const int slot = u % kGvInFlight, n = col_base + u;
    float acc[kGvMaxRows];
#pragma unroll
    for (int t = 0; t < kGvMaxRows; ++t) acc[t] = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = min(lane + 64 * i, nch - 1);  // chunks past D hold zero weights
      const _Float16 s0 = e4m3_f16(wsv[slot][i] & 0xFFu), s1 = e4m3_f16(wsv[slot][i] >> 8);
      const half8_t w0 = fp4x8_to_f16(wv[slot][i][0], s0), w1 = fp4x8_to_f16(wv[slot][i][1], s0);
      const half8_t w2 = fp4x8_to_f16(wv[slot][i][2], s1), w3 = fp4x8_to_f16(wv[slot][i][3], s1);
#pragma unroll
      for (int t = 0; t < kGvMaxRows; ++t) {
        if (t < nr) {
          const half8_t* xp = xg + (int64_t)t * (nch * 4) + 4 * c;
          acc[t] += dot8(xp[1], w1, dot8(xp[0], w0, 0.0f));
          acc[t] += dot8(xp[3], w3, dot8(xp[2], w2, 0.0f));
        }
      }
    }
    if (u + kGvInFlight < kGvRowsPerWave) load_row(slot, u + kGvInFlight);
#pragma unroll
    for (int t = 0; t < kGvMaxRows; ++t) {
      if (t < nr) {
        const float y = wave_sum(acc[t]) * scale;
        if (lane == 0 && n < a.N) a.out[(int64_t)(r_begin + t) * a.N + n] = y;
      }
    }
  }
}

__global__ void grouped_offsets_kernel(const int32_t* __restrict__ range, int n, int32_t padded_rows,
                                       int32_t* __restrict__ offsets) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    offsets[i] = range[i] * padded_rows;
}

struct GroupedPlan {
  int bm, ntw;
};

// Rows per group up to 32 or 64: one row tile of that height, 128 columns
// per workgroup (two K groups) so that a decode-size call still spreads the
// weight stream over many workgroups. Larger groups: 128-row tiles and the
// widest column tile that still gives every compute unit a workgroup.
static GroupedPlan plan_grouped(int64_t G, int64_t max_rows, int64_t N) {
  if (max_rows <= 32) return {32, 1};
  if (max_rows <= 64) return {64, 1};
  const int64_t rtiles = G * ((max_rows + 127) / 128);
  for (int ntw = 3; ntw > 1; --ntw)
    if (rtiles * ((N + 128 * ntw - 1) / (128 * ntw)) >= 256) return {128, ntw};
  return {128, 1};
}

static bool gemv_fits(int64_t max_rows, int64_t D) {
  return max_rows <= kGvMaxRows && max_rows * D <= kGvMaxXHalves && D <= 16384;
}

template <int CPL>
static hipError_t launch_gemv_t(const GroupedArgs& a, int max_rows, int nwg, hipStream_t stream) {
  const size_t lds = (size_t)max_rows * (size_t)a.D * sizeof(_Float16);
  grouped_gemv_kernel<CPL><<<nwg, kGvThreads, lds, stream>>>(a, max_rows);
  return hipGetLastError();
}

static hipError_t launch_gemv(const GroupedArgs& a, int max_rows, int nwg, hipStream_t stream) {
  const int cpl = ((a.D >> 5) + 63) / 64;  // 32-element chunks per lane, D <= 16384
  switch (cpl) {
    case 1: return launch_gemv_t<1>(a, max_rows, nwg, stream);
    case 2: return launch_gemv_t<2>(a, max_rows, nwg, stream);
    case 3: return launch_gemv_t<3>(a, max_rows, nwg, stream);
    case 4: return launch_gemv_t<4>(a, max_rows, nwg, stream);
    case 5: return launch_gemv_t<5>(a, max_rows, nwg, stream);
    case 6: return launch_gemv_t<6>(a, max_rows, nwg, stream);
    case 7: return launch_gemv_t<7>(a, max_rows, nwg, stream);
    default: return launch_gemv_t<8>(a, max_rows, nwg, stream);
  }
}

}  // namespace nvr

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

template <int BM, int NTW>
hipError_t launch_grouped(nvr::GroupedArgs a, int64_t max_rows, hipStream_t stream) {
  a.row_tiles = (int)((max_rows + BM - 1) / BM);
  a.col_tiles = (a.N + 128 * NTW - 1) / (128 * NTW);
  a.nsteps = nvr::mma_padded_steps<BM, NTW>(a.D);
  a.nwg = a.G * a.row_tiles * a.col_tiles;
  constexpr int KS = nvr::mma_ksplit<BM, NTW>();
  // Scale windows take 16-byte loads: rows of D / 16 scale bytes must keep
  // them aligned.
  if (a.D % 256 == 0) nvr::grouped_mfma_kernel<BM, NTW, KS, true><<<a.nwg, nvr::kMmaThreads * KS, 0, stream>>>(a);
  else nvr::grouped_mfma_kernel<BM, NTW, KS, false><<<a.nwg, nvr::kMmaThreads * KS, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

extern "C" {

int grouped_offsets(const int32_t* range, int64_t G, int64_t padded_rows, int32_t* offsets, void* stream) {
  if (G < 1 || G > (int64_t(1) << 24) || padded_rows < 0 || G * padded_rows >= (int64_t(1) << 31)) return ROUTER_EINVAL;
  if (!range || !offsets || !aligned(range, 4) || !aligned(offsets, 4)) return ROUTER_EINVAL;
  const int n = (int)(G + 1);
  nvr::grouped_offsets_kernel<<<(n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024, 256, 0,
                                static_cast<hipStream_t>(stream)>>>(range, n, (int32_t)padded_rows, offsets);
  return hipGetLastError() == hipSuccess ? ROUTER_OK : ROUTER_EHIP;
}

int grouped_gemm(const uint8_t* x_codes, const uint8_t* x_scales, const float* gsa, const uint8_t* w_codes,
                 const uint8_t* w_scales, const float* gsw, const int32_t* offsets, int64_t G, int64_t R,
                 int64_t max_rows, int64_t N, int64_t D, float* out, void* stream) {
  if (G < 1 || G > (int64_t(1) << 24) || R < 0 || R >= (int64_t(1) << 31) || max_rows < 0 || N < 1 ||
      N >= (int64_t(1) << 31) || D < 16 || D % 16 != 0)
    return ROUTER_EINVAL;
  if (D % 32 != 0 || D > ROUTER_MAX_GATE_D) return ROUTER_EUNSUPPORTED;
  if (!gsa || !w_codes || !w_scales || !gsw || !offsets) return ROUTER_EINVAL;
  if (R > 0 && (!x_codes || !x_scales || !out)) return ROUTER_EINVAL;
  if (!aligned(x_codes, 16) || !aligned(w_codes, 16) || !aligned(x_scales, 2) || !aligned(w_scales, 2) ||
      !aligned(gsa, 4) || !aligned(gsw, 4) || !aligned(offsets, 4) || !aligned(out, 4))
    return ROUTER_EINVAL;
  if (G * N * (D / 2) >= (int64_t(1) << 62)) return ROUTER_EINVAL;
  const nvr::GroupedPlan p = nvr::plan_grouped(G, max_rows, N);
  const int64_t row_tiles = (max_rows + p.bm - 1) / p.bm, col_tiles = (N + 128 * p.ntw - 1) / (128 * p.ntw);
  if (G * row_tiles * col_tiles >= (int64_t(1) << 31)) return ROUTER_EUNSUPPORTED;
  if (R == 0 || max_rows == 0) return ROUTER_OK;
  nvr::GroupedArgs a{x_codes, x_scales, gsa, w_codes, w_scales, gsw, offsets, out, (int)G, (int)R, (int)N, (int)D,
                     0, 0, 0, 0};
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (nvr::gemv_fits(max_rows, D)) {
    const int64_t nwg = G * ((N + nvr::kGvCols - 1) / nvr::kGvCols);
    if (nwg >= (int64_t(1) << 31)) return ROUTER_EUNSUPPORTED;
    e = nvr::launch_gemv(a, (int)max_rows, (int)nwg, s);
    return e == hipSuccess ? ROUTER_OK : ROUTER_EHIP;
  }
  switch (p.bm * 8 + p.ntw) {
    case 32 * 8 + 1: e = launch_grouped<32, 1>(a, max_rows, s); break;
    case 64 * 8 + 1: e = launch_grouped<64, 1>(a, max_rows, s); break;
    case 128 * 8 + 2: e = launch_grouped<128, 2>(a, max_rows, s); break;
    case 128 * 8 + 3: e = launch_grouped<128, 3>(a, max_rows, s); break;
    default: e = launch_grouped<128, 1>(a, max_rows, s); break;
  }
  return e == hipSuccess ? ROUTER_OK : ROUTER_EHIP;
}

}  // extern "C"
