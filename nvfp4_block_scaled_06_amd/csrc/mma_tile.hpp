// MFMA tile machinery shared by the prefill gate and the grouped GEMM
// (gfx950): a workgroup computes a BM x 128 NTW tile of products of two
// NVFP4 operands (rows of [rows, D/2] codes and [rows, D/16] E4M3 scales),
// both converted to exact fp16 q S values, on 32x32x16 f16 MFMAs.
//
//  * Tiles: four wavefronts per K group; wavefront w owns the 32-column
//    tiles w, w + 4, ... and all BM rows. K advances 128 elements per step.
//  * A (rows): each step's BM x 128 tile is converted once per workgroup
//    (32 elements per thread and row) into an LDS tile of fp16 q S values,
//    double-buffered, which every wavefront reads with ds_read_b128.
//  * B (columns): each lane loads two 32-element chunks of its column row
//    per step (16 code bytes + 2 scale bytes each) and converts them in
//    registers; no other wavefront needs them.
//  * Both operands of a step are converted during the step before it,
//    spread evenly between that step's MFMAs (mma_step).
//  * K permutation: lane (r, h) of a 32x32x16 MFMA supplies 8 K values of
//    row/column r from group h; in step-relative K, MFMA j (0..7) takes
//    [32h + 8j, +8) for j < 4 and [64 + 32h + 8(j - 4), +8) for j >= 4, on A
//    and on B alike, so every product meets its partner and each K value is
//    used once. Every product is exact (at most 6 significant bits per
//    operand), so only the fp32 accumulation rounds.
//  * Loads are raw buffer loads whose descriptors cover only the tile's
//    rows, so rows past the end and chunks past D read zeros without a
//    branch; they run mma_ring() steps ahead in a register ring.
//  * Scales (STAGED, D a multiple of 256): the E4M3 bytes of kMmaWin
//    consecutive K steps of every A and B row of the tile are loaded ahead
//    by the whole workgroup, 16 bytes per lane and four lanes per row, into
//    one of two LDS windows; each step reads its scale bytes there. A vector
//    load costs the address unit about one pass per cache line it touches,
//    whatever its width, so a per-step load of two scale bytes per lane
//    cost as much as a 16-byte code load (measured on gfx950: ~56 cycles per
//    compute unit for 16 rows, for 2 bytes or 16 per lane). Otherwise each
//    step loads its scale bytes with its codes.
#pragma once

#include "gate_common.hpp"

namespace nvr {

constexpr int kMmaThreads = 256;

// K steps of loads in flight: four for the small tiles, two when the
// accumulators and weight fragments of a wide tile already need most
// registers (32 x 256 tiles too: two wavefronts per SIMD share the
// registers, and the weight units stay live from one step to the next).
template <int BM, int NTW>
constexpr int mma_ring() {
  return (BM / 32) * NTW >= 6 || (BM == 32 && NTW == 2) ? 2 : 4;
}
constexpr int kMmaARow = 136;  // LDS row stride of the A tile in halves (128 values + 8 pad)


// Eight E2M1 codes times the block scale s, as fp16 (exact), like
// fp4x8_to_f16 but with its instructions in a fixed order: the four converts
// are all issued before the first multiply: left to itself the compiler
// alternates them through one temporary register, a chain in which every
// instruction waits for the one before it (one wavefront per SIMD has no
// other wavefront to fill those cycles).
__device__ __forceinline__ half8_t fp4x8_scaled(uint32_t c, _Float16 s) {
  const half2_t ss = {s, s};
  half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 0);
  half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 1);
  half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 2);
  half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 3);
  asm volatile("" : "+v"(h0), "+v"(h1), "+v"(h2), "+v"(h3));
  h0 *= ss;
  h1 *= ss;
  h2 *= ss;
  h3 *= ss;
  return half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// The two E4M3 scale bytes in the low half of w as f16 values (exact: every
// E4M3 value is an f16 value; the bytes 0x7F and 0xFF decode to NaN, as the
// format defines them).
__device__ __forceinline__ half2_t e4m3x2_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}

__device__ __forceinline__ half8_t fp4x8_scaled(uint32_t c, half2_t s2, int sel) {
  return fp4x8_scaled(c, sel ? s2[1] : s2[0]);
}

// Token rows per thread in the A tile (4 threads per row): one slot per 64
// rows; with BM = 32 only threads 0..127 have a row.
template <int BM>
constexpr int mma_row_slots() {
  return BM >= 64 ? BM / 64 : 1;
}

template <int BM, int NTW>
struct MmaRegs {
  u32x4_t a[mma_row_slots<BM>()];  // A: this thread's 32-element chunk of rows tid/4 (+ 64 i)
  uint32_t as[mma_row_slots<BM>()];
  u32x4_t b[NTW][2];   // B: this lane's two chunks per expert tile
  uint32_t bs[NTW][2];
};

// Operand reads are raw buffer loads: each workgroup's descriptors cover
// only its token rows and its expert rows, and a read past a descriptor's
// end returns zeros. Rows past T or E and chunks past D (given an
// out-of-range offset) therefore load zeros without a branch, so the wait
// counters of the load ring stay exact. Offsets are per lane; a step adds 64
// code bytes and 8 scale bytes.
constexpr uint32_t kMmaOob = 0x80000000u;  // beyond every descriptor's range
constexpr int kNtAux = 2;                  // raw buffer load cache policy: nontemporal (streaming)
constexpr int kBufferWord3 = 0x00020000;   // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}

template <int BM, int NTW>
struct MmaPtrs {
  __amdgpu_buffer_rsrc_t xc, xs, wc, ws;
  uint32_t a[mma_row_slots<BM>()], as[mma_row_slots<BM>()];
  uint32_t b[NTW], bs[NTW];
  int ka, kb;  // K offset of this thread's A chunk / this lane's first B chunk within a step
};

// Descriptors and per-lane offsets of one workgroup tile: its token (row)
// tile starts at xc / xs and has nr valid rows, its weight (column) tile
// starts at wc / ws and has nc valid rows; both are [rows, D / 2] codes and
// [rows, D / 16] scales.
template <int BM, int NTW>
__device__ __forceinline__ MmaPtrs<BM, NTW> mma_ptrs(const uint8_t* xc, const uint8_t* xs, int64_t nr,
                                                     const uint8_t* wc, const uint8_t* ws, int64_t nc, int64_t D,
                                                     int wave, int lane) {
  MmaPtrs<BM, NTW> P;
  const int tid = threadIdx.x & (kMmaThreads - 1), q = tid & 3, r = lane & 31, h = lane >> 5;
  const int64_t rowc = D / 2, rows = D / 16;
  P.xc = make_rsrc(xc, nr * rowc);
  P.xs = make_rsrc(xs, nr * rows);
  P.wc = make_rsrc(wc, nc * rowc);
  P.ws = make_rsrc(ws, nc * rows);
  P.ka = 32 * q;
  P.kb = 32 * h;
#pragma unroll
  for (int i = 0; i < mma_row_slots<BM>(); ++i) {
    const int rl = (tid >> 2) + 64 * i;  // row within the tile
    P.a[i] = rl < BM ? (uint32_t)(rl * rowc + 16 * q) : kMmaOob;
    P.as[i] = rl < BM ? (uint32_t)(rl * rows + 2 * q) : kMmaOob;
  }
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int el = (wave + 4 * t) * 32 + r;  // expert within the block
    P.b[t] = (uint32_t)(el * rowc + 16 * h);
    P.bs[t] = (uint32_t)(el * rows + 2 * h);
  }
  return P;
}

template <bool STAGED, int BM, int NTW>
__device__ __forceinline__ void mma_load(MmaRegs<BM, NTW>& R, const MmaPtrs<BM, NTW>& P, int D, int step) {
  if constexpr (STAGED) {
    // D is a multiple of 256, so every step but the padding ones lies
    // wholly before D. Those read the last real step again, through the
    // scalar offset (the loop computes no addresses); their scales in the
    // window are zero, so they add nothing (E2M1 codes are always finite).
    const int so = 64 * min(step, D / 128 - 1);
#pragma unroll
    for (int i = 0; i < mma_row_slots<BM>(); ++i)
      R.a[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(P.xc, P.a[i], so, 0));
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < NTW; ++t)
        R.b[t][c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(P.wc, P.b[t] + 32 * c, so, 0));
    return;
  }
  const int k0 = step * 128;
  const bool aok = k0 + P.ka < D;
#pragma unroll
  for (int i = 0; i < mma_row_slots<BM>(); ++i) {
    const uint32_t oc = aok ? P.a[i] + 64 * step : kMmaOob, os = aok ? P.as[i] + 8 * step : kMmaOob;
    R.a[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(P.xc, oc, 0, 0));
    if constexpr (!STAGED) R.as[i] = __builtin_amdgcn_raw_buffer_load_b16(P.xs, os, 0, 0);
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const bool bok = k0 + 64 * c + P.kb < D;
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const uint32_t oc = bok ? P.b[t] + 64 * step + 32 * c : kMmaOob;
      const uint32_t os = bok ? P.bs[t] + 8 * step + 4 * c : kMmaOob;
      R.b[t][c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(P.wc, oc, 0, 0));
      if constexpr (!STAGED) R.bs[t][c] = __builtin_amdgcn_raw_buffer_load_b16(P.ws, os, 0, 0);
    }
  }
}

// Scale windows. LDS layout per window: row (A rows 0 .. BM - 1, then the
// 128 NTW B rows) at kMmaWinLd bytes, its kMmaWin steps' 8 scale bytes each
// in step order. The row stride of 17 dwords makes the reads of 32 rows at
// one offset conflict-free.
constexpr int kMmaWin = 8;     // K steps per scale window
constexpr int kMmaWinLd = 68;  // LDS bytes per row and window (64 + 4)

template <int BM, int NTW>
constexpr int mma_win_bytes() { return 2 * (BM + 128 * NTW) * kMmaWinLd; }  // both windows

// One window's loads, in flight between their issue and their LDS store:
// piece p = tid + NT j (j < NL) is bytes [16 (p % 4), +16) of the window's
// 64 bytes of row p / 4. A wavefront's 64 pieces are 16 whole rows, all of
// A or all of B. Pieces past the row's D / 16 scale bytes (the last window)
// and rows past the tile's valid rows load zeros.
template <int BM, int NTW, int KS>
struct ScaleWin {
  static constexpr int ROWS = BM + 128 * NTW, NP = 4 * ROWS, NT = kMmaThreads * KS, NL = (NP + NT - 1) / NT;
  u32x4_t v[NL];

  template <int J>
  __device__ __forceinline__ void load(const MmaPtrs<BM, NTW>& P, int win, int rows) {
    const int tid = threadIdx.x;
    const int p = tid + NT * J, row = p >> 2, part = p & 3;
    // The wavefront's first row, as a scalar: A or B is uniform per wavefront.
    const int row_w = __builtin_amdgcn_readfirstlane((tid & ~63) + NT * J) >> 2;
    const bool isA = row_w < BM;
    const int rr = isA ? row : row - BM;
    const int byte = 64 * win + 16 * part;
    const uint32_t off = (p < NP && byte < rows) ? (uint32_t)(rr * rows + byte) : kMmaOob;
    v[J] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(isA ? P.xs : P.ws, off, 0, 0));
  }

  template <int J>
  __device__ __forceinline__ void store(uint8_t* buf) const {
    const int p = threadIdx.x + NT * J;
    if (NP % NT == 0 || p < NP) {
      uint32_t* d = reinterpret_cast<uint32_t*>(buf + (p >> 2) * kMmaWinLd + 16 * (p & 3));
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = v[J][i];
    }
  }
};

__device__ __forceinline__ uint32_t lds_u16(const uint8_t* p) { return *reinterpret_cast<const uint16_t*>(p); }

// This thread's A chunks, converted, into the LDS tile.
template <int BM, int NTW>
__device__ __forceinline__ void mma_store_a(const MmaRegs<BM, NTW>& R, const uint32_t (&asw)[mma_row_slots<BM>()],
                                            _Float16* abuf) {
  const int tid = threadIdx.x & (kMmaThreads - 1), q = tid & 3;
#pragma unroll
  for (int i = 0; i < mma_row_slots<BM>(); ++i) {
    const int r = (tid >> 2) + 64 * i;
    if (r >= BM) break;  // BM = 32: threads 128..255 hold no row
    const half2_t sp = e4m3x2_f16(asw[i]);
    const _Float16 s0 = sp[0], s1 = sp[1];
    half8_t* dst = reinterpret_cast<half8_t*>(abuf + r * kMmaARow + 32 * q);
    dst[0] = fp4x8_scaled(R.a[i][0], s0);
    dst[1] = fp4x8_scaled(R.a[i][1], s0);
    dst[2] = fp4x8_scaled(R.a[i][2], s1);
    dst[3] = fp4x8_scaled(R.a[i][3], s1);
  }
}

// Accumulator sets per output tile: two (MFMAs j < 4 and j >= 4 alternate
// between them) when a wavefront has fewer than four tiles, so that enough
// independent MFMAs are in flight; they are added at the end.
template <int BM, int NTW>
constexpr int mma_sets() {
  return (BM / 32) * NTW < 4 ? 2 : 1;
}

// Two K groups (eight wavefronts) when a wavefront's accumulators leave room
// for two wavefronts per SIMD.
template <int BM, int NTW>
constexpr int mma_ksplit() {
  return (BM / 32) * NTW <= 2 ? 2 : 1;
}

// Look-ahead of the A-fragment reads, in K slices (8 per step): one, each
// fragment read right after the last MFMA that uses its register (with the
// row tiles outermost in a slice that leaves (BM / 32 - 1) NTW MFMAs to
// cover the LDS latency at the wide tiles; the other wavefront on the SIMD
// covers it at the narrow ones). Measured against two slices ahead:
// large-prefill gate 171 -> 160 us (fewer registers held), prefill
// unchanged; row tiles outermost instead of innermost and B parts three
// MFMAs apart: 165.6 -> 160.1 us, prefill 49.2 -> 47.5.
template <int BM, int NTW>
constexpr int mma_afrag_ahead() {
  return 1;
}
// A fragments in flight: [K slice mod mma_afrag_ahead()][row tile].
template <int BM, int NTW>
using MmaAFrags = half8_t[mma_afrag_ahead<BM, NTW>()][BM / 32];

// This lane's 32-element chunks of the B rows, converted (one unit per
// expert tile t and K slice j), from raw chunks R.b under scale words bsw.
template <int BM, int NTW>
__device__ __forceinline__ void mma_convert_b(half8_t (&B)[NTW][8], const MmaRegs<BM, NTW>& R,
                                              const uint32_t (&bsw)[NTW][2]) {
#pragma unroll
  for (int t = 0; t < NTW; ++t)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const half2_t sc = e4m3x2_f16(bsw[t][c]);
#pragma unroll
      for (int i = 0; i < 4; ++i) B[t][4 * c + i] = fp4x8_scaled(R.b[t][c][i], sc, i >> 1);
    }
}

// A fragment (row tile rt, K slice j) of this lane from the step's LDS tile:
// lane (r, h) takes row r, K [32h + 8j, +8) for j < 4 and [64 + 32h + 8(j - 4), +8)
// for j >= 4.
__device__ __forceinline__ half8_t mma_afrag(const _Float16* abuf, int lane, int rt, int j) {
  const _Float16* arow = abuf + (lane & 31) * kMmaARow + 32 * (lane >> 5);
  return *reinterpret_cast<const half8_t*>(arow + rt * 32 * kMmaARow + (j < 4 ? 8 * j : 64 + 8 * (j - 4)));
}

// The reads of a step's first mma_afrag_ahead() K slices of A fragments,
// issued before anything else of the step (after the barrier that makes the
// tile visible), so the first MFMA waits for one LDS round trip only.
template <int BM, int NTW>
__device__ __forceinline__ void mma_afrags_first(const _Float16* abuf, int lane, MmaAFrags<BM, NTW>& A) {
#pragma unroll
  for (int jj = 0; jj < mma_afrag_ahead<BM, NTW>(); ++jj)
#pragma unroll
    for (int rt = 0; rt < BM / 32; ++rt) A[jj][rt] = mma_afrag(abuf, lane, rt, jj);
}

// One step: the MFMAs of step s, A fragments from the LDS tile (the first
// slices already requested in A) and B units (converted during the previous
// step) from registers, in K-slice-major order (slice j: every row tile rt,
// and for each every expert tile t), so an A fragment's register is free
// after NTW MFMAs and the next slice's fragment is read R NTW - NTW MFMAs
// before its use. The next step's operands are converted during this one,
// one converted pair (two VALU instructions) at a time: part k of B unit
// (t, j) after the (3k + 1)-th MFMA past the last one that reads the unit
// (from Rn under scale words bswn), the parts of the next step's A
// chunks spread evenly over the MFMAs, each chunk stored to the other LDS
// tile after its last part. A wavefront alone on its SIMD issues one
// instruction every few clocks while an MFMA keeps the matrix core busy for
// 32, so this even spread (two or three VALU instructions per MFMA at the
// widest tiles) lets them overlap: with every B unit converted at the top
// of the step the MFMAs and the conversions ran largely one after the other
// (large-prefill gate 180 -> 168 us). Scheduling fences keep the order.
template <int BM, int NTW>
__device__ __forceinline__ void mma_step(MmaAFrags<BM, NTW>& A, half8_t (&B)[NTW][8],
                                         const MmaRegs<BM, NTW>& Rn, const uint32_t (&bswn)[NTW][2],
                                         const uint32_t (&aswn)[mma_row_slots<BM>()], const _Float16* abuf,
                                         _Float16* abuf_n, int lane,
                                         f32x16_t (&acc)[mma_sets<BM, NTW>()][BM / 32][NTW]) {
  constexpr int NS = mma_sets<BM, NTW>();
  constexpr int SL = mma_row_slots<BM>();
  constexpr int R = BM / 32;
  constexpr int NM = R * 8 * NTW;  // MFMAs
  constexpr int NA = 4 * SL;       // A chunks (units)
  constexpr int PF = mma_afrag_ahead<BM, NTW>();
  const int tid = threadIdx.x & (kMmaThreads - 1), q4 = tid & 3;
  // Scales of the next step, converted after the first MFMA is issued (their
  // LDS reads went out after the A fragments').
  half2_t bsc[NTW][2], asc[SL];
  auto scales = [&]() {
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int c = 0; c < 2; ++c) bsc[t][c] = e4m3x2_f16(bswn[t][c]);
#pragma unroll
    for (int i = 0; i < SL; ++i) asc[i] = e4m3x2_f16(aswn[i]);
  };
  // Part k of B unit u = (t, j): elements 2k, 2k + 1 of the unit.
  auto bpart = [&](auto uc) {
    constexpr int u = decltype(uc)::value, t = u / 32, j = (u / 4) % 8, k = u % 4;
    const half2_t sc = bsc[t][j / 4];
    const _Float16 sv = ((j % 4) >> 1) ? sc[1] : sc[0];
    reinterpret_cast<half2_t*>(&B[t][j])[k] =
        __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(Rn.b[t][j / 4][j % 4], 1.0f, k) * half2_t{sv, sv};
  };
  half2_t Ap[NA][4];
  auto apart = [&](auto pc) {
    constexpr int pi = decltype(pc)::value, u = pi / 4, k = pi % 4, i = u / 4, q = u % 4;
    const half2_t sc = asc[i];
    const _Float16 sv = (q >> 1) ? sc[1] : sc[0];
    Ap[u][k] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(Rn.a[i][q], 1.0f, k) * half2_t{sv, sv};
    if constexpr (k == 3) {
      const int row = (tid >> 2) + 64 * i;
      if (BM >= 64 || row < BM)  // BM = 32: threads 128..255 hold no row
        reinterpret_cast<half8_t*>(abuf_n + row * kMmaARow + 32 * q4)[q] = half8_t{
            Ap[u][0][0], Ap[u][0][1], Ap[u][1][0], Ap[u][1][1], Ap[u][2][0], Ap[u][2][1], Ap[u][3][0], Ap[u][3][1]};
    }
  };
  static_for<0, NM>([&](auto mc) {
    constexpr int m = decltype(mc)::value;
    constexpr int j = m / (NTW * R), rt = (m / NTW) % R, t = m % NTW;
    f32x16_t& c = acc[NS == 2 ? (j >> 2) : 0][rt][t];
    c = mfma32(A[j % PF][rt], B[t][j], c);
    if constexpr (m == 0) scales();
    if constexpr (t == NTW - 1 && j + PF < 8) A[j % PF][rt] = mma_afrag(abuf, lane, rt, j + PF);
    static_for<0, NTW * 32>([&](auto uc) {
      constexpr int u = decltype(uc)::value, tt = u / 32, jj = (u / 4) % 8, k = u % 4;
      constexpr int last = jj * NTW * R + (R - 1) * NTW + tt;  // the unit's last MFMA in this step
      constexpr int want = last + 1 + 3 * k;
      constexpr int slot = want < NM ? want : NM - 1;
      if constexpr (slot == m) bpart(uc);
    });
    static_for<(m * 4 * NA + NM - 1) / NM, ((m + 1) * 4 * NA + NM - 1) / NM>(apart);
    __builtin_amdgcn_sched_barrier(0);
  });
}

// The K loop of one workgroup tile: KS K groups of four wavefronts (group
// grp takes K steps grp, grp + KS, ...), loads RING steps ahead in a register
// ring, A converted into the group's two LDS tiles (abuf + (2 grp + i) BM
// kMmaARow halves), B converted in registers, each during the group's step
// before the one that uses them. One iteration covers a scale window of
// kMmaWin steps (kMmaWin / (KS RING) ring passes); nsteps is padded to a
// multiple of it, and padding steps load nothing (k >= D) and add zeros.
// STAGED: the next window's scale loads are spread over the first half of
// the window's positions (a position is one step of each group, ending at a
// barrier) and their LDS stores over the next ones, all before the barrier
// ahead of the last position, whose conversions (for the next window's
// first steps) read them. swin holds mma_win_bytes()
// bytes. Leaves acc[0] holding this group's sums (the two accumulator sets
// added).
template <int BM, int NTW, int KS, bool STAGED>
__device__ __forceinline__ void mma_mainloop(const MmaPtrs<BM, NTW>& P, int D, int nsteps, _Float16* abuf_base,
                                             uint8_t* swin, int lane,
                                             f32x16_t (&acc)[mma_sets<BM, NTW>()][BM / 32][NTW]) {
  constexpr int NS = mma_sets<BM, NTW>(), SL = mma_row_slots<BM>();
  constexpr int RING = mma_ring<BM, NTW>(), SPI = KS * RING, IPW = kMmaWin / SPI, POS = IPW * RING;
  static_assert(kMmaWin % SPI == 0, "a window holds whole ring passes");
  // The K group as a scalar, so that step indexes (and the staged loads'
  // scalar offsets) stay scalar.
  const int grp = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 8));
  const int tid = threadIdx.x & (kMmaThreads - 1), q4 = tid & 3, r = lane & 31, h = lane >> 5;
  const int rows = D / 16;
  auto abuf = [&](int i) { return abuf_base + (2 * grp + i) * (BM * kMmaARow); };
  constexpr int WB = (BM + 128 * NTW) * kMmaWinLd;  // one window
  // This lane's scale words of step-in-window sw from window buffer wb:
  // its A rows (the A conversion's 2 bytes at 2 q4) and its B rows (2 bytes
  // per 64-element chunk c at 4c + 2h).
  auto a_words = [&](int wb, int sw, uint32_t (&w)[SL]) {
#pragma unroll
    for (int i = 0; i < SL; ++i)
      w[i] = lds_u16(swin + wb * WB + min((tid >> 2) + 64 * i, BM - 1) * kMmaWinLd + 8 * sw + 2 * q4);
  };
  auto b_words = [&](int wb, int sw, uint32_t (&w)[NTW][2]) {
    const int wt = (threadIdx.x >> 6) & 3;
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        w[t][c] = lds_u16(swin + wb * WB + (BM + (wt + 4 * t) * 32 + r) * kMmaWinLd + 8 * sw + 4 * c + 2 * h);
  };
#pragma unroll
  for (int q = 0; q < NS; ++q)
#pragma unroll
    for (int rt = 0; rt < BM / 32; ++rt)
#pragma unroll
      for (int t = 0; t < NTW; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[q][rt][t][v] = 0.0f;
  MmaRegs<BM, NTW> R[RING];
#pragma unroll
  for (int p = 0; p < RING; ++p) mma_load<STAGED, BM, NTW>(R[p], P, D, KS * p + grp);
  ScaleWin<BM, NTW, KS> win;
  uint32_t aw[SL], bw[NTW][2];
  if constexpr (STAGED) {
    static_for<0, ScaleWin<BM, NTW, KS>::NL>([&](auto jc) { win.template load<decltype(jc)::value>(P, 0, rows); });
    static_for<0, ScaleWin<BM, NTW, KS>::NL>([&](auto jc) { win.template store<decltype(jc)::value>(swin); });
    __syncthreads();
    a_words(0, grp, aw);
    b_words(0, grp, bw);
  } else {
#pragma unroll
    for (int i = 0; i < SL; ++i) aw[i] = R[0].as[i];
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int c = 0; c < 2; ++c) bw[t][c] = R[0].bs[t][c];
  }
  // The group's first step: A into its first LDS tile, B into registers.
  half8_t B[NTW][8];
  mma_store_a<BM, NTW>(R[0], aw, abuf(0));
  mma_convert_b<BM, NTW>(B, R[0], bw);
  __syncthreads();
  for (int s0 = 0; s0 < nsteps; s0 += kMmaWin) {
    const int wi = s0 / kMmaWin, wb = wi & 1;
    static_for<0, IPW>([&](auto ic) {
      constexpr int it = decltype(ic)::value;
      static_for<0, RING>([&](auto pc) {
        constexpr int p = decltype(pc)::value, pos = it * RING + p;
        // Step s0 + it SPI + KS p + grp: its A (converted during the step
        // before) is in tile pos & 1 and its B in registers, so R[p] is
        // free: it reloads the step RING ahead first. The group's next step
        // (R[(p + 1) % RING]) is converted during this one: A into the
        // other tile, B into the registers as this step is done with them.
        constexpr int sw = it * SPI + KS * p;  // step in window, less grp
        uint32_t bn[NTW][2], an[SL];
        MmaAFrags<BM, NTW> A;
        mma_afrags_first<BM, NTW>(abuf(pos & 1), lane, A);
        __builtin_amdgcn_sched_barrier(0);
        mma_load<STAGED, BM, NTW>(R[p], P, D, s0 + it * SPI + KS * (p + RING) + grp);
        if constexpr (STAGED) {
          constexpr int NL = ScaleWin<BM, NTW, KS>::NL, NLP = POS / 2;
          if constexpr (pos < NLP)
            static_for<pos * NL / NLP, (pos + 1) * NL / NLP>(
                [&](auto jc) { win.template load<decltype(jc)::value>(P, wi + 1, rows); });
          // The next step is the next window's when sw + KS reaches kMmaWin.
          if constexpr (sw + KS < kMmaWin) {
            a_words(wb, sw + KS + grp, an);
            b_words(wb, sw + KS + grp, bn);
          } else {
            a_words(wb ^ 1, sw + KS - kMmaWin + grp, an);
            b_words(wb ^ 1, sw + KS - kMmaWin + grp, bn);
          }
        } else {
#pragma unroll
          for (int t = 0; t < NTW; ++t)
#pragma unroll
            for (int c = 0; c < 2; ++c) bn[t][c] = R[(p + 1) % RING].bs[t][c];
#pragma unroll
          for (int i = 0; i < SL; ++i) an[i] = R[(p + 1) % RING].as[i];
        }
        mma_step<BM, NTW>(A, B, R[(p + 1) % RING], bn, an, abuf(pos & 1), abuf((pos + 1) & 1), lane, acc);
        if constexpr (STAGED) {
          constexpr int NL = ScaleWin<BM, NTW, KS>::NL, NSP = POS - 1 - POS / 2;
          if constexpr (pos >= POS / 2 && pos < POS - 1)
            static_for<(pos - POS / 2) * NL / NSP, (pos - POS / 2 + 1) * NL / NSP>(
                [&](auto jc) { win.template store<decltype(jc)::value>(swin + (wb ^ 1) * WB); });
        }
        __syncthreads();
      });
    });
  }
  if (NS == 2) {
#pragma unroll
    for (int rt = 0; rt < BM / 32; ++rt)
#pragma unroll
      for (int t = 0; t < NTW; ++t) acc[0][rt][t] += acc[NS - 1][rt][t];
  }
}

// K steps of 128 elements for D, padded to a whole number of scale windows
// (each a whole number of K groups times the ring depth).
template <int BM, int NTW>
inline int mma_padded_steps(int64_t D) {
  const int steps = (int)((D + 127) / 128);
  return (steps + kMmaWin - 1) / kMmaWin * kMmaWin;
}

}  // namespace nvr
