// Device helpers shared by the quantizer and the gate kernels (gfx950 only).
//
// Number formats: NVFP4 = E2M1 element codes (1 sign, 2 exponent bits with
// bias 1, 1 mantissa bit; values 0, 0.5, 1, 1.5, 2, 3, 4, 6) times an E4M3FN
// block scale per 16 elements (bias 7, 3 mantissa bits, largest finite 448)
// times one fp32 global scale. The 448 ceiling and the global scale
// max|x| / (6 * 448) come from commit 04cf8ca8 (dsv4/layers/router.py,
// runtime-gsa paragraph).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvr {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kGsaDivisor = 2688.0f;  // 6 (largest E2M1) * 448 (largest E4M3)

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// |x| of both bf16 halves as 15-bit magnitudes; the larger one. Magnitude bit
// patterns of non-negative bf16 order like their values (NaN above +inf).
__device__ __forceinline__ uint32_t bf16_pair_absmax(uint32_t w) {
  return max(w & 0x7FFFu, (w >> 16) & 0x7FFFu);
}

// Value of a non-negative E4M3FN byte (0x00..0x7E): m * 2^-9 when the
// exponent field is 0, (8 + m) * 2^(e - 10) otherwise. Exact in fp32.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 0xFu, m = b & 7u;
  return e ? ldexpf((float)(8u + m), (int)e - 10) : (float)m * 0x1p-9f;
}

// Code of the value nearest to q >= 0 on a minifloat grid with MBITS
// mantissa bits, smallest normal exponent EMIN and largest code MAXCODE;
// ties to even, saturating. Exact for every double q: with e = floor(log2 q)
// (clamped to EMIN for the subnormal range), q * 2^(MBITS - e) is exact and
// rint() rounds it to the nearest integer, ties to even; the carry of a
// round-up lands in the exponent field by itself.
template <int MBITS, int EMIN, int MAXCODE>
__device__ __forceinline__ uint32_t round_minifloat(double q) {
  if (!(q > 0.0)) return 0u;
  if (!(q < 0x1p40)) return (uint32_t)MAXCODE;
  int e;
  (void)frexp(q, &e);  // q = f * 2^e with f in [0.5, 1)
  e = max(e - 1, EMIN);
  const double r = rint(ldexp(q, MBITS - e));
  const int code = ((e - EMIN) << MBITS) + (int)r;
  return (uint32_t)min(code, MAXCODE);
}

__device__ __forceinline__ uint32_t e4m3_round(double q) { return round_minifloat<3, -6, 0x7E>(q); }
__device__ __forceinline__ uint32_t e2m1_round(double q) { return round_minifloat<1, 0, 7>(q); }

// Sign-only codes of the 8 elements held in four bf16 pairs, packed as the
// quantizer packs them (element 2i in the low nibble of byte i).
__device__ __forceinline__ uint32_t sign_codes4(const uint32_t* w) {
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t byte = ((w[i] >> 12) & 0x8u) | ((w[i] >> 24) & 0x80u);
    out |= byte << (8 * i);
  }
  return out;
}

// Distance key of a scaled element to the nearest value with at most two
// explicit mantissa bits (every E2M1 rounding threshold 0.25, 0.75, 1.25,
// 1.75, 2.5, 3.5, 5 is one). Values below 0.2 always give magnitude 0 and
// are clamped away from the test. A key below kNearKeyLimit means "within
// 32 fp32 ulps of such a value".
__device__ __forceinline__ uint32_t near_grid_key(float q) {
  const uint32_t u = __float_as_uint(fmaxf(fabsf(q), 0.2f));
  return (u + 32u) << 11;  // low 21 mantissa bits, offset by 32 ulps
}
constexpr uint32_t kNearKeyLimit = 64u << 11;

// One bf16 pair scaled by inv and rounded to two E2M1 codes by the hardware
// conversion (scale operand 1.0), written into byte I of `old`: the even
// element in the low nibble. Also folds both elements into the near-tie key.
template <int I>
__device__ __forceinline__ uint32_t fp4_fast_pair(uint32_t old, uint32_t w, float inv, uint32_t& key) {
  const float a = bf16_lo(w) * inv, b = bf16_hi(w) * inv;
  key = min(key, min(near_grid_key(a), near_grid_key(b)));
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, I);
}

__device__ __forceinline__ uint32_t fp4_fast8(const uint32_t* w, float inv, uint32_t& key) {
  uint32_t o = 0;
  o = fp4_fast_pair<0>(o, w[0], inv, key);
  o = fp4_fast_pair<1>(o, w[1], inv, key);
  o = fp4_fast_pair<2>(o, w[2], inv, key);
  o = fp4_fast_pair<3>(o, w[3], inv, key);
  return o;
}

// Quantize one 16-element block held as eight bf16 pairs (element 2i in the
// low half of w[i]) with global scale gsa. Produces 8 code bytes (c0 =
// elements 0..7, c1 = elements 8..15) and the E4M3 scale byte.
//
// Block scale: E4M3 nearest to bmax / (6 gsa), decided in double (6 gsa is
// exact there, the quotient is correctly rounded, and a quotient of these
// operands can only be as close to an E4M3 midpoint as ~2^-31 relative
// unless it equals it, so the double result rounds the same way as the
// exact one).
//
// Element codes, fast path: q = x * rcp(gsa * S) is within ~4 ulps of the
// exact quotient. The hardware FP4 conversion rounds q to nearest; this is
// the exact answer unless q lies near a rounding threshold, which the
// near_grid_key test detects. Blocks with such an element (rare on real
// data), and blocks whose gsa * S is too small for an accurate fp32
// reciprocal, are redone exactly in double, element by element.
__device__ __forceinline__ void quant_block16(const uint32_t* w, float gsa, uint32_t& c0, uint32_t& c1,
                                              uint32_t& sbyte) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, bf16_pair_absmax(w[i]));
  if (!(gsa > 0.0f)) {  // gsa == 0: all-zero tensor or zero override
    sbyte = 0;
    c0 = sign_codes4(w);
    c1 = sign_codes4(w + 4);
    return;
  }
  const float bmax = __uint_as_float(m << 16);
  sbyte = e4m3_round((double)bmax / (6.0 * (double)gsa));
  const float S = e4m3_value(sbyte);
  if (S == 0.0f) {
    c0 = sign_codes4(w);
    c1 = sign_codes4(w + 4);
    return;
  }
  const float G = gsa * S;
  bool exact = !(G >= 0x1p-100f);
  if (!exact) {
    const float inv = __builtin_amdgcn_rcpf(G);
    uint32_t key = 0xFFFFFFFFu;
    c0 = fp4_fast8(w, inv, key);
    c1 = fp4_fast8(w + 4, inv, key);
    exact = key < kNearKeyLimit;
  }
  if (exact) {
    const double G64 = (double)gsa * (double)S;  // exact product
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t lo = e2m1_round(fabs((double)bf16_lo(w[i])) / G64) | ((w[i] >> 12) & 0x8u);
      const uint32_t hi = e2m1_round(fabs((double)bf16_hi(w[i])) / G64) | ((w[i] >> 28) & 0x8u);
      out[i >> 2] |= (lo | (hi << 4)) << (8 * (i & 3));
    }
    c0 = out[0];
    c1 = out[1];
  }
}

// Eight E2M1 codes (one dword) times the block scale, as fp16 (exact: a code
// value has at most 2 significant bits, an E4M3 scale 4, and the product
// lies in [2^-10, 2688]). The element order inside the vector is whatever
// the hardware conversion gives; both MFMA operands use this same function,
// so products pair up element for element.
__device__ __forceinline__ half8_t fp4x8_to_f16(uint32_t c, _Float16 s) {
  const half2_t ss = {s, s};
  const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 0) * ss;
  const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 1) * ss;
  const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 2) * ss;
  const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 3) * ss;
  return half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

__device__ __forceinline__ _Float16 e4m3_f16(uint32_t b) { return (_Float16)e4m3_value(b); }

// Eight E2M1 codes as their exact fp16 values, in the hardware conversion's
// element order (scale operand 1.0: the conversion applies only the exponent
// of its scale operand, so block scales are multiplied separately).
__device__ __forceinline__ half8_t fp4x8_q(uint32_t c) {
  const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 0);
  const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 1);
  const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 2);
  const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 3);
  return half8_t{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// sum_i a_i * b_i over 8 fp16 pairs with fp32 accumulation. For E2M1 code
// values every product (|q q| <= 36, a multiple of 1/4) and every partial sum
// is exact in fp32.
__device__ __forceinline__ float dot8(half8_t a, half8_t b, float acc) {
  acc = __builtin_amdgcn_fdot2(half2_t{a[0], a[1]}, half2_t{b[0], b[1]}, acc, false);
  acc = __builtin_amdgcn_fdot2(half2_t{a[2], a[3]}, half2_t{b[2], b[3]}, acc, false);
  acc = __builtin_amdgcn_fdot2(half2_t{a[4], a[5]}, half2_t{b[4], b[5]}, acc, false);
  acc = __builtin_amdgcn_fdot2(half2_t{a[6], a[7]}, half2_t{b[6], b[7]}, acc, false);
  return acc;
}

// Wavefront-wide reductions with DPP row operations (VALU latency, no LDS
// crossbar): xor-1 and xor-2 quad permutes, the 8-lane and 16-lane mirrors
// leave every lane with its 16-lane row's result; four readlanes finish.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7-i within 8
constexpr int kDppMirror = 0x140;      // lane i <- 15-i within 16

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __int_as_float(dpp_i<kDppXor1>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_i<kDppXor2>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_i<kDppHalfMirror>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_i<kDppMirror>(__float_as_int(v))));
  const int iv = __float_as_int(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(iv, 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(iv, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(iv, 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(iv, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)dpp_i<kDppXor1>((int)v));
  v = max(v, (uint32_t)dpp_i<kDppXor2>((int)v));
  v = max(v, (uint32_t)dpp_i<kDppHalfMirror>((int)v));
  v = max(v, (uint32_t)dpp_i<kDppMirror>((int)v));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Sum over the wavefront in a fixed order (deterministic).
__device__ __forceinline__ float wave_sum(float v) {
  v += __int_as_float(dpp_i<kDppXor1>(__float_as_int(v)));
  v += __int_as_float(dpp_i<kDppXor2>(__float_as_int(v)));
  v += __int_as_float(dpp_i<kDppHalfMirror>(__float_as_int(v)));
  v += __int_as_float(dpp_i<kDppMirror>(__float_as_int(v)));
  const int iv = __float_as_int(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(iv, 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(iv, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(iv, 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(iv, 48));
  return (r0 + r1) + (r2 + r3);
}

// Six-step routing of one token by one wavefront (commit e0f60b9f,
// dsv4/kernels/router/__init__.py: the single-pass activation/top-k
// epilogue; sorted output as in the selection sort of commit 04cf8ca8):
// s = sigmoid(L); b = s + bias; the k largest b in descending order (exact
// ties to the lower expert); gather the unbiased s of each; w = s / sum s;
// w *= routed_scale. Lane l holds experts l, l + 64, ...; each round takes
// the wave maximum and the lowest expert index that attains it, so the
// chosen list comes out sorted. Lrow may point to LDS or global memory.
template <int JMAX>
__device__ __forceinline__ void wave_route_row(const float* Lrow, const float* __restrict__ bias, int E, int k,
                                               float routed_scale, int32_t* __restrict__ out_idx,
                                               float* __restrict__ out_w) {
  const int lane = threadIdx.x & 63;
  float s[JMAX], b[JMAX];
  uint32_t live = 0;
#pragma unroll
  for (int j = 0; j < JMAX; ++j) {
    const int e = lane + 64 * j;
    s[j] = 0.0f;
    b[j] = -INFINITY;
    if (e < E) {
      s[j] = 1.0f / (1.0f + expf(-Lrow[e]));
      b[j] = s[j] + bias[e];
      live |= 1u << j;
    }
  }
  int my_idx = 0;
  float my_s = 0.0f, ssum = 0.0f;
  for (int r = 0; r < k; ++r) {
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < JMAX; ++j)
      if ((live >> j) & 1u) m = fmaxf(m, b[j]);
    const float M = wave_max(m);
    int win = -1;
#pragma unroll
    for (int j = 0; j < JMAX; ++j) {
      if (win < 0) {
        const uint64_t bal = __ballot(((live >> j) & 1u) && b[j] == M);
        if (bal) win = 64 * j + (__ffsll((unsigned long long)bal) - 1);
      }
    }
    if (win < 0) {  // only NaN scores left: take the lowest remaining expert
#pragma unroll
      for (int j = 0; j < JMAX; ++j) {
        if (win < 0) {
          const uint64_t bal = __ballot((live >> j) & 1u);
          if (bal) win = 64 * j + (__ffsll((unsigned long long)bal) - 1);
        }
      }
    }
    const int wj = win >> 6, wl = win & 63;
    float sv = 0.0f;
#pragma unroll
    for (int j = 0; j < JMAX; ++j)
      if (j == wj) sv = s[j];
    sv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv), wl));
    if (lane == wl) live &= ~(1u << wj);
    if (lane == r) {
      my_idx = win;
      my_s = sv;
    }
    ssum += sv;
  }
  if (lane < k) {
    out_idx[lane] = my_idx;
    out_w[lane] = routed_scale * (my_s / ssum);
  }
}

}  // namespace nvr
