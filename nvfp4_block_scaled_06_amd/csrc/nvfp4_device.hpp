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

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// Largest |x| (15-bit magnitude pattern) over N bf16 pairs, with packed
// 16-bit maxima.
template <int N>
__device__ __forceinline__ uint32_t bf16_words_absmax(const uint32_t* w) {
  u16x2_t m = __builtin_bit_cast(u16x2_t, w[0] & 0x7FFF7FFFu);
#pragma unroll
  for (int i = 1; i < N; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, w[i] & 0x7FFF7FFFu));
  return max((uint32_t)m[0], (uint32_t)m[1]);
}
__device__ __forceinline__ uint32_t bf16_block_absmax(const uint32_t* w) { return bf16_words_absmax<8>(w); }

// Value of a non-negative E4M3FN byte (0x00..0x7E): m * 2^-9 when the
// exponent field e is 0, (8 + m) * 2^(e - 10) otherwise. Shifted left by 7,
// the byte is the fp16 pattern of the same value times 2^-8 (fp16's
// exponent bias is 8 more, its subnormals continue E4M3's), so one shift and
// one exact multiply by 256 decode it.
__device__ __forceinline__ _Float16 e4m3_f16(uint32_t b) {
  return __builtin_bit_cast(_Float16, (uint16_t)(b << 7)) * (_Float16)256.0f;
}
__device__ __forceinline__ float e4m3_value(uint32_t b) { return (float)e4m3_f16(b); }

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

// E2M1 code of one element, exact for every quotient q = |x| / (gsa S)
// (gsa in [2^-80, 2^100], S > 0 or inv = 0), from the approximate quotient
// qa = x * inv (signed, as inv >= 0; within a few ulps of +-q), as the fp32
// value that the hardware conversion (round to nearest even on the
// magnitude, saturating, sign kept) then maps to the right code. Every E2M1
// value and every rounding threshold (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5)
// has at most two explicit mantissa bits:
//  1. v = the value nearest qa with at most two explicit mantissa bits (the
//     rounding acts on the magnitude bits; the sign bit is kept). Between |v|
//     and q there is no threshold other than |v| itself. A huge qa (a
//     too-small static gsa) may round to +-inf; then |v| S gsa is +inf, the
//     residual below is -inf, v moves toward zero to a large finite value and
//     the conversion saturates to +-6, as q does.
//  2. r = |x| - |v| S gsa by one fma (abs modifiers) has the exact sign of
//     q - |v|: |v| S is exact (at most 7 significant bits) and every term is
//     a multiple of 2^-31 |v| S gsa, far above the fp32 underflow threshold in
//     this range, so the fma's one rounding cannot reach or cross zero. r is
//     never -0 (|x| >= 0, and an exact zero sum rounds to +0), so its bit
//     pattern read as an integer and clamped to [-1, 1] is the sign of
//     q - |v|.
//  3. |v| moves toward q by 2^12 units in its last place (between 2^-12 |v|
//     and 2^-11 |v|; one shift-add on the bit pattern, which moves the
//     magnitude the same way for either sign): a threshold then converts to
//     the code on q's side, an exact tie (r = 0) stays on the threshold and
//     converts to the even code, and any other v keeps its own code. When
//     v = +-0 (x = +-0, or a zero scale with inv = 0) r >= 0, and the move
//     gives a tiny value of x's sign that converts to code 0 with that sign
//     (so -0 and tiny negatives keep their sign).
__device__ __forceinline__ float e2m1_exact_input(float x, float inv, float S, float gsa) {
  const float qa = x * inv;
  const uint32_t vb = (__float_as_uint(qa) + 0x100000u) & 0xFFE00000u;
  const float r = fmaf(-(fabsf(__uint_as_float(vb)) * S), gsa, fabsf(x));
  // One v_med3_i32 (the compiler would otherwise lower the clamp to two
  // compare/select pairs).
  int sgn;
  asm("v_med3_i32 %0, %1, -1, 1" : "=v"(sgn) : "v"(__float_as_uint(r)));
  return __uint_as_float(vb + ((uint32_t)sgn << 12));
}

// One bf16 pair rounded to two E2M1 codes, written into byte I of `old`: the
// even element in the low nibble.
template <int I>
__device__ __forceinline__ uint32_t fp4_exact_pair(uint32_t old, uint32_t w, float inv, float S, float gsa) {
  const float a = e2m1_exact_input(bf16_lo(w), inv, S, gsa);
  const float b = e2m1_exact_input(bf16_hi(w), inv, S, gsa);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, I);
}

__device__ __forceinline__ uint32_t fp4_exact8(const uint32_t* w, float inv, float S, float gsa) {
  uint32_t o = 0;
  o = fp4_exact_pair<0>(o, w[0], inv, S, gsa);
  o = fp4_exact_pair<1>(o, w[1], inv, S, gsa);
  o = fp4_exact_pair<2>(o, w[2], inv, S, gsa);
  o = fp4_exact_pair<3>(o, w[3], inv, S, gsa);
  return o;
}

// E4M3 byte of a non-negative fp32 p <= 448, rounded to nearest (exact ties
// are not decided here: callers screen them out with near_scale_key). Normal
// range: round the fp32 pattern to 3 mantissa bits (the carry rolls into the
// exponent) and rebias 127 -> 7; subnormal range (p < 2^-6): p * 2^9 rounded.
// Both roundings are formed and one is selected (no branch: blocks of one
// wavefront often mix normal and subnormal scales).
__device__ __forceinline__ uint32_t e4m3_from_f32(float p) {
  const uint32_t u = __float_as_uint(p);
  const uint32_t normal = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
  const uint32_t subnormal = (uint32_t)rintf(p * 512.0f);
  return p >= 0x1p-6f ? normal : subnormal;
}

// Distance key to the nearest value with at most four explicit mantissa bits
// (every E4M3 rounding midpoint, subnormal ones included, is one). p is
// clamped to [1.2 * 2^-12, 440]: below, the scale is always 0; from 440 up
// it is always 448 (the top midpoint 432 is far below), and neither clamp
// value is near a four-bit value, so the block holding the tensor's max
// (p within an ulp of 448) does not trip the test.
__device__ __forceinline__ uint32_t near_scale_key(float p) {
  const uint32_t u = __float_as_uint(__builtin_amdgcn_fmed3f(p, 0x1.3p-12f, 440.0f));  // p >= 0
  return (u << 13) + (32u << 13);  // low 19 mantissa bits, offset by 32 ulps
}
constexpr uint32_t kNearScaleLimit = 64u << 13;

// Exact E4M3 scale byte of bmax / (6 gsa) for an approximate quotient p near
// a value v with at most four explicit mantissa bits (near_scale_key); the
// same construction with 6v (at most 7 significant bits, exact) and the
// E4M3 midpoints as the thresholds.
__device__ __forceinline__ uint32_t e4m3_byte_exact(float bmax, float p, float gsa) {
  const float v = __uint_as_float((__float_as_uint(p) + 0x40000u) & ~0x7FFFFu);
  const uint32_t lo = e4m3_from_f32(fminf(v * 0x1.ffep-1f, 448.0f));
  const uint32_t hi = e4m3_from_f32(fminf(v * 0x1.001p+0f, 448.0f));
  if (lo == hi) return lo;
  const float r = fmaf(-(6.0f * v), gsa, bmax);
  return r > 0.0f ? hi : (r < 0.0f ? lo : ((lo & 1u) ? hi : lo));
}

// Block scale of a 16-element block from its bf16 absolute maximum m (the
// bit pattern) and the global scale gsa, with what the element encoder needs.
//
// For gsa in [2^-80, 2^100] (every real tensor; `fast`):
//  * p = bmax * rcp(6 gsa) is within ~3 ulps of the exact quotient; rounding
//    it is exact unless it lies near an E4M3 midpoint (near_scale_key),
//    where e4m3_byte_exact decides;
//  * elements then take e2m1_exact_input, with no data-dependent branch
//    (with bf16 inputs and E4M3 scales, quotients land exactly on E2M1
//    values and thresholds in a sizeable fraction of blocks, so a screened
//    fallback would be taken by nearly every wavefront). A zero scale gives
//    inv = 0 and sign-only codes.
// Outside that range (tensors of tiny or huge magnitude, or gsa = 0) every
// quotient is formed in double: the operands' products are exact there, the
// division is correctly rounded, and a quotient of these operands is either
// exactly on a rounding boundary or ~2^-31 (relative) away from it, so the
// double result rounds like the exact one.
struct BlockScale {
  uint32_t sbyte;
  float S, inv;
  double G64;  // gsa * S, exact (slow path)
  bool fast;
};

__device__ __forceinline__ BlockScale block_scale(uint32_t m, float gsa) {
  BlockScale b;
  const float bmax = __uint_as_float(m << 16);
  b.fast = gsa >= 0x1p-80f && gsa <= 0x1p100f;
  if (b.fast) {
    const float p = bmax * __builtin_amdgcn_rcpf(6.0f * gsa);
    b.sbyte = near_scale_key(p) < kNearScaleLimit ? e4m3_byte_exact(bmax, p, gsa) : e4m3_from_f32(fminf(p, 448.0f));
  } else {
    b.sbyte = gsa > 0.0f ? e4m3_round((double)bmax / (6.0 * (double)gsa)) : 0u;
  }
  b.S = e4m3_value(b.sbyte);
  b.inv = (b.fast && b.S > 0.0f) ? __builtin_amdgcn_rcpf(gsa * b.S) : 0.0f;
  b.G64 = (double)gsa * (double)b.S;
  return b;
}

// Codes of 8 elements (four bf16 pairs) under block scale b, packed as the
// quantizer packs them (element 2i in the low nibble of byte i).
__device__ __forceinline__ uint32_t encode8(const uint32_t* w, const BlockScale& b, float gsa) {
  if (b.fast) return fp4_exact8(w, b.inv, b.S, gsa);
  if (b.S == 0.0f) return sign_codes4(w);
  uint32_t out = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = e2m1_round(fabs((double)bf16_lo(w[i])) / b.G64) | ((w[i] >> 12) & 0x8u);
    const uint32_t hi = e2m1_round(fabs((double)bf16_hi(w[i])) / b.G64) | ((w[i] >> 28) & 0x8u);
    out |= (lo | (hi << 4)) << (8 * i);
  }
  return out;
}

// Quantize one 16-element block held as eight bf16 pairs (element 2i in the
// low half of w[i]) with global scale gsa: 8 code bytes (c0 = elements 0..7,
// c1 = elements 8..15) and the E4M3 scale byte.
__device__ __forceinline__ void quant_block16(const uint32_t* w, float gsa, uint32_t& c0, uint32_t& c1,
                                              uint32_t& sbyte) {
  const BlockScale b = block_scale(bf16_block_absmax(w), gsa);
  sbyte = b.sbyte;
  c0 = encode8(w, b, gsa);
  c1 = encode8(w + 4, b, gsa);
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

// sum_i a_i * b_i over 8 fp16 pairs with fp32 accumulation. For the scaled
// code values of one block pair (q_x S_x and q_w S_w) every product is a
// multiple of S_x S_w / 4 below 36 S_x S_w, so products and partial sums
// are exact in fp32.
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
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
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

// Logistic function 1 / (1 + e^-L) from the hardware base-2 exponential and
// reciprocal: e^-L = 2^(-L log2 e); relative error ~1e-6 for |L| <= 20 (the
// scores it feeds are compared and summed at 1e-5). Saturates to exactly 0 and
// 1 at the extremes.
__device__ __forceinline__ float sigmoid_fast(float L) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * L));
}

// Order-preserving key of an fp32 selection score: larger b gives a larger
// unsigned key, equal b equal keys (-0 is folded into +0 first). Key 0 is
// reserved for "already chosen"; only a negative NaN could map there and it
// is lifted to 1.
__device__ __forceinline__ uint32_t score_key(float b) {
  const uint32_t u = __float_as_uint(b + 0.0f);
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return max(k, 1u);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)dpp_i<CTRL>((int)v);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_u<kDppXor1>(v));
  v = min(v, dpp_u<kDppXor2>(v));
  v = min(v, dpp_u<kDppHalfMirror>(v));
  v = min(v, dpp_u<kDppMirror>(v));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return min(min(r0, r1), min(r2, r3));
}

// Max over aligned groups of GL lanes (GL a power of two up to 16); every
// lane of a group gets the group's maximum.
template <int GL>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  if (GL >= 2) v = max(v, dpp_u<kDppXor1>(v));
  if (GL >= 4) v = max(v, dpp_u<kDppXor2>(v));
  if (GL >= 8) v = max(v, dpp_u<kDppHalfMirror>(v));
  if (GL >= 16) v = max(v, dpp_u<kDppMirror>(v));
  return v;
}

constexpr int kRouteFastSurvivors = 32;

// LDS scratch of one wavefront's router; entry 64 JMAX of cand / cs is a
// spare slot that absorbs the writes of keys that do not survive.
template <int JMAX>
struct WaveRouteScratch {
  uint64_t cand[64 * JMAX + 8];
  float cs[64 * JMAX + 8];
  float sel_s[64];
  int sel_i[32];
};

// Row broadcasts of the wave-wide reductions (lane 15 of rows 0 and 2 into
// rows 1 and 3; lane 31 into rows 2 and 3); rows not written keep `id`.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_bcast(uint32_t v, uint32_t id) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, CTRL, ROWS, 0xF, false);
}
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

// Smallest value over the wavefront, for values already equal within each
// aligned group of GL lanes (GL = 2, 4, 8 or 16): the other groups of each
// row (pairs into quads, quads into eights, eights into rows), then the rows;
// read from lane 63.
template <int GL>
__device__ __forceinline__ uint32_t wave_min_of_groups(uint32_t v) {
  if constexpr (GL <= 2) v = min(v, dpp_u<kDppXor2>(v));
  if constexpr (GL <= 4) v = min(v, dpp_u<kDppHalfMirror>(v));
  if constexpr (GL <= 8) v = min(v, dpp_u<kDppMirror>(v));
  v = min(v, dpp_bcast<kDppRowBcast15, 0xA>(v, 0xFFFFFFFFu));
  v = min(v, dpp_bcast<kDppRowBcast31, 0xC>(v, 0xFFFFFFFFu));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Sum over the wavefront in a fixed order (deterministic), left in lane 63.
__device__ __forceinline__ float wave_sum_bcast(float v) {
  v += __int_as_float(dpp_i<kDppXor1>(__float_as_int(v)));
  v += __int_as_float(dpp_i<kDppXor2>(__float_as_int(v)));
  v += __int_as_float(dpp_i<kDppHalfMirror>(__float_as_int(v)));
  v += __int_as_float(dpp_i<kDppMirror>(__float_as_int(v)));
  v += __uint_as_float(dpp_bcast<kDppRowBcast15, 0xA>(__float_as_uint(v), 0u));
  v += __uint_as_float(dpp_bcast<kDppRowBcast31, 0xC>(__float_as_uint(v), 0u));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// The value this lane's partner in the other half of the wavefront holds
// (lane l and l +- 32): one v_permlane32_swap.
__device__ __forceinline__ uint32_t other_half(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}

// Six-step routing of one token by one wavefront (commit e0f60b9f,
// dsv4/kernels/router/__init__.py: the single-pass activation/top-k
// epilogue; sorted output as in the selection sort of commit 04cf8ca8):
// s = sigmoid(L); b = s + bias; the k largest b in descending order (exact
// ties to the lower expert); gather the unbiased s of each; w = s / sum s;
// w *= routed_scale.
//
// Lane l holds experts l, l+64, ... (JMAX of them). Selection without k
// serial rounds, and without divergent branches on the usual path:
//  1. every lane forms s and the order-preserving score key of its experts;
//  2. the lanes form G >= k aligned groups; the smallest group maximum is a
//     lower bound on the k-th largest key (the G group maxima are G >= k
//     distinct experts at or above it), so experts below it cannot be chosen;
//  3. the survivors (at least k, typically a few more) are compacted into LDS
//     by ballot (the others write a spare slot) and each one's exact rank
//     among them is counted: larger key first, lower expert first on equal
//     keys, i.e. the larger (key, ~expert) pair. Survivors outrank every
//     other expert, so that is the global rank. With at most 32 survivors,
//     lanes l and l + 32 both take survivor l, each against half of the list,
//     and add their counts across the halves;
//  4. ranks below k are the chosen list, already sorted; the weights use a
//     fixed-order (DPP tree) sum of the chosen s.
// One wavefront, no workgroup barrier: LDS traffic of a single wave is
// processed in order, and a compiler fence keeps the code order.
template <int JMAX>
__device__ __forceinline__ void wave_route_regs(const float (&L)[JMAX], const float (&bv)[JMAX], int E, int k,
                                                float routed_scale, int32_t* __restrict__ out_idx,
                                                float* __restrict__ out_w, WaveRouteScratch<JMAX>& sc) {
  const int lane = threadIdx.x & 63;
  float s[JMAX];
  uint32_t key[JMAX];
#pragma unroll
  for (int j = 0; j < JMAX; ++j) {
    s[j] = sigmoid_fast(L[j]);
    const uint32_t kk = score_key(s[j] + bv[j]);
    key[j] = lane + 64 * j < E ? kk : 0u;
  }
  uint32_t lm = key[0];
#pragma unroll
  for (int j = 1; j < JMAX; ++j) lm = max(lm, key[j]);
  // Groups of GL lanes, GL the largest power of two with 64 / GL >= k (up to
  // 16: one DPP row); fewer than four groups take row maxima and fold them.
  uint32_t tau;
  if (k > 4) {
    if (k <= 8) tau = wave_min_of_groups<8>(group_max_u32<8>(lm));
    else if (k <= 16) tau = wave_min_of_groups<4>(group_max_u32<4>(lm));
    else tau = wave_min_of_groups<2>(group_max_u32<2>(lm));
  } else {
    const uint32_t gmax = group_max_u32<16>(lm);
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)gmax, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)gmax, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)gmax, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)gmax, 48);
    const uint32_t g01 = max(r0, r1), g23 = max(r2, r3);
    tau = k <= 1 ? max(g01, g23) : (k <= 2 ? min(g01, g23) : min(min(r0, r1), min(r2, r3)));
  }

  // Compact the survivors: each writes its slot, the others the spare one.
  constexpr int kSpare = 64 * JMAX;
  int C = 0;
#pragma unroll
  for (int j = 0; j < JMAX; ++j) {
    const bool cand = key[j] != 0u && key[j] >= tau;
    const uint64_t bal = __ballot(cand);
    const int pos = C + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
    const int slot = cand ? pos : kSpare;
    sc.cand[slot] = ((uint64_t)key[j] << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)(lane + 64 * j));
    sc.cs[slot] = s[j];
    C += (int)__popcll(bal);
  }
  const float rsc = routed_scale;
  if (C <= kRouteFastSurvivors) {
    // Usual case. Entries C .. 31 are zero and rank below everything.
    if (lane >= C && lane < kRouteFastSurvivors) sc.cand[lane] = 0ull;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int u = lane & 31, half = lane >> 5;
    const uint64_t mine = sc.cand[u];
    const float ms = sc.cs[u];
    uint64_t part[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) part[i] = sc.cand[16 * half + i];
    int rank = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) rank += part[i] > mine ? 1 : 0;
    rank += (int)other_half((uint32_t)rank);
    const bool chosen = lane < C && lane < 32 && rank < k;
    const float ssum = wave_sum_bcast(chosen ? ms : 0.0f);
    if (chosen) {
      out_idx[rank] = (int)(0xFFFFFFFFu - (uint32_t)mine);
      out_w[rank] = ms * (rsc * __builtin_amdgcn_rcpf(ssum));
    }
    return;
  }
  if (lane < 8) sc.cand[C + lane] = 0ull;  // padding: ranks below nobody
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // Many survivors (flat or tied scores): rank in batches of 8.
  for (int c = lane; c < ((C + 63) & ~63); c += 64) {
    const uint64_t mine = sc.cand[min(c, C - 1)];
    const float ms = sc.cs[min(c, C - 1)];
    int rank = 0;
    for (int c0 = 0; c0 < C; c0 += 8) {
      uint64_t v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = sc.cand[c0 + q];
#pragma unroll
      for (int q = 0; q < 8; ++q) rank += v[q] > mine ? 1 : 0;
    }
    if (c < C && rank < k) {
      sc.sel_i[rank] = (int)(0xFFFFFFFFu - (uint32_t)mine);
      sc.sel_s[rank] = ms;
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const float sv = lane < k ? sc.sel_s[min(lane, 63)] : 0.0f;
  const int si = sc.sel_i[min(lane, 31)];
  const float ssum = wave_sum_bcast(sv);
  if (lane < k) {
    out_idx[lane] = si;
    out_w[lane] = sv * (rsc * __builtin_amdgcn_rcpf(ssum));
  }
}

// The same for logits and bias in LDS (lane l takes experts l, l+64, ...).
template <int JMAX>
__device__ __forceinline__ void wave_route_row(const float* Lrow, const float* bias_lds, int E, int k,
                                               float routed_scale, int32_t* __restrict__ out_idx,
                                               float* __restrict__ out_w, WaveRouteScratch<JMAX>& sc) {
  const int lane = threadIdx.x & 63;
  float L[JMAX], bv[JMAX];
#pragma unroll
  for (int j = 0; j < JMAX; ++j) {
    const int e = min(lane + 64 * j, E - 1);
    L[j] = Lrow[e];
    bv[j] = bias_lds[e];
  }
  wave_route_regs<JMAX>(L, bv, E, k, routed_scale, out_idx, out_w, sc);
}

}  // namespace nvr
