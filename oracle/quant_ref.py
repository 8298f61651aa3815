"""Runtime NVFP4 quantization of a bf16 tensor, written as its plain definition.

TEST INFRASTRUCTURE (CPU oracle); see the package docstring.

Steps, in the order the method takes them:

1. amax = max |x| over the whole tensor handed to one call (one global
   scale per call: the flattened single-launch quantizer with a device-only
   global scale, commit df05289d, dsv4/layers/grouped_linear.py, paragraph
   on replacing the host-side gsa).
2. gsa = amax / (6 * 448), one IEEE binary32 division by 2688 (commit
   04cf8ca8, dsv4/layers/router.py, the runtime-gsa fix). 6 is the largest
   E2M1 magnitude, 448 the largest E4M3 block scale, so x/gsa <= 2688 up to
   the single rounding of gsa.
3. For every row and every 16-element block along D, the block scale is
   the E4M3 value nearest to bmax / (6 * gsa), saturating at 448.
4. Every element's code is the E2M1 value nearest to |x| / (gsa * S), with
   the sign bit of x kept (so -0.0 and small negatives give code 0x8). A
   zero block scale gives magnitude 0.
5. Two codes per byte, the even element in the low nibble; codes are
   [rows, D/2] and scales [rows, D/16], both row-major.

gsa == 0 (an all-zero tensor, or a zero override) makes every scale byte
0x00 and every code sign-only.

All roundings are decided in float64 on quotients of exactly represented
operands (bf16 x, fp32 gsa, E4M3 S: gsa*S and 6*gsa are exact in float64);
``formats.round_to_grid`` explains why that decides the exact real quotient.
``quantize_exact_scalar`` is the same definition with exact rationals.
"""

from fractions import Fraction

import numpy as np

from .formats import E2M1_GRID, E4M3_GRID, e4m3_decode, round_to_grid, round_to_grid_exact

BLOCK = 16
GSA_DIVISOR = np.float32(6.0 * 448.0)  # 2688, exact in fp32


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16 array) -> exact float64 values."""
    bits = np.asarray(bits, dtype=np.uint16)
    f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def amax_ref(bits):
    """max |x| over every element (float64, exact)."""
    v = bf16_bits_to_f64(bits)
    return float(np.max(np.abs(v))) if v.size else 0.0


def gsa_ref(amax):
    """Global scale: fp32(amax) / fp32(2688) as one IEEE binary32 division."""
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        return np.float32(amax) / GSA_DIVISOR


def block_scale_bytes(bmax, gsa):
    """E4M3 byte nearest to bmax / (6*gsa) for each block max (float64 array)."""
    bmax = np.asarray(bmax, dtype=np.float64)
    g = float(gsa)
    if g == 0.0:
        return np.zeros(bmax.shape, dtype=np.uint8)
    q = bmax / (6.0 * g)  # 6*g exact in float64
    return round_to_grid(q, E4M3_GRID).astype(np.uint8)


def element_codes(x, scale_vals, gsa, signbits):
    """4-bit codes: E2M1 nearest to |x| / (gsa*S) with the sign bit of x.

    ``x``/``scale_vals``/``signbits`` broadcast elementwise; a zero scale (or
    zero gsa) gives magnitude 0.
    """
    x = np.asarray(x, dtype=np.float64)
    s = np.broadcast_to(np.asarray(scale_vals, dtype=np.float64), x.shape)
    g = float(gsa)
    denom = g * s  # exact in float64
    mag = np.zeros(x.shape, dtype=np.int64)
    nz = denom != 0.0
    mag[nz] = round_to_grid(np.abs(x[nz]) / denom[nz], E2M1_GRID)
    sign = np.broadcast_to(np.asarray(signbits, dtype=np.int64), x.shape)
    return ((sign << 3) | mag).astype(np.uint8)


def pack_codes(codes):
    """[rows, D] 4-bit codes -> [rows, D/2] bytes, even element in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_codes(packed):
    """[rows, D/2] bytes -> [rows, D] 4-bit codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def quantize_ref(bits, gsa_override=None):
    """Quantize a bf16 tensor [rows, D] (uint16 bit patterns).

    Returns ``(codes [rows, D/2] uint8, scales [rows, D/16] uint8, gsa float32)``.
    ``gsa_override`` replaces the runtime global scale (a test hook that
    reproduces the static-scale saturation the runtime fix removed).
    """
    bits = np.asarray(bits, dtype=np.uint16)
    rows, d = bits.shape
    assert d % BLOCK == 0, "D must be a multiple of 16"
    x = bf16_bits_to_f64(bits)
    if gsa_override is None:
        gsa = gsa_ref(amax_ref(bits))
    else:
        gsa = np.float32(gsa_override)
    xb = x.reshape(rows, d // BLOCK, BLOCK)
    bmax = np.max(np.abs(xb), axis=2) if d else np.zeros((rows, 0))
    sbytes = block_scale_bytes(bmax, gsa)
    svals = E4M3_GRID[sbytes.astype(np.int64)]
    signs = (bits.reshape(rows, d // BLOCK, BLOCK) >> 15).astype(np.int64)
    codes = element_codes(xb, svals[:, :, None], gsa, signs).reshape(rows, d)
    return pack_codes(codes), sbytes, np.float32(gsa)


def quantize_exact_scalar(bits, gsa_override=None):
    """Exact-rational twin of ``quantize_ref`` (element by element; tiny inputs).

    Every quotient is a ``Fraction`` and every rounding a brute-force nearest
    search, so it shares only the format definitions with ``quantize_ref``.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    rows, d = bits.shape
    vals = bf16_bits_to_f64(bits)
    if gsa_override is None:
        amax = max((abs(float(v)) for v in vals.ravel()), default=0.0)
        gsa = np.float32(amax) / GSA_DIVISOR
    else:
        gsa = np.float32(gsa_override)
    g = Fraction(float(gsa))
    codes = np.zeros((rows, d), dtype=np.uint8)
    scales = np.zeros((rows, d // BLOCK), dtype=np.uint8)
    for r in range(rows):
        for b in range(d // BLOCK):
            blk = [Fraction(float(v)) for v in vals[r, b * BLOCK:(b + 1) * BLOCK]]
            bmax = max(abs(v) for v in blk)
            sbyte = 0 if g == 0 else round_to_grid_exact(bmax / (6 * g), E4M3_GRID)
            scales[r, b] = sbyte
            s = Fraction(e4m3_decode(sbyte))
            for i, v in enumerate(blk):
                sign = int(bits[r, b * BLOCK + i]) >> 15
                mag = 0 if (g == 0 or s == 0) else round_to_grid_exact(abs(v) / (g * s), E2M1_GRID)
                codes[r, b * BLOCK + i] = (sign << 3) | mag
    return pack_codes(codes), scales, np.float32(gsa)


def dequant_ref(codes_packed, scales, gscale):
    """Exact real values v = val(code) * val(S) * gscale, float64 [rows, D]."""
    c = unpack_codes(codes_packed).astype(np.int64)
    mag = E2M1_GRID[c & 7]
    val = np.where((c & 8) != 0, -mag, mag)
    s = E4M3_GRID[np.asarray(scales, dtype=np.int64)]
    rows, d = val.shape
    v = val.reshape(rows, d // BLOCK, BLOCK) * s[:, :, None] * float(gscale)
    return v.reshape(rows, d)
