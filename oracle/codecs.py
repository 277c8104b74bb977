"""The oracle's own number codecs (test infrastructure; see the package header).

bfloat16 is IEEE binary32 with the low 16 bits of the significand dropped:
1 sign bit, 8 exponent bits (bias 127), 7 explicit significand bits. The pages
keep the KV cache, the activations and the q/k/v heads in this format (page
``code/alpamayo_tt/EXPERT_NOTES.md``, table "Layouts").

Decoding is exact. Encoding rounds a float64 value straight to the nearest
bfloat16 with ties to even (no intermediate float32 step, so there is no double
rounding), keeps subnormals, and overflows to infinity like IEEE round-to-
nearest.

e4m3 (OCP 8-bit floating point, the "fn" variant) is the cache format of the
fp8 variant of the step: the pages keep an 8-bit block-floating-point cache
as an option (page ``code/alpamayo_tt/expert.py``, ``TTExpert.__init__``, the
kv_cache dtype choice; page ``code/alpamayo_tt/EXPERT_NOTES.md``, the decode
timing row of the bfp8 cache), and the e4m3 format with one float32 scale
per (kv head, row) stands in for it here. Layout: 1 sign bit, 4 exponent bits
with bias 7, 3 explicit significand bits; exponent field 0 holds the
subnormals (m/8 * 2^-6); there are no infinities; S.1111.111 is NaN, so the
largest finite magnitude is 1.75 * 2^8 = 448.
"""
from __future__ import annotations

import numpy as np

_BF16_MIN_EXP = -126        # exponent of the smallest normal bfloat16
_BF16_MANT = 7              # explicit significand bits
_BF16_MAX = float(np.frombuffer(np.uint32(0x7F7F0000).tobytes(), np.float32)[0])


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16) as float64."""
    u = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even); return uint16 bits.

    For a finite nonzero x with binary exponent e (|x| in [2^e, 2^(e+1))), the
    bfloat16 spacing there is 2^(max(e, -126) - 7). x is divided by that
    spacing (exact: a power of two), rounded to an integer with ties to even
    (``np.rint``), and multiplied back (exact again). The result is a bfloat16
    value held in float64, so its float32 image is exact and its upper 16 bits
    are the encoding.
    """
    x = np.asarray(x, dtype=np.float64)
    shape = x.shape
    x = x.reshape(-1)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    nz = finite & (x != 0.0)
    xm = x[nz]
    _, e2 = np.frexp(np.abs(xm))          # |x| = f * 2^e2 with f in [0.5, 1)
    e = e2.astype(np.int64) - 1           # |x| in [2^e, 2^(e+1))
    spacing = np.ldexp(1.0, np.maximum(e, _BF16_MIN_EXP) - _BF16_MANT)
    r = np.rint(xm / spacing) * spacing
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, xm), r)
    out[nz] = r
    out[finite & (x == 0.0)] = x[finite & (x == 0.0)]   # keeps the sign of zero
    out[~finite] = x[~finite]
    f32 = out.astype(np.float32)          # exact: every value is a bfloat16
    bits = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    bits[nan] = np.uint16(0x7FC0)
    return bits.reshape(shape)


_E4M3_BIAS = 7
_E4M3_MANT = 3
_E4M3_MIN_EXP = 1 - _E4M3_BIAS   # exponent of the smallest normal: 2^-6
E4M3_MAX = 448.0


def e4m3_bits_to_f64(bits) -> np.ndarray:
    """Exact value of e4m3 codes (uint8) as float64; the two NaN codes give NaN."""
    c = np.asarray(bits).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> _E4M3_MANT) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 8.0, e - _E4M3_BIAS)
    sub = sign * np.ldexp(m / 8.0, _E4M3_MIN_EXP)
    v = np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def f64_to_e4m3_bits(x) -> np.ndarray:
    """Round to e4m3 with ties to even, saturating to +-448; return uint8 codes.

    Same scheme as the bfloat16 encoder: for |x| in [2^e, 2^(e+1)) the e4m3
    spacing is 2^(max(e, -6) - 3); x / spacing is rounded to an integer with
    ties to even and scaled back (both steps exact), then the magnitude is
    clipped to 448 (values that round past the largest finite code saturate
    instead of becoming NaN). The encoding is read off the rounded value. A
    NaN input gives 0x7F. Zeros, and values that round to zero, keep their sign.
    """
    x = np.asarray(x, dtype=np.float64)
    shape = x.shape
    x = x.reshape(-1)
    out = np.zeros(x.shape, dtype=np.uint8)
    nan = np.isnan(x)
    sign = np.where(np.signbit(x), 0x80, 0x00).astype(np.int64)
    ax = np.abs(np.where(nan, 0.0, x))
    r = np.zeros_like(ax)
    nz = ax > 0.0
    _, e2 = np.frexp(ax[nz])
    e = e2.astype(np.int64) - 1
    spacing = np.ldexp(1.0, np.maximum(e, _E4M3_MIN_EXP) - _E4M3_MANT)
    r[nz] = np.minimum(np.rint(ax[nz] / spacing) * spacing, E4M3_MAX)
    code = np.zeros(ax.shape, dtype=np.int64)
    pos = r > 0.0
    _, re2 = np.frexp(r[pos])
    re = re2.astype(np.int64) - 1                      # exponent of the rounded value
    is_norm = re >= _E4M3_MIN_EXP
    mant_n = np.rint((np.ldexp(r[pos], -re) - 1.0) * 8.0).astype(np.int64)
    mant_s = np.rint(np.ldexp(r[pos], -_E4M3_MIN_EXP) * 8.0).astype(np.int64)
    code[pos] = np.where(is_norm, ((re + _E4M3_BIAS) << _E4M3_MANT) | mant_n, mant_s)
    out[:] = (code | sign).astype(np.uint8)
    out[nan] = np.uint8(0x7F)
    return out.reshape(shape)
