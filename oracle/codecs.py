"""The oracle's own number codecs (test infrastructure; see the package header).

bfloat16 is IEEE binary32 with the low 16 bits of the significand dropped:
1 sign bit, 8 exponent bits (bias 127), 7 explicit significand bits. The pages
keep the KV cache, the activations and the q/k/v heads in this format (page
``code/alpamayo_tt/EXPERT_NOTES.md``, table "Layouts").

Decoding is exact. Encoding rounds a float64 value straight to the nearest
bfloat16 with ties to even (no intermediate float32 step, so there is no double
rounding), keeps subnormals, and overflows to infinity like IEEE round-to-
nearest.
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
