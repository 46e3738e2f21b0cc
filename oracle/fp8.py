"""FP8 (e4m3) KV-cache values: exact decoding and quantization.  TEST INFRASTRUCTURE ONLY.

An FP8 KV cache stores one byte per element, halving the cache's bytes ("vLLM explained",
jackchen890311.github.io, block-size section: FP8 is 1 byte per value; appendix:
quantization such as FP8 / INT8 shrinks the KV cache).  The pages do not fix the
8-bit format; this oracle follows the OCP 8-bit floating-point specification's E4M3
encoding (the format of the gfx950 conversion instructions):

* bit 7 sign, bits 6..3 exponent e (bias 7), bits 2..0 mantissa m;
* e = 0: subnormal, value m/8 * 2^-6;  e > 0: (1 + m/8) * 2^(e - 7);
* e = 15, m = 7 (0x7F / 0xFF) is NaN; there are no infinities; the largest finite
  magnitude is 448 (0x7E).

Quantization of a value x with a per-tensor scale s (the stored value times s
approximates x): y = x * (1/s) computed in float32 (one rounding, ``inv_scale`` is the
float32 reciprocal), clamped to [-448, 448] (NaN stays NaN), then rounded to the
nearest representable value with ties to an even mantissa.  The rounding here is a
search over the representable values, not a bit trick.
"""

import numpy as np

MAX = 448.0


def decode(bits):
    """float64 array of the values of uint8 codes ``bits`` (any shape)."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = s * val
    return np.where((e == 15) & (m == 7), np.nan, val)


# Non-negative finite codes 0x00 .. 0x7E in increasing value.
_CODES = np.arange(0x7F, dtype=np.uint8)
_VALUES = decode(_CODES)


def round_to_code(y):
    """Codes of float values ``y`` (already scaled and clamped): nearest, ties to even."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    hi = np.searchsorted(_VALUES, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _VALUES[lo]
    dhi = _VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((_CODES[hi] & 1) == 0))
    code = np.where(pick_hi, _CODES[hi], _CODES[lo]).astype(np.uint8)
    code = np.where(_VALUES[hi] == a, _CODES[hi], code)     # exact hits
    code = code | np.where(np.signbit(y), 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(y), np.where(np.signbit(y), 0xFF, 0x7F), code).astype(np.uint8)


def quantize(x, inv_scale):
    """Codes of float32 values ``x`` stored with float32 reciprocal scale ``inv_scale``."""
    y = np.asarray(x, dtype=np.float32) * np.float32(inv_scale)     # one float32 rounding
    y = np.where(np.isnan(y), y, np.clip(y, -MAX, MAX))
    return round_to_code(y)


def dequantize(bits, scale):
    """float64 values the cache holds: decoded code times the scale."""
    return decode(bits) * float(np.float32(scale))
