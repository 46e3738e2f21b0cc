"""Exact decoding of floating-point bit patterns to float64.  TEST INFRASTRUCTURE ONLY.

The oracle reads the raw bits of q, K and V and widens them to float64 itself,
field by field (sign, biased exponent, fraction), so that no conversion routine
is shared with the GPU path.  Every binary16 and bfloat16 value is exactly
representable in float64, so the decode is exact.

Formats (IEEE 754-2008 binary16; bfloat16 = the top 16 bits of binary32):

* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
* binary32: 1 sign bit, 8 exponent bits (bias 127), 23 fraction bits.

The pages fix the element sizes only (FP16 = 2 bytes, FP8 = 1 byte: "vLLM explained",
section on block size); the formats themselves are the IEEE / bfloat16 definitions.
"""

import numpy as np

F32, F16, BF16 = 0, 1, 2
ELEM_BYTES = {F32: 4, F16: 2, BF16: 2}
_LAYOUT = {
    # dtype: (total bits, exponent bits, fraction bits, bias)
    F16: (16, 5, 10, 15),
    BF16: (16, 8, 7, 127),
    F32: (32, 8, 23, 127),
}


def decode(dtype, bits):
    """Widen an array of raw bit patterns of format ``dtype`` to float64, exactly.

    ``bits`` is an unsigned integer array (uint16 for F16/BF16, uint32 for F32) or,
    for F32, a float32 array (reinterpreted).  Subnormals, signed zeros, infinities
    and NaNs are decoded by their definitions.
    """
    total, ebits, fbits, bias = _LAYOUT[dtype]
    b = np.asarray(bits)
    if dtype == F32 and b.dtype == np.float32:
        b = b.view(np.uint32)
    b = b.astype(np.int64)
    sign = np.where((b >> (total - 1)) & 1, -1.0, 1.0)
    exp = (b >> fbits) & ((1 << ebits) - 1)
    frac = (b & ((1 << fbits) - 1)).astype(np.float64)
    emax = (1 << ebits) - 1
    normal = sign * np.ldexp(1.0 + frac / float(1 << fbits), (exp - bias).astype(np.int64))
    subnormal = sign * np.ldexp(frac / float(1 << fbits), 1 - bias)
    special = np.where(frac == 0, sign * np.inf, np.nan)
    out = np.where(exp == 0, subnormal, np.where(exp == emax, special, normal))
    return out.astype(np.float64)
