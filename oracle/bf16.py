"""Exact bfloat16 <-> float64 conversion (oracle; test infrastructure only).

bfloat16 is the top half of an IEEE binary32: 1 sign bit, 8 exponent bits,
7 stored mantissa bits.  The pages never fix a precision; bf16 storage with
float32 accumulation is the reading taken here for the attention path.

The conversion float64 -> bf16 here is written from the definition of
round-to-nearest-even, not from a bit trick: scale |x| onto the integer grid
of bf16 values of its binade, round half to even with ``numpy.rint``, scale
back.  It converts directly (no float32 detour, which would round twice).
"""

import numpy as np

# Smallest normal exponent of bf16 (same exponent field as binary32).
_EMIN = -126
# Stored mantissa bits.
_MANT = 7
# Largest finite bf16 magnitude: (2 - 2^-7) * 2^127.
BF16_MAX = (2.0 - 2.0 ** -_MANT) * 2.0 ** 127


def bits_to_f64(bits):
    """bf16 bit patterns (uint16 array) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns widen to NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_f64(x):
    """Round float64 values to the nearest bf16 value (ties to even), as float64.

    Finite results are bf16 values held exactly in float64; magnitudes that
    round beyond BF16_MAX become +-inf, as IEEE round-to-nearest requires.
    NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0.0)
    a = np.abs(x[fin])
    # a = m * 2**E with m in [0.5, 1)  =>  floor(log2 a) = E - 1  (exact).
    _, E = np.frexp(a)
    e = np.maximum(E - 1, _EMIN)           # binade exponent, clamped for subnormals
    ulp = np.ldexp(1.0, e - _MANT)         # spacing of bf16 values in that binade
    q = a / ulp                            # exact: division by a power of two
    r = np.rint(q) * ulp                   # rint rounds halves to even
    r = np.where(r > BF16_MAX, np.inf, r)  # overflow of the rounded value
    out[fin] = np.copysign(r, x[fin])
    return out


def f64_to_bits(x):
    """float64 -> bf16 bit patterns (uint16), round to nearest even."""
    r = round_f64(x)
    # Every rounded value (and +-0, +-inf) is exact in float32; bf16 is its top half.
    u = r.astype(np.float32).view(np.uint32)
    bits = (u >> np.uint32(16)).astype(np.uint16)
    # Canonical quiet NaN for NaN inputs.
    bits = np.where(np.isnan(r), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)
