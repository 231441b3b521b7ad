"""Round-to-nearest-even into narrow binary floating-point formats (TEST INFRASTRUCTURE ONLY).

Written from the format definitions, not from any library:

  OCP 8-bit e5m2 ("bf8"): 1 sign, 5 exponent bits (bias 15), 2 fraction bits;
      subnormals down to 2^-16, largest finite 57344, exponent field 31 holds
      inf (fraction 0) and NaN.  The fused-attention page [FA-A, _attn_fwd_inner]
      casts the softmax weights to this format before P.V when V is stored in it.
  bfloat16: 1 sign, 8 exponent bits (bias 127), 7 fraction bits.
  IEEE binary16: 1 sign, 5 exponent bits (bias 15), 10 fraction bits.

Rounding is to nearest, ties to even, starting from the exact fp64 value;
results too large for the format become +-inf (non-saturating conversion).
All arithmetic below is exact in fp64: scaling by powers of two and np.rint
(which rounds half to even) on integers below 2^53.
"""
import numpy as np


def round_to_format(x, frac_bits, emin, max_finite):
    """Round fp64 values to the nearest value of a binary format (ties to even).

    frac_bits  -- number of stored fraction bits
    emin       -- exponent of the smallest normal number
    max_finite -- largest finite magnitude; larger rounded results become inf
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    finite_nz = np.isfinite(a) & (a > 0)
    safe = np.where(finite_nz, a, 1.0)
    # a = f * 2^E with f in [0.5, 1), so the unbiased exponent of a is E - 1.
    _, E = np.frexp(safe)
    e = np.maximum(E.astype(np.int64) - 1, emin)          # subnormals share emin's quantum
    quantum = np.ldexp(1.0, (e - frac_bits).astype(np.int64))
    y = np.rint(safe / quantum) * quantum                   # exact: power-of-two scaling
    y = np.where(y > max_finite, np.inf, y)
    y = np.where(finite_nz, y, a)                           # 0, inf and NaN pass through
    return np.copysign(y, x)


E5M2_MAX = 57344.0


def round_e5m2(x):
    return round_to_format(x, 2, -14, E5M2_MAX)


def round_bf16(x):
    return round_to_format(x, 7, -126, (2.0 - 2.0 ** -7) * 2.0 ** 127)


def round_f16(x):
    return round_to_format(x, 10, -14, 65504.0)


def e5m2_decode(codes):
    """uint8 codes -> fp64 values, from the field layout."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(b >> 7, -1.0, 1.0)
    ef = (b >> 2) & 31
    m = (b & 3).astype(np.float64)
    normal = np.ldexp(1.0 + m / 4.0, (ef - 15).astype(np.int64))
    sub = np.ldexp(m / 4.0, -14)
    special = np.where(m == 0, np.inf, np.nan)
    mag = np.where(ef == 0, sub, np.where(ef == 31, special, normal))
    return s * mag


def e5m2_encode(x):
    """fp64 values -> uint8 codes (rounds first; NaN -> 0x7F / 0xFF)."""
    y = round_e5m2(x)
    sign = np.signbit(y).astype(np.int64) << 7
    a = np.abs(y)
    out = np.zeros(a.shape, dtype=np.int64)
    nan = np.isnan(a)
    inf = np.isinf(a)
    sub = (a < 2.0 ** -14) & ~nan
    normal = ~(nan | inf | sub)
    out = np.where(sub, np.rint(np.where(sub, a, 0.0) / 2.0 ** -16).astype(np.int64), out)
    safe = np.where(normal, a, 1.0)
    _, E = np.frexp(safe)
    e = E.astype(np.int64) - 1
    mant = np.rint((safe / np.ldexp(1.0, e) - 1.0) * 4.0).astype(np.int64)
    out = np.where(normal, ((e + 15) << 2) | mant, out)
    out = np.where(inf, 31 << 2, out)
    out = np.where(nan, (31 << 2) | 3, out)
    return (out | sign).astype(np.uint8)
