"""Explicit rounding functions used by the oracle (test infrastructure only).

Every function takes and returns float64 NumPy arrays whose values are exactly the
rounded results, so later FP64 arithmetic sees the same numbers a lower-precision
format would hold.

- ``fl32``: IEEE binary32, round-to-nearest-even (NumPy's float64→float32 cast).
- ``bf16``: bfloat16 (8 significant bits), round-to-nearest-even, overflow to ±inf.
- ``e4m3``: OCP FP8 E4M3FN (4 significant bits, exponent bias 7, subnormal spacing
  2^-9, largest finite 448), round-to-nearest-even.  Results above 448 in magnitude
  saturate to ±448.  The pages name the format ("FP8 E4M3 probability words",
  Phase 2B report, section "Exactness") without a rounding or overflow rule; RNE with
  saturation is the plainest reading and only matters at |x| >= 464, which the program
  never produces (its inputs are scaled to at most 448).
- ``rne``: round half to even to an integer (``numpy.rint``).
"""
import numpy as np

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
E4M3_MAX = 448.0


def fl32(x):
    """Round float64 values to the nearest binary32 value (ties to even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def _round_to_bits(x, sig_bits, min_exp):
    """Round to a binary grid with `sig_bits` significant bits and spacing >= 2**min_exp.

    For |x| in [2**(e-1), 2**e) the spacing of such a format is 2**(e - sig_bits); below
    the normal range the spacing is fixed at 2**min_exp (gradual underflow).  The
    scaled value x / spacing is exact in float64 (the spacing is a power of two), so a
    single numpy.rint performs the one round-half-even of the format.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    step = np.maximum(e - sig_bits, min_exp)
    return np.ldexp(np.rint(np.ldexp(x, -step)), step)


def bf16(x):
    """bfloat16 round-to-nearest-even; magnitudes that round past the largest finite go to inf."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        q = _round_to_bits(np.where(np.isfinite(x), x, 0.0), 8, -133)
        q = np.where(np.abs(q) > BF16_MAX, np.copysign(np.inf, x), q)
    return np.where(np.isfinite(x), q, x)


def e4m3(x):
    """OCP E4M3FN value of x: round-to-nearest-even, saturating at ±448."""
    x = np.asarray(x, dtype=np.float64)
    q = _round_to_bits(np.where(np.isnan(x), 0.0, x), 4, -9)
    q = np.clip(q, -E4M3_MAX, E4M3_MAX)
    return np.where(np.isnan(x), np.nan, q)


def e4m3_decode(codes):
    """Value of each E4M3FN byte (0x7F and 0xFF are NaN)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = (c >> 7) & 1
    exp = (c >> 3) & 15
    man = c & 7
    mag = np.where(exp == 0, man * 2.0 ** -9, (1.0 + man / 8.0) * np.ldexp(1.0, exp - 7))
    mag = np.where((exp == 15) & (man == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def e4m3_encode(values):
    """Byte code of values that already lie on the E4M3FN grid (e.g. outputs of e4m3)."""
    v = np.asarray(values, dtype=np.float64)
    sign = np.signbit(v).astype(np.int64)
    a = np.abs(v)
    _, e = np.frexp(a)  # a in [2**(e-1), 2**e)
    normal = a >= 2.0 ** -6
    exp_field = np.where(normal, e - 1 + 7, 0)
    man = np.where(normal, np.rint(np.ldexp(a, -(e - 1)) * 8.0) - 8.0, np.rint(a * 2.0 ** 9))
    code = (sign << 7) | (exp_field.astype(np.int64) << 3) | man.astype(np.int64)
    code = np.where(np.isnan(v), 0x7F, code)
    return code.astype(np.uint8)


def rne(x):
    """Round half to even to the nearest integer (as float64)."""
    return np.rint(np.asarray(x, dtype=np.float64))
