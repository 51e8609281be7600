"""Exact decode of the cache and query number formats to float64.

Test infrastructure only (see ``oracle/__init__``).

* BF16: the upper 16 bits of an IEEE-754 binary32.  Decoding is exact:
  shift the pattern into the high half of a binary32 and widen.
* FP8 E4M3 as defined in the OCP 8-bit Floating Point Specification (OFP8),
  the "FN" variant without infinities: 1 sign bit, 4 exponent bits with bias
  7, 3 mantissa bits.  Exponent field 0 encodes subnormals m/8 * 2^-6; the
  all-ones pattern S.1111.111 is NaN; every other code is normal,
  (1 + m/8) * 2^(e-7).  The largest finite magnitude is 448.  The pages state
  that DCP keeps one per-tensor FP8 scale for the whole latent cache
  ("Context Parallel Guide (PCP & DCP)", CLI table row ``--kv-cache-dtype
  fp8`` and "How it works" item 4); the stored value is code * scale.
"""
import numpy as np


def _e4m3_code_value(code: int) -> float:
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return float("nan")
    if exp_field == 0:
        return sign * (mant / 8.0) * 2.0 ** -6
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


#: value of each of the 256 E4M3 codes, built from the bit fields above
E4M3_TABLE = np.array([_e4m3_code_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(codes, scale: float = 1.0) -> np.ndarray:
    """uint8 E4M3 codes (any shape) -> float64 values times ``scale``."""
    codes = np.asarray(codes, dtype=np.uint8)
    return E4M3_TABLE[codes] * np.float64(scale)


def decode_bf16(bits) -> np.ndarray:
    """uint16 BF16 bit patterns (any shape) -> float64 (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def decode_cache(raw, kv_format: str, scale: float = 1.0) -> np.ndarray:
    """Decode latent-cache rows stored as ``kv_format`` ('bf16' or 'fp8_e4m3')."""
    if kv_format == "bf16":
        return decode_bf16(raw) * np.float64(scale)
    if kv_format == "fp8_e4m3":
        return decode_e4m3(raw, scale)
    raise ValueError(f"unknown cache format {kv_format!r}")


# ------------------------------------------------------------------ BF16 rounding
#
# BF16 is the upper half of an IEEE-754 binary32: the same 8-bit exponent
# (normal range 2^-126 .. 2^128, subnormals with the fixed quantum 2^-133) and
# 8 significant bits (7 stored).  A real in [2^E, 2^(E+1)) with E >= -126 is
# therefore stored to a multiple of 2^(E-7); below 2^-126 the multiple is 2^-133.
# Round-to-nearest-even picks the nearest multiple and breaks exact ties to the
# even one; a magnitude at or above (2 - 2^-8) 2^127 (half a step past the
# largest finite value) becomes infinity.

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
_BF16_OVERFLOW = (2.0 - 2.0 ** -8) * 2.0 ** 127


def bf16_quantum(x) -> np.ndarray:
    """Spacing of the BF16 values around |x| (the step of the binade holding x)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    ax = np.where(np.isfinite(ax), ax, 1.0)   # non-finite inputs: any quantum (unused)
    _, ex = np.frexp(ax)                      # ax = m 2^ex, m in [0.5, 1); frexp(0) = (0, 0)
    e = np.where(ax < 2.0 ** -126, -126, np.maximum(ex.astype(np.int64) - 1, -126))
    return np.ldexp(1.0, e - 7)


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest BF16 value, ties to even (float64 out).

    A single rounding of the given value: a float64 input that is not a
    binary32 value is not first rounded to binary32.
    """
    x = np.asarray(x, dtype=np.float64)
    q = bf16_quantum(x)
    with np.errstate(invalid="ignore", over="ignore"):
        r = np.round(x / q) * q               # x / q is exact (q a power of two); np.round ties to even
        r = np.where(np.abs(x) >= _BF16_OVERFLOW, np.copysign(np.inf, x), r)
        r = np.where(np.isnan(x), np.nan, r)
        r = np.where(np.isinf(x), x, r)
    return np.copysign(np.abs(r), x)          # keep the sign of zero results


def bf16_rounding_interval(v):
    """The closed interval of reals that round to the finite BF16 value ``v``.

    Its half-widths are half the steps to the neighbouring BF16 values: below a
    power of two the step below is half the step above.
    """
    v = np.asarray(v, dtype=np.float64)
    av = np.abs(v)
    up = bf16_quantum(v)                      # step to the next value away from zero
    _, ex = np.frexp(av)
    at_pow2 = (av == np.ldexp(0.5, ex)) & (av > np.ldexp(1.0, -126))
    down = np.where(at_pow2, up / 2, up)      # step to the next value towards zero
    down = np.where(av == 0, up, down)
    lo_mag, hi_mag = av - down / 2, av + up / 2
    lo = np.where(v < 0, -hi_mag, np.where(v == 0, -up / 2, lo_mag))
    hi = np.where(v < 0, -lo_mag, hi_mag)
    return lo, hi


def bf16_step(v, k: int) -> np.ndarray:
    """The BF16 value ``k`` positions from the BF16 value ``v`` along the real line.

    BF16 patterns are sign-magnitude: on the magnitude field (15 bits) the order
    of the finite values is the integer order, so a signed position is
    +-magnitude (both zeros at 0).
    """
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.int64)
    mag = bits & 0x7FFF
    pos = np.where(bits >> 15 == 1, -mag, mag) + k
    out = (np.where(pos < 0, 0x8000, 0) | np.abs(pos)).astype(np.uint16)
    return decode_bf16(out)
