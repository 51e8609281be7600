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
