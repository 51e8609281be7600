"""Exact two-term E4M3 split of BF16 query rows (float64 oracle).

Test infrastructure only (see ``oracle/__init__``).

The query is BF16 ("[ROCm][MLA][DCP] Support causal multi-token
verification", the workloads' BF16 Q; "Context Parallel Guide (PCP & DCP)",
"How it works" item 4 for the FP8 cache it meets).  To multiply it against
an FP8 E4M3 cache on the FP8 matrix units without losing precision, each
head-row q is written as

    q = (hi + lo) / 2^k

with hi and lo E4M3 codes and 2^k a power of two per row.  This is
arithmetic, not quantisation: a BF16 value has 8 significant bits, E4M3 has
4, so once x = q * 2^k is rounded to the nearest E4M3 value hi (ties to even,
OCP "FN" E4M3 as in ``formats``), the residual x - hi has at most 4
significant bits and its lowest bit sits 7 binades below x's leading bit.  It
is therefore an E4M3 value itself whenever that lowest bit is at or above
the subnormal step 2^-9, i.e. whenever |x| >= 2^-2, and then hi + lo = x
exactly.  Smaller elements are off by at most half the subnormal step,
2^-10, in x units.

k is the largest integer with max|q| * 2^k <= 448 (the largest finite E4M3
magnitude), so the largest element uses the whole range; an all-zero row
takes k = 0.  With k maximal, every element of magnitude >= max|q| / 896 is
split exactly.
"""
import numpy as np

from .formats import E4M3_TABLE

E4M3_MAX = 448.0

#: finite non-negative codes and their values, in increasing order
_POS_CODES = np.arange(0x7F, dtype=np.int64)   # 0x00 .. 0x7E (0x7F is NaN)
_POS_VALUES = E4M3_TABLE[_POS_CODES]


def e4m3_rne(x) -> np.ndarray:
    """float64 values (|x| <= 448) -> E4M3 codes, round to nearest, ties to the
    code with an even mantissa, by search over the table of finite codes."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_rne takes finite |x| <= 448")
    a = np.abs(x).ravel()
    # index of the largest table value <= a, and the next one up
    lo_i = np.searchsorted(_POS_VALUES, a, side="right") - 1
    hi_i = np.minimum(lo_i + 1, len(_POS_VALUES) - 1)
    d_lo = a - _POS_VALUES[lo_i]
    d_hi = _POS_VALUES[hi_i] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[lo_i] & 1 == 1) & (hi_i != lo_i))
    code = np.where(pick_hi, _POS_CODES[hi_i], _POS_CODES[lo_i])
    # sign-magnitude: the sign is kept, also on a zero result (IEEE-style)
    sign = np.signbit(x.ravel()).astype(np.int64) << 7
    return (code | sign).astype(np.uint8).reshape(x.shape)


def row_exponent(amax: float) -> int:
    """Largest k with amax * 2^k <= 448 (0 for amax == 0)."""
    if amax == 0.0:
        return 0
    k = int(np.floor(np.log2(E4M3_MAX / amax)))
    # guard the floor against rounding in log2
    while amax * 2.0 ** (k + 1) <= E4M3_MAX:
        k += 1
    while amax * 2.0 ** k > E4M3_MAX:
        k -= 1
    return k


def split_rows(q: np.ndarray):
    """q [R, D] float64 (BF16 values) -> (hi codes [R, D] uint8, lo codes
    [R, D] uint8, inv_scale [R] float64 = 2^-k per row)."""
    q = np.asarray(q, dtype=np.float64)
    R = q.shape[0]
    hi = np.zeros(q.shape, dtype=np.uint8)
    lo = np.zeros(q.shape, dtype=np.uint8)
    inv = np.zeros(R, dtype=np.float64)
    for r in range(R):
        k = row_exponent(float(np.max(np.abs(q[r]))) if q.shape[1] else 0.0)
        x = q[r] * 2.0 ** k
        hi[r] = e4m3_rne(x)
        lo[r] = e4m3_rne(x - E4M3_TABLE[hi[r]])
        inv[r] = 2.0 ** -k
    return hi, lo, inv


def join_rows(hi, lo, inv) -> np.ndarray:
    """Inverse of ``split_rows`` (exact for elements the split keeps exactly)."""
    return (E4M3_TABLE[np.asarray(hi)] + E4M3_TABLE[np.asarray(lo)]) * np.asarray(inv)[:, None]


def quantize_rows(q: np.ndarray) -> np.ndarray:
    """The FP8 query: each element as its one nearest E4M3 value at the row's
    scale 2^-k (the hi term of ``split_rows`` alone), as float64.  This is the
    quantised query of "Context Parallel Guide (PCP & DCP)", "How it works"
    item 4 (decode gathers an FP8 query for an FP8 cache), with a power-of-two
    scale per head-row."""
    q = np.asarray(q, dtype=np.float64)
    hi, _, inv = split_rows(q.reshape(-1, q.shape[-1]))
    return (E4M3_TABLE[hi] * inv[:, None]).reshape(q.shape)
