"""Pins of the two-term E4M3 split of BF16 query rows (oracle/qsplit.py)."""
import numpy as np
import pytest
import torch

from oracle import formats, qsplit


def _finite_codes():
    return np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_rne_round_trips_every_finite_code():
    codes = _finite_codes()
    assert np.array_equal(qsplit.e4m3_rne(formats.E4M3_TABLE[codes]), codes)


def test_rne_ties_go_to_even_mantissa():
    vals = formats.E4M3_TABLE[np.arange(0x7F)]
    mids = (vals[:-1] + vals[1:]) / 2            # exact in float64
    got = qsplit.e4m3_rne(mids)
    assert np.all(got & 1 == 0)                   # the even neighbour
    assert np.all((got == np.arange(0x7E)) | (got == np.arange(1, 0x7F)))
    # just off the midpoint goes to the nearer neighbour
    eps = np.diff(vals) * 1e-6
    assert np.array_equal(qsplit.e4m3_rne(mids - eps), np.arange(0x7E))
    assert np.array_equal(qsplit.e4m3_rne(mids + eps), np.arange(1, 0x7F))


def test_rne_matches_library_conversion():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(-448, 448, 50000), rng.normal(0, 0.02, 50000),
                        (formats.E4M3_TABLE[np.arange(0x7F)][:-1] + formats.E4M3_TABLE[np.arange(1, 0x7F)]) / 2])
    ref = torch.tensor(x, dtype=torch.float64).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(qsplit.e4m3_rne(x), ref)


def test_rne_rejects_out_of_range():
    with pytest.raises(ValueError):
        qsplit.e4m3_rne(np.array([449.0]))
    with pytest.raises(ValueError):
        qsplit.e4m3_rne(np.array([np.nan]))


@pytest.mark.parametrize("amax", [1.0, 448.0, 447.9, 448.1, 3.5, 0.875, 0.8751, 1e-3, 2.0 ** -20, 1e5])
def test_row_exponent_is_the_largest_fitting_power(amax):
    k = qsplit.row_exponent(amax)
    assert amax * 2.0 ** k <= 448.0 < amax * 2.0 ** (k + 1)


def test_every_bf16_value_in_range_splits_exactly():
    # brute force over every BF16 value with 2^-2 <= |x| <= 448 (both signs)
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = formats.decode_bf16(bits)
    x = x[np.isfinite(x) & (np.abs(x) >= 0.25) & (np.abs(x) <= 448.0)]
    assert len(x) == 2 * (10 * 128 + 97)   # binades 2^-2 .. 2^7 whole, [256, 448] in steps of 2
    hi = qsplit.e4m3_rne(x)
    lo = qsplit.e4m3_rne(x - formats.E4M3_TABLE[hi])
    assert np.array_equal(formats.E4M3_TABLE[hi] + formats.E4M3_TABLE[lo], x)


def _bf16_rows(rng, R, D, wide=False):
    v = rng.standard_normal((R, D)).astype(np.float32)
    if wide:
        v *= np.exp2(rng.uniform(-12, 4, (R, D))).astype(np.float32)
    bits = (v.view(np.uint32) + 0x7FFF + ((v.view(np.uint32) >> 16) & 1)) >> 16
    return formats.decode_bf16(bits.astype(np.uint16))


@pytest.mark.parametrize("wide", [False, True])
def test_split_rows_reconstruct(wide):
    rng = np.random.default_rng(11 + wide)
    q = _bf16_rows(rng, 64, 576, wide)
    q[3] = 0.0                                     # an all-zero row
    hi, lo, inv = qsplit.split_rows(q)
    back = qsplit.join_rows(hi, lo, inv)
    x_abs = np.abs(q) / inv[:, None]               # |q| * 2^k
    big = x_abs >= 0.25
    assert np.array_equal(back[big], q[big])
    assert np.all(np.abs(back - q)[~big] <= (2.0 ** -10) * np.broadcast_to(inv[:, None], q.shape)[~big])
    assert inv[3] == 1.0 and not hi[3].any() and not lo[3].any()
    # the scale is maximal: the row's largest element lands in [224, 448]
    amax = np.abs(q).max(axis=1)
    nz = amax > 0
    assert np.all(amax[nz] / inv[nz] <= 448.0) and np.all(amax[nz] / inv[nz] > 224.0)


def test_quantize_rows_error_bound_and_idempotence():
    rng = np.random.default_rng(21)
    q = _bf16_rows(rng, 32, 576, wide=True)
    qq = qsplit.quantize_rows(q)
    inv = np.array([2.0 ** -qsplit.row_exponent(float(np.abs(r).max())) for r in q])
    x = np.abs(q) / inv[:, None]
    normal = x >= 2.0 ** -6
    # nearest E4M3: half an ulp, 2^-4 of the value in the normal range, 2^-10 (x units) below
    assert np.all(np.abs(qq - q)[normal] <= 2.0 ** -4 * np.abs(q)[normal])
    assert np.all((np.abs(qq - q) / inv[:, None])[~normal] <= 2.0 ** -10)
    assert np.array_equal(qsplit.quantize_rows(qq), qq)


def test_quantize_rows_matches_library_conversion():
    rng = np.random.default_rng(22)
    q = _bf16_rows(rng, 16, 576)
    k = np.array([qsplit.row_exponent(float(np.abs(r).max())) for r in q])
    x = q * np.exp2(k)[:, None]
    lib = torch.tensor(x, dtype=torch.float64).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(qsplit.quantize_rows(q), lib * np.exp2(-k)[:, None])
