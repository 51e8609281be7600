"""Pins of the exchange oracle: the LSE halves round trip, the message layout
(pack -> all-to-all -> unpack then merge equals the direct rank merge), the
per-head projection against a brute-force loop, and the commutation of the
projection with the merge that "Context Parallel Guide (PCP & DCP)",
enable_project_before_merge, states."""
import numpy as np
import pytest

from oracle import attention as A
from oracle import exchange as X
from oracle import formats


def test_lse_halves_round_trip_exact():
    special = np.array([-np.inf, np.inf, np.nan, 0.0, -0.0, 1e-40, -3.5e-39, 1.0, -123.456, 3.4e38],
                       dtype=np.float32)
    rnd = np.random.default_rng(0).standard_normal(1000).astype(np.float32) * 50
    for v in (special, rnd):
        lo, hi = X.lse_halves(v)
        back = X.join_halves(lo, hi)
        assert np.array_equal(back.view(np.uint32), v.view(np.uint32))
        # the high half is the value's top 16 bits: sign, exponent, 7 mantissa bits
        assert np.array_equal(hi, (v.view(np.uint32) >> 16).astype(np.uint16))


def _rank_partials(seed, W, T, H, D=512):
    rng = np.random.default_rng(seed)
    out = rng.standard_normal((W, T, H, D)).astype(np.float32)
    bits = (out.view(np.uint32) >> 16).astype(np.uint16)     # bf16 patterns (truncated; any pattern works)
    lse = (rng.standard_normal((W, T, H)) * 3).astype(np.float32)
    lse[0, 0, :] = -np.inf                                     # an empty (token, rank)
    lse[:, 1, 0] = -np.inf                                     # a row empty on every rank
    return bits, lse


@pytest.mark.parametrize("W,T,H,D", [(2, 3, 4, 512), (8, 5, 16, 128), (4, 2, 8, 64)])
def test_pack_exchange_combine_is_the_rank_merge(W, T, H, D):
    bits, lse = _rank_partials(W * 10 + T, W, T, H, D)
    sends = [X.a2a_pack(bits[r], lse[r], W) for r in range(W)]
    recvs = X.all_to_all(sends)
    direct_o, direct_l = A.merge_ranks(formats.decode_bf16(bits), lse.astype(np.float64))
    Hl = H // W
    for p in range(W):
        ob, ll = X.unpack(recvs[p])
        o, l = A.merge_ranks(formats.decode_bf16(ob), ll.astype(np.float64))
        heads = slice(p * Hl, (p + 1) * Hl)
        assert np.array_equal(o, direct_o[:, heads]) and np.array_equal(l, direct_l[:, heads])
        assert np.all(recvs[p][..., D + 2:] == 0)


def test_project_heads_brute_force():
    rng = np.random.default_rng(3)
    T, H, DV = 3, 2, 5
    o = rng.standard_normal((T, H, 512))
    w = rng.standard_normal((H, 512, DV))
    ref = np.zeros((T, H, DV))
    for t in range(T):
        for h in range(H):
            for n in range(DV):
                ref[t, h, n] = sum(o[t, h, k] * w[h, k, n] for k in range(512))
    assert np.abs(X.project_heads(o, w) - ref).max() < 1e-10


@pytest.mark.parametrize("W", [1, 2, 8])
def test_projection_commutes_with_merge(W):
    rng = np.random.default_rng(W)
    T, H, DV = 4, 8, 128
    o = rng.standard_normal((W, T, H, 512))
    lse = rng.standard_normal((W, T, H)) * 2
    lse[0, 1, 3] = -np.inf
    w = rng.standard_normal((H, 512, DV)) / np.sqrt(512)
    mo, ml = A.merge_ranks(o, lse)
    po, pl = A.merge_ranks(np.stack([X.project_heads(o[r], w) for r in range(W)]), lse)
    assert np.abs(po - X.project_heads(mo, w)).max() < 1e-12
    assert np.array_equal(pl, ml)
