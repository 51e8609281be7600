"""Pins for ``oracle.formats`` and ``oracle.attention`` (CPU only).

Library routines (torch's float8/bfloat16 casts, scaled_dot_product_attention,
logsumexp) and identities the pages state (merge of exact per-rank softmaxes
equals global attention; natural LSE = ln 2 x base-2 LSE; empty ranks add
nothing) hold the float64 oracle in place.  ``test_pins_catch_mutants`` plants
plausible mistakes in the oracle and checks that a pin fails for each.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import formats, layout


# ---------------------------------------------------------------- formats ----

def test_e4m3_table_matches_torch_and_spec():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = formats.E4M3_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))
    # values fixed by the OCP E4M3 encoding: max normal, one, subnormals, NaN
    spec = {0x7E: 448.0, 0xFE: -448.0, 0x38: 1.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
            0x08: 2.0 ** -6, 0x00: 0.0, 0x40: 2.0, 0x3C: 1.5}
    for c, v in spec.items():
        assert formats.E4M3_TABLE[c] == v
    assert np.isnan(formats.E4M3_TABLE[0x7F]) and np.isnan(formats.E4M3_TABLE[0xFF])
    assert np.signbit(formats.E4M3_TABLE[0x80])


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    mine = formats.decode_bf16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])


# ----------------------------------------------------------- attention pins ----

def _sdpa_reference(q, X, ctx, scale):
    """Causal attention on positions with torch SDPA (float64): the verify token at
    global position t = ctx - qlen + i sees every key at position <= t."""
    qlen, H, _ = q.shape
    qt = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)            # [1, H, qlen, 576]
    k = torch.from_numpy(X[:ctx]).unsqueeze(0).unsqueeze(0).expand(1, H, ctx, 576)
    v = torch.from_numpy(X[:ctx, :512]).unsqueeze(0).unsqueeze(0).expand(1, H, ctx, 512)
    qpos = torch.arange(ctx - qlen, ctx).unsqueeze(1)
    kpos = torch.arange(ctx).unsqueeze(0)
    mask = kpos <= qpos                                              # [qlen, ctx]
    out = torch.nn.functional.scaled_dot_product_attention(qt, k, v, attn_mask=mask, scale=scale)
    scores = (qt @ k.transpose(-1, -2)) * scale
    scores = scores.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(scores, dim=-1)
    return out[0].permute(1, 0, 2).numpy(), lse[0].permute(1, 0).numpy()


def _tiny(seed, qlen=3, H=4, ctx=37):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, qlen, H, 576))
    X = rng.standard_normal((ctx, 576))
    return q, X


def _latents_of(X):
    return lambda b, pos: X[pos]


def sdpa_pin_error(seed=0, qlen=3, H=4, ctx=37, scale=1 / math.sqrt(192)):
    q, X = _tiny(seed, qlen, H, ctx)
    out, lse = A.verify_attention(q, _latents_of(X), [ctx], scale)
    ro, rl = _sdpa_reference(q[0], X, ctx, scale)
    return max(np.abs(out[0] - ro).max(), np.abs(lse[0] - rl).max())


@pytest.mark.parametrize("seed,qlen,ctx", [(0, 3, 37), (1, 1, 5), (2, 5, 64), (3, 2, 2)])
def test_global_attention_matches_sdpa(seed, qlen, ctx):
    assert sdpa_pin_error(seed, qlen, 3, ctx) < 1e-12


def test_single_visible_token():
    # g = 1: the output is the first token's value exactly and LSE is its score
    q, X = _tiny(7, qlen=3, H=2, ctx=3)
    scale = 0.125
    out, lse = A.verify_attention(q, _latents_of(X), [3], scale)
    assert np.array_equal(out[0, 0], np.broadcast_to(X[0, :512], (2, 512)))
    assert np.allclose(lse[0, 0], scale * q[0, 0] @ X[0], rtol=0, atol=1e-12)


def test_abs_value_attention_brute_force():
    # sum_t w_t |v_t| with the softmax weights written out as loops
    q, X = _tiny(11, qlen=2, H=2, ctx=9)
    scale = 0.09
    out, _ = A.verify_attention(q, _latents_of(X), [9], scale, abs_values=True)
    for i in range(2):
        g = 9 - 2 + 1 + i
        for h in range(2):
            s = [scale * float(np.dot(q[0, i, h], X[t])) for t in range(g)]
            m = max(s)
            e = [math.exp(v - m) for v in s]
            z = sum(e)
            want = [sum(e[t] / z * abs(X[t, d]) for t in range(g)) for d in range(512)]
            assert np.abs(out[0, i, h] - np.array(want)).max() < 1e-12


def test_abs_value_attention_bounds_and_special_cases():
    q, X = _tiny(12, qlen=3, H=3, ctx=40)
    scale = 0.11
    lat = _latents_of(X)
    out, lse = A.verify_attention(q, lat, [40], scale)
    oabs, lse_abs = A.verify_attention(q, lat, [40], scale, abs_values=True)
    assert np.array_equal(lse, lse_abs)                 # same weights
    assert (np.abs(out) <= oabs + 1e-15).all()           # triangle inequality
    # one visible token: |v_0|
    o1, _ = A.verify_attention(q, lat, [3], scale, abs_values=True)
    assert np.array_equal(o1[0, 0], np.broadcast_to(np.abs(X[0, :512]), (3, 512)))
    # non-negative values: the two coincide
    latp = _latents_of(np.abs(X))
    a, _ = A.verify_attention(q, latp, [40], scale)
    b, _ = A.verify_attention(q, latp, [40], scale, abs_values=True)
    assert np.abs(a - b).max() < 1e-12


def merge_identity_error(seed, W, S, qlen=3, H=3, ctx=53, scale=0.07):
    q, X = _tiny(seed, qlen, H, ctx)
    lat = _latents_of(X)
    g_out, g_lse = A.verify_attention(q, lat, [ctx], scale)
    outs, lses = [], []
    for r in range(W):
        o, l = A.verify_attention(q, lat, [ctx], scale, world=W, interleave=S, rank=r)
        outs.append(o)
        lses.append(l)
    m_out, m_lse = A.merge_ranks(np.stack(outs), np.stack(lses))
    return max(np.abs(m_out - g_out).max(), np.abs(m_lse - g_lse).max())


@pytest.mark.parametrize("W,S", [(1, 1), (2, 1), (3, 1), (8, 1), (2, 4), (8, 16), (4, 2)])
def test_merge_of_rank_partials_is_global(W, S):
    assert merge_identity_error(W * 10 + S, W, S) < 1e-12


def test_empty_rank_contributes_nothing():
    # ctx small relative to W*S: high ranks own nothing for early rows
    q, X = _tiny(11, qlen=3, H=2, ctx=5)
    lat = _latents_of(X)
    W, S = 8, 16
    for r in range(1, W):
        o, l = A.verify_attention(q, lat, [5], 0.1, world=W, interleave=S, rank=r)
        assert np.all(o == 0.0) and np.all(np.isneginf(l))
    o0, l0 = A.verify_attention(q, lat, [5], 0.1, world=W, interleave=S, rank=0)
    g, gl = A.verify_attention(q, lat, [5], 0.1)
    assert np.allclose(o0, g, atol=1e-13) and np.allclose(l0, gl, atol=1e-13)
    # all ranks empty -> (0, -inf)
    mo, ml = A.merge_ranks(np.zeros((3, 2, 512)), np.full((3, 2), -np.inf))
    assert np.all(mo == 0.0) and np.all(np.isneginf(ml))


def segment_merge_error(seed, nseg, n=41, H=3, scale=0.09):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((H, 576))
    K = rng.standard_normal((n, 576))
    cuts = np.sort(rng.choice(np.arange(1, n), size=nseg - 1, replace=False)) if nseg > 1 else []
    bounds = [0, *cuts, n]
    outs, l2s = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        o, l2 = A.base2_stats(q, K[a:b], scale)
        outs.append(o)
        l2s.append(l2)
    # an empty segment too
    o_e, l_e = A.base2_stats(q, K[:0], scale)
    outs.append(o_e)
    l2s.append(l_e)
    m_o, m_l = A.merge_segments_base2(np.stack(outs), np.stack(l2s))
    d_o, d_l = A.attend(q, K, scale)
    return max(np.abs(m_o - d_o).max(), np.abs(m_l - d_l).max())


@pytest.mark.parametrize("nseg", [1, 2, 5, 17])
def test_segment_merge_base2_to_natural(nseg):
    assert segment_merge_error(nseg, nseg) < 1e-12


def test_base2_natural_relation():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 576))
    K = rng.standard_normal((9, 576))
    _, l2 = A.base2_stats(q, K, 0.1)
    s = 0.1 * q @ K.T
    ref_nat = torch.logsumexp(torch.from_numpy(s), dim=1).numpy()
    ref_b2 = torch.logsumexp(torch.from_numpy(s * math.log2(math.e) * math.log(2)), dim=1).numpy() / math.log(2)
    assert np.allclose(l2 * math.log(2), ref_nat, atol=1e-12)
    assert np.allclose(l2, ref_b2, atol=1e-12)


def test_negative_control_shape():
    # one sequence of the pages' FP8 test: 96 heads x 3 rows x 512 value dims
    vals = {}
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "negative_control.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v)
    out = np.zeros((1, int(vals["qlen"]), int(vals["heads"]), int(vals["v_dim"])))
    assert out.size == int(vals["elements"])


def _boundary_committed_prefix(ctx, qlen, i):
    return ctx - qlen            # old form: every row sees only the committed prefix


def _boundary_noncausal(ctx, qlen, i):
    return ctx                   # every row sees the whole context


@pytest.mark.parametrize("mutant", [_boundary_committed_prefix, _boundary_noncausal])
def test_negative_control_mutated_boundary_fails(mutant):
    # the merged per-rank result with a mutated row boundary must miss global attention
    q, X = _tiny(21, qlen=3, H=8, ctx=64)
    lat = _latents_of(X)
    g_out, _ = A.verify_attention(q, lat, [64], 1 / math.sqrt(192))
    outs, lses = [], []
    for r in range(2):
        o, l = A.verify_attention(q, lat, [64], 1 / math.sqrt(192), world=2, interleave=1, rank=r,
                                  boundary=mutant)
        outs.append(o)
        lses.append(l)
    m_out, _ = A.merge_ranks(np.stack(outs), np.stack(lses))
    assert np.abs(m_out - g_out).max() > 1.5e-2


# ------------------------------------------------------- pins catch mutants ----

def test_pins_catch_mutants(monkeypatch):
    real_attend = A.attend

    def attend_no_rope(q_rows, keys, s):          # dropped the 64 rope dims from the scores
        q2 = q_rows.copy()
        q2[:, 512:] = 0.0
        return real_attend(q2, keys, s)

    def attend_wrong_values(q_rows, keys, s):     # values taken from the wrong 512 dims
        k2 = np.concatenate([keys[:, 64:], keys[:, :64]], axis=1) if keys.shape[0] else keys
        o, l = real_attend(q_rows, keys, s)
        if keys.shape[0]:
            sc = s * q_rows @ keys.T
            p = np.exp(sc - l[:, None])
            o = p @ k2[:, :512]
        return o, l

    def attend_no_scale(q_rows, keys, s):
        return real_attend(q_rows, keys, 1.0)

    for bad in (attend_no_rope, attend_wrong_values, attend_no_scale):
        monkeypatch.setattr(A, "attend", bad)
        assert sdpa_pin_error(0) > 1e-6, bad.__name__
        monkeypatch.setattr(A, "attend", real_attend)

    real_owner = layout.owner_rank
    monkeypatch.setattr(layout, "owner_rank", lambda p, w, s: np.asarray(p) % w)   # ignores S
    assert merge_identity_error(1, 4, 2) < 1e-12          # still a partition ...
    caught = any(layout.rank_local_positions(g, 4, 2, r).shape[0] != _page_len(g, r, 4, 2)
                 for g in range(40) for r in range(4))
    assert caught                                         # ... but the page formula catches it
    monkeypatch.setattr(layout, "owner_rank", real_owner)

    real_merge = A.merge_ranks

    def merge_plain_mean(outs, lses):                     # forgot the LSE weights
        o, l = real_merge(outs, lses)
        return np.mean(outs, axis=0), l
    monkeypatch.setattr(A, "merge_ranks", merge_plain_mean)
    assert merge_identity_error(3, 2, 1) > 1e-6
    monkeypatch.setattr(A, "merge_ranks", real_merge)

    real_seg = A.merge_segments_base2

    def seg_natural_weights(outs, lse2):                   # used e^x instead of 2^x
        o, l = real_seg(outs, lse2 * math.log2(math.e))
        return o, l
    monkeypatch.setattr(A, "merge_segments_base2", seg_natural_weights)
    assert segment_merge_error(5, 5) > 1e-6
    monkeypatch.setattr(A, "merge_segments_base2", real_seg)

    monkeypatch.setattr(layout, "verify_row_boundary", lambda c, q, i: c - q + i)   # off by one
    q, X = _tiny(0)
    out, _ = A.verify_attention(q, _latents_of(X), [37], 0.07, boundary=layout.verify_row_boundary)
    ro, _ = _sdpa_reference(q[0], X, 37, 0.07)
    assert np.abs(out[0] - ro).max() > 1e-6


def _page_len(g, rank, W, S):
    span = W * S
    return g // span * S + min(max(g % span - rank * S, 0), S)


def _sdpa_full_prefix(q, X, ctx, scale):
    """Unmasked attention of every row over positions [0, ctx) (torch SDPA, float64)."""
    qlen, H, _ = q.shape
    qt = torch.from_numpy(q).permute(1, 0, 2).unsqueeze(0)
    k = torch.from_numpy(X[:ctx]).unsqueeze(0).unsqueeze(0).expand(1, H, ctx, 576)
    v = torch.from_numpy(X[:ctx, :512]).unsqueeze(0).unsqueeze(0).expand(1, H, ctx, 512)
    out = torch.nn.functional.scaled_dot_product_attention(qt, k, v, scale=scale)
    lse = torch.logsumexp((qt @ k.transpose(-1, -2)) * scale, dim=-1)
    return out[0].permute(1, 0, 2).numpy(), lse[0].permute(1, 0).numpy()


@pytest.mark.parametrize("seed,qlen,ctx,W,S", [(0, 3, 37, 2, 1), (1, 5, 64, 8, 16), (2, 2, 9, 4, 2)])
def test_block_rows_match_unmasked_sdpa(seed, qlen, ctx, W, S):
    # "Context Parallel Guide", DSpark: a bidirectional draft block has no mask
    # on global positions -- plain attention over the whole cache for every row,
    # and the rank split still merges back to it
    q, X = _tiny(seed, qlen=qlen, H=3, ctx=ctx)
    scale = 1 / math.sqrt(192)
    lat = _latents_of(X)
    out, lse = A.verify_attention(q, lat, [ctx], scale, boundary=layout.block_row_boundary)
    ro, rl = _sdpa_full_prefix(q[0], X, ctx, scale)
    assert np.abs(out[0] - ro).max() < 1e-12 and np.abs(lse[0] - rl).max() < 1e-12
    parts = [A.verify_attention(q, lat, [ctx], scale, world=W, interleave=S, rank=r,
                                boundary=layout.block_row_boundary) for r in range(W)]
    mo, ml = A.merge_ranks(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    assert np.abs(mo - out).max() < 1e-12 and np.abs(ml - lse).max() < 1e-12
