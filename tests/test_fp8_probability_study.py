"""FP8 probabilities for the p.v product: a float64 study of their error on
rows shaped like the pages' decode and long-context runs.

The FP8-probability variant (geometry p_format "fp8") forms each 64-token
stage's probabilities against that stage's own ceiling ms = ceil(max s)
(scores s in base 2): p' = 2^(s - ms + 8) lies in (0, 256], inside E4M3's
range, and is rounded to E4M3 (nearest, ties to even; below half the
smallest subnormal it becomes 0).  The product applies 2^(ms - mref) as the
E8M0 scale of the P operand, and the row is normalised by the sum of the
unrounded p' in fp32, so the output is

    O = sum_t E4M3(p'_t) 2^(ms_t - 8) v_t / sum_t p'_t 2^(ms_t - 8).

This file emulates exactly that in float64 and compares it with exact
attention over the same decoded cache ("Context Parallel Guide (PCP &
DCP)", "How it works" item 4 runs attention with an FP8 KV cache; the bar
on the output is max-abs 1.5e-2).  A stage with no visible token keeps
p' = 0.  Rows: the decode workload's rank shard (16,384 tokens) and a
longer 65,536-token shard of the 1M-context run, query and latents N(0, 1)
as BF16 and per-tensor-scaled E4M3, softmax scale 1/sqrt(192) as the
workloads use.

The error of a weight is up to 2^-4 of it (three mantissa bits), so a row's
output error scales with |v| / sqrt(n_eff), n_eff = 1 / sum w^2 being its
effective number of tokens: on these long N(0, 1) rows (n_eff about 100 at
the least) it stays inside the bar -- about 1e-2 at worst over 256 decode
rows -- while a row dominated by a few tokens can leave it.  Rows that short
are compared with attention under the same rounding instead.
"""
import numpy as np
import pytest

from oracle import formats, qsplit

BAR = 1.5e-2
STAGE = 64
SHIFT = 8


def _row_inputs(n_tok, heads, seed):
    rng = np.random.default_rng(seed)
    q = formats.decode_bf16(_bf16_bits(rng.standard_normal((heads, 576), dtype=np.float32)))
    lat = rng.standard_normal((n_tok, 576), dtype=np.float32).astype(np.float64)
    scale = float(np.abs(lat).max()) / 448.0
    kv = formats.decode_e4m3(qsplit.e4m3_rne(np.clip(lat / scale, -448, 448)), scale)
    return q, kv


def _bf16_bits(x):
    # round-to-nearest-even float32 -> BF16 bits
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def _exact(q, kv, sm_scale):
    s = (kv @ q.T) * sm_scale              # [T, H], natural units
    m = s.max(axis=0)
    p = np.exp(s - m)
    return (p.T @ kv[:, :512]) / p.sum(axis=0)[:, None]


def _fp8_probs(q, kv, sm_scale):
    s2 = (kv @ q.T) * (sm_scale / np.log(2.0))   # [T, H], base 2
    T, H = s2.shape
    num = np.zeros((H, 512))
    den = np.zeros(H)
    for st in range(0, T, STAGE):
        blk = s2[st:st + STAGE]
        ms = np.ceil(blk.max(axis=0))                 # stage ceiling per head-row
        pp = np.exp2(blk - ms + SHIFT)                # in (0, 256]
        pq = formats.decode_e4m3(qsplit.e4m3_rne(pp))
        w = np.exp2(ms - SHIFT)
        num += (pq * w).T @ kv[st:st + STAGE, :512]
        den += (pp * w).sum(axis=0)
    return num / den[:, None]


@pytest.mark.parametrize("n_tok,heads,seed", [(16384, 16, 11), (65536, 4, 12)])
def test_fp8_probabilities_within_bar(n_tok, heads, seed):
    q, kv = _row_inputs(n_tok, heads, seed)
    sm = 1.0 / np.sqrt(192.0)
    ref = _exact(q, kv, sm)
    got = _fp8_probs(q, kv, sm)
    err = np.abs(got - ref)
    print(f"{n_tok} tokens x {heads} rows: max|dO| {err.max():.3e}, mean {err.mean():.3e}, "
          f"max|O| {np.abs(ref).max():.3e}")
    assert err.max() < BAR


def test_e4m3_probabilities_need_the_stage_scale():
    # without the per-stage ceiling (p = 2^(s - row max), unscaled) most of a
    # long row's weights fall below E4M3's smallest step and the error grows
    # past the per-stage figure: the scale is what makes FP8 P usable
    q, kv = _row_inputs(16384, 4, 13)
    sm = 1.0 / np.sqrt(192.0)
    ref = _exact(q, kv, sm)
    s2 = (kv @ q.T) * (sm / np.log(2.0))
    p = np.exp2(s2 - s2.max(axis=0))
    pq = formats.decode_e4m3(qsplit.e4m3_rne(p))
    unscaled = (pq.T @ kv[:, :512]) / p.sum(axis=0)[:, None]
    staged = _fp8_probs(q, kv, sm)
    e_uns = np.abs(unscaled - ref).max()
    e_stg = np.abs(staged - ref).max()
    print(f"unscaled max|dO| {e_uns:.3e}, per-stage scale {e_stg:.3e}")
    assert e_stg < e_uns
