"""Pins for the BF16 rounding of ``oracle.formats`` and the expectation and
acceptance rule of ``oracle.parity`` (CPU only).

Round-to-nearest-even is pinned against torch's float32 -> bfloat16 cast over
sampled binary32 patterns of every exponent, and by hand-checked values where
a float64 input would round differently through binary32; the rounding
interval and the neighbour steps against brute force over every finite BF16
value; the two-rounding expectation against the plain merge and a case where
rounding before the merge changes the result; the acceptance rule against a
brute-force search over reals.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import formats, parity


def _all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = formats.decode_bf16(bits)
    return v[np.isfinite(v)]


# ------------------------------------------------------------ BF16 rounding ----

def test_round_bf16_matches_torch_on_binary32_patterns():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, 4_000_000, dtype=np.uint64).astype(np.uint32)
    # every exponent, ties (low 16 bits 0x8000) and their neighbours, subnormals, the overflow edge
    ties = (rng.integers(0, 2 ** 16, 200_000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    edge = np.array([0x7F7F8000, 0x7F7F7FFF, 0x7F7FFFFF, 0x00008000, 0x00018000, 0x80008000,
                     0x3F808000, 0x3F818000, 0x00000001, 0x80000000, 0x00000000], dtype=np.uint32)
    bits = np.concatenate([bits, ties, ties + 1, ties - 1, edge])
    x = bits.view(np.float32)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    with np.errstate(invalid="ignore"):
        mine = formats.round_bf16(x.astype(np.float64))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


def test_round_bf16_single_rounding_of_float64():
    # exact ties break to the even significand
    assert formats.round_bf16(1 + 2.0 ** -8) == 1.0
    assert formats.round_bf16(1 + 3 * 2.0 ** -8) == 1 + 2 * 2.0 ** -7
    # just above a tie rounds up; through binary32 it would first become the tie and go down
    x = 1 + 2.0 ** -8 + 2.0 ** -40
    assert formats.round_bf16(x) == 1 + 2.0 ** -7
    assert torch.tensor(x, dtype=torch.float64).float().bfloat16().double().item() == 1.0
    # the largest finite value, overflow at half a step past it, signed zeros, subnormal quantum
    assert formats.round_bf16(formats.BF16_MAX) == formats.BF16_MAX
    assert np.isinf(formats.round_bf16((2 - 2.0 ** -8) * 2.0 ** 127))
    assert formats.round_bf16((2 - 2.0 ** -8) * 2.0 ** 127 * (1 - 2.0 ** -30)) == formats.BF16_MAX
    assert np.signbit(formats.round_bf16(-1e-60)) and formats.round_bf16(-1e-60) == 0.0
    assert formats.round_bf16(2.0 ** -133) == 2.0 ** -133
    assert formats.round_bf16(1.5 * 2.0 ** -133) == 2.0 ** -132
    assert formats.round_bf16(0.5 * 2.0 ** -133) == 0.0


def test_bf16_quantum_values():
    assert formats.bf16_quantum(1.0) == 2.0 ** -7
    assert formats.bf16_quantum(1.99) == 2.0 ** -7
    assert formats.bf16_quantum(2.0) == 2.0 ** -6
    assert formats.bf16_quantum(-3.5) == 2.0 ** -6
    assert formats.bf16_quantum(0.5) == 2.0 ** -8
    assert formats.bf16_quantum(0.0) == 2.0 ** -133
    assert formats.bf16_quantum(2.0 ** -130) == 2.0 ** -133


def test_bf16_step_walks_the_sorted_values():
    v = np.unique(_all_finite_bf16())             # -0 and +0 collapse to one value
    up = formats.bf16_step(v[:-1], 1)
    assert np.array_equal(up, v[1:])
    down = formats.bf16_step(v[1:], -1)
    assert np.array_equal(down, v[:-1])


def test_rounding_interval_brute_force():
    v = np.unique(_all_finite_bf16())
    v = v[np.abs(v) < formats.BF16_MAX]           # the outermost values border the overflow
    lo, hi = formats.bf16_rounding_interval(v)
    # consecutive intervals tile the line
    assert np.array_equal(hi[:-1], lo[1:])
    # points just inside round to v, points just outside do not
    eps_lo = np.abs(lo) * 2.0 ** -40 + 2.0 ** -160
    eps_hi = np.abs(hi) * 2.0 ** -40 + 2.0 ** -160
    assert np.array_equal(formats.round_bf16(lo + eps_lo), v)
    assert np.array_equal(formats.round_bf16(hi - eps_hi), v)
    assert not np.any(formats.round_bf16(lo - eps_lo) == v)
    assert not np.any(formats.round_bf16(hi + eps_hi) == v)


# -------------------------------------------------------- two-rounding expectation ----

def test_expectation_single_rank_is_the_rounded_output():
    rng = np.random.default_rng(1)
    o = rng.standard_normal((1, 5, 512)) * 3
    l = rng.standard_normal((1, 5))
    a, z, e, lse = parity.merged_expectation(o, l)
    assert np.array_equal(e, formats.round_bf16(o[0]))
    assert np.array_equal(a[0], z) and np.array_equal(lse, l[0])


def test_expectation_equals_plain_merge_on_representable_partials():
    rng = np.random.default_rng(2)
    o = formats.round_bf16(rng.standard_normal((4, 7, 512)))
    l = rng.standard_normal((4, 7)) * 4
    l[1, 3] = -np.inf
    a, z, e, lse = parity.merged_expectation(o, l)
    mo, ml = A.merge_ranks(o, l)
    assert np.array_equal(a, o) and np.array_equal(z, mo) and np.array_equal(lse, ml)
    assert np.array_equal(e, formats.round_bf16(mo))


def test_expectation_rounds_each_rank_before_the_merge():
    # two equal-weight ranks; rounding each rank first (1 + 2^-7 and 1) gives the tie
    # 1 + 2^-8, which goes to the even value 1; rounding only the exact merge
    # (1 + 0.525 2^-7) gives 1 + 2^-7
    o = np.array([[1 + 0.6 * 2.0 ** -7], [1 + 0.45 * 2.0 ** -7]])
    l = np.zeros((2, 1))
    a, z, e, _ = parity.merged_expectation(o[..., None], l)
    assert a[0, 0, 0] == 1 + 2.0 ** -7 and a[1, 0, 0] == 1.0
    assert z[0, 0] == 1 + 2.0 ** -8 and e[0, 0] == 1.0
    mo, _ = A.merge_ranks(o[..., None], l)
    assert formats.round_bf16(mo)[0, 0] == 1 + 2.0 ** -7


# --------------------------------------------------------------- acceptance ----

def test_accept_rounded_brute_force():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(300) * np.exp2(rng.integers(-6, 3, 300))
    bar = np.exp2(rng.uniform(-14, -6, 300))
    for k in (-3, -2, -1, 0, 1, 2, 3):
        v = formats.bf16_step(formats.round_bf16(x), k)
        got = parity.accept_rounded(v, x, bar)
        # brute force: a dense grid over [x - bar, x + bar], endpoints included
        t = np.linspace(-1.0, 1.0, 4001)
        ys = x[:, None] + bar[:, None] * t[None, :]
        want = (formats.round_bf16(ys) == v[:, None]).any(axis=1)
        assert np.array_equal(got, want), k


def test_accept_rounded_bar_zero_is_exact_rounding():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(10000)
    r = formats.round_bf16(x)
    assert parity.accept_rounded(r, x, 0.0).all()
    assert not parity.accept_rounded(formats.bf16_step(r, 1), x, 0.0).any()


def test_accept_merged_flags_kernel_error_beyond_the_bar():
    rng = np.random.default_rng(5)
    o = rng.standard_normal((8, 64, 512)) * 0.3
    l = rng.standard_normal((8, 64)) * 2
    bar = 1.5e-2
    _, z, e, _ = parity.merged_expectation(o, l)
    assert parity.accept_merged(e, o, l, bar).all()
    # an arithmetic error of 1.01 x the bar beyond the largest shift the admitted
    # flips allow (one step on every rank, weighted, and one on the output) is
    # always rejected
    _, lse = A.merge_ranks(o, l)
    wts = np.exp(l - lse[None])[..., None]
    flips = (wts * formats.bf16_quantum(formats.round_bf16(o))).sum(axis=0)
    q = formats.bf16_quantum(z)
    bad = formats.round_bf16(z + 1.01 * bar + flips + 2 * q)
    assert not parity.accept_merged(bad, o, l, bar).any()
    bad = formats.round_bf16(z - 1.01 * bar - flips - 2 * q)
    assert not parity.accept_merged(bad, o, l, bar).any()
    # half the bar is always accepted
    ok = formats.round_bf16(z + 0.5 * bar)
    assert parity.accept_merged(ok, o, l, bar).all()


def test_rank_choices_one_step_where_the_boundary_is_within_the_bar():
    x = np.array([1 + 0.45 * 2.0 ** -7, 1 + 0.1 * 2.0 ** -7, 1 + 0.9 * 2.0 ** -7])
    lo, hi = parity.rank_choices(x, 2.0 ** -9)
    # 0.45: the midpoint (0.5) is 0.05 steps away -> the upper neighbour is admissible
    assert lo[0] == 1.0 and hi[0] == 1 + 2.0 ** -7
    # 0.1: nothing within a quarter step -> only the rounded value
    assert lo[1] == hi[1] == 1.0
    # 0.9: rounds up; the midpoint is 0.4 steps (> 0.25) away -> no neighbour
    assert lo[2] == hi[2] == 1 + 2.0 ** -7


@pytest.mark.parametrize("mutant", ["merge_unrounded", "round_merge_only"])
def test_expectation_mutants_fail_a_pin(mutant):
    # plausible mistakes in the expectation are caught by the pins above
    o = np.array([[1 + 0.6 * 2.0 ** -7], [1 + 0.45 * 2.0 ** -7]])[..., None]
    l = np.zeros((2, 1))
    if mutant == "merge_unrounded":
        z, _ = A.merge_ranks(o, l)
        e = formats.round_bf16(z)
    else:
        e = formats.round_bf16(A.merge_ranks(formats.round_bf16(o), l)[0] * (1 + 2.0 ** -9))
    assert e[0, 0] != 1.0
