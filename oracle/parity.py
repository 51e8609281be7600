"""Expected BF16 outputs and the acceptance rule of the parity tests.

Test infrastructure only (see ``oracle/__init__``).

The method rounds twice on the way out ("[ROCm][MLA][DCP] Support causal
multi-token verification", "Implementation" item 3: each rank's base-2
statistics are merged into a BF16 output plus a natural-log LSE; the
cross-rank merge then combines those BF16 partials with their fp32 LSEs,
"Context Parallel Guide (PCP & DCP)", "How it works" item 3).  The expected
values therefore take the exact float64 partials through the same two
roundings:

  * rank output: ``a_r = RNE_bf16(O_r)``;
  * merged output: ``z = sum_r exp(LSE_r - LSE) a_r`` in float64 with the
    exact LSEs, then ``E = RNE_bf16(z)``.

A kernel computes its fp32 result ``y`` with some arithmetic error and then
rounds ``y`` to BF16.  Only the rounded value is visible, so an output ``v``
is accepted when some real within the arithmetic bar of the expected real
rounds to ``v``: the distance from the expected real to the rounding interval
of ``v`` is at most the bar.  Where a rank's exact output lies within the bar
of a rounding boundary, the rank may hand the merge the neighbouring BF16
value instead of ``a_r`` (one step, no more); the merged output is then
accepted against the range those choices span.
"""
import numpy as np

from . import attention, formats


def merged_expectation(rank_outs, rank_lses):
    """The two roundings applied to exact per-rank results.

    ``rank_outs[W, ..., 512]`` and ``rank_lses[W, ...]`` (natural log, -inf for
    an empty rank) are float64.  Returns ``(a, z, E, lse)``: the rounded rank
    outputs, the float64 merge of them, its BF16 rounding, and the merged LSE.
    """
    a = formats.round_bf16(rank_outs)
    z, lse = attention.merge_ranks(a, rank_lses)
    return a, z, formats.round_bf16(z), lse


def distance_to_rounding(v, x):
    """Distance from the real ``x`` to the set of reals that round to the BF16 value ``v``."""
    lo, hi = formats.bf16_rounding_interval(v)
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(np.maximum(lo - x, x - hi), 0.0)


def accept_rounded(v, x, bar):
    """True where the BF16 output ``v`` is the rounding of a real within ``bar`` of ``x``."""
    return distance_to_rounding(v, x) <= bar


def rank_choices(x, bar):
    """Lowest and highest BF16 values within one step of ``RNE_bf16(x)`` that a
    rank within ``bar`` of ``x`` can produce."""
    a = formats.round_bf16(x)
    lo_c, hi_c = a.copy(), a.copy()
    for k in (-1, 1):
        n = formats.bf16_step(a, k)
        ok = accept_rounded(n, x, bar)
        if k < 0:
            lo_c = np.where(ok, np.minimum(lo_c, n), lo_c)
        else:
            hi_c = np.where(ok, np.maximum(hi_c, n), hi_c)
    return lo_c, hi_c


def merged_range(rank_outs, rank_lses, bar):
    """Range of ``sum_r w_r c_r`` over the per-rank choices of ``rank_choices``,
    with the exact merge weights ``w_r = exp(LSE_r - LSE)``."""
    rank_lses = np.asarray(rank_lses, dtype=np.float64)
    _, lse = attention.merge_ranks(np.zeros(rank_lses.shape + (1,)), rank_lses)
    safe = np.where(np.isfinite(lse), lse, 0.0)
    wts = np.where(np.isfinite(rank_lses), np.exp(rank_lses - safe), 0.0)[..., None]
    lo_c, hi_c = rank_choices(rank_outs, bar)
    return (wts * lo_c).sum(axis=0), (wts * hi_c).sum(axis=0)


def merged_gap(v, rank_outs, rank_lses, bar):
    """Distance from the range of admissible merges to the reals that round to
    the merged BF16 output ``v``: the least arithmetic error that explains ``v``."""
    lo, hi = merged_range(rank_outs, rank_lses, bar)
    ilo, ihi = formats.bf16_rounding_interval(v)
    return np.maximum(np.maximum(ilo - hi, lo - ihi), 0.0)


def accept_merged(v, rank_outs, rank_lses, bar):
    """True where the merged BF16 output ``v`` is the rounding of a real within
    ``bar`` of a merge of admissible per-rank BF16 outputs."""
    return merged_gap(v, rank_outs, rank_lses, bar) <= bar
