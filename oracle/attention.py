"""Float64 MLA causal-verification attention: global, per-rank split, merges.

Test infrastructure only (see ``oracle/__init__``).

What is computed (plain definitions, no blocking or reordering):

* MLA latent attention.  Every query head attends to the same cached latent
  vector per token ("Context Parallel Guide (PCP & DCP)", opening of the
  "Decode Context Parallel (DCP) Guide": the MLA KV is a single latent head).
  Scores use all 576 dims (512 latent + 64 rope); values are the first 512
  dims of the same cached vector.
* Causal verification.  Row i of a sequence sees global positions
  [0, ctx - qlen + 1 + i) ("[ROCm][MLA][DCP] Support causal multi-token
  verification", "Implementation" item 1; boundary in ``layout``).
* Per-rank partial.  The same softmax restricted to the positions the rank
  owns; the rank returns its output and a natural-log LSE ("Context Parallel
  Guide", "How it works" item 3 and the commit message of PR #51705, which
  states that decode LSE is natural-log).  A rank that owns no visible
  position returns output 0 and LSE -inf, so it contributes nothing.
* Cross-rank merge.  A per-(token, head) scalar weight exp(LSE_r - LSE) times
  each rank's output, summed over ranks ("Context Parallel Guide",
  ``enable_project_before_merge``); LSE = log sum_r exp(LSE_r).
* Segment merge.  Split-KV segments carry base-2 statistics; merging them
  gives the rank output and converts the base-2 LSE to natural log
  (PR #51705, "Implementation" item 3).
"""
import numpy as np

from . import layout

D_QK = 576
D_V = 512
LN2 = np.log(2.0)


def attend(q_rows: np.ndarray, keys: np.ndarray, softmax_scale: float, abs_values: bool = False):
    """Softmax attention of ``q_rows[H, 576]`` over ``keys[n, 576]`` (float64).

    Returns ``(out[H, 512], lse[H])`` with natural-log LSE; n = 0 gives
    ``(0, -inf)``.  With ``abs_values`` the values are |v| under the same
    weights: sum_t w_t |v_t|, the scale of the error that rounding each weight
    to a relative precision puts on the output.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    H = q_rows.shape[0]
    if keys.shape[0] == 0:
        return np.zeros((H, D_V)), np.full(H, -np.inf)
    scores = softmax_scale * (q_rows @ keys.T)            # [H, n]
    mx = scores.max(axis=1, keepdims=True)
    e = np.exp(scores - mx)
    z = e.sum(axis=1, keepdims=True)
    lse = (mx + np.log(z))[:, 0]
    vals = keys[:, :D_V]
    out = (e / z) @ (np.abs(vals) if abs_values else vals)
    return out, lse


def _visible_positions(ctx, qlen, i, world, interleave, rank, boundary):
    g = boundary(ctx, qlen, i)
    if rank is None:
        return np.arange(max(g, 0), dtype=np.int64)
    return layout.rank_local_positions(g, world, interleave, rank)


def verify_attention(q: np.ndarray, latents, ctx_lens, softmax_scale: float, *,
                     world: int = 1, interleave: int = 1, rank=None, rows=None,
                     boundary=layout.verify_row_boundary, abs_values: bool = False):
    """Causal-verify attention for selected rows, globally or for one rank.

    ``q``: float64 ``[B, qlen, H, 576]``.  ``latents``: callable
    ``latents(b, positions) -> float64 [n, 576]`` returning the decoded global
    latent rows of sequence b.  ``rank=None`` attends to every visible global
    position; an int restricts to the positions that rank owns.  ``rows``:
    iterable of ``(b, i)``; default all.  ``boundary`` is the row-boundary
    rule (replaceable only by the negative-control tests).  ``abs_values``:
    see ``attend``.

    Returns ``(out[B, qlen, H, 512], lse[B, qlen, H])``; rows not selected
    are NaN.
    """
    B, qlen, H, _ = q.shape
    out = np.full((B, qlen, H, D_V), np.nan)
    lse = np.full((B, qlen, H), np.nan)
    if rows is None:
        rows = [(b, i) for b in range(B) for i in range(qlen)]
    for b, i in rows:
        pos = _visible_positions(int(ctx_lens[b]), qlen, i, world, interleave, rank, boundary)
        keys = latents(b, pos) if pos.shape[0] else np.zeros((0, D_QK))
        out[b, i], lse[b, i] = (attend(q[b, i], keys, softmax_scale, abs_values=True) if abs_values
                                else attend(q[b, i], keys, softmax_scale))
    return out, lse


def merge_ranks(outs: np.ndarray, lses: np.ndarray):
    """LSE-merge W partials: ``outs[W, ..., 512]``, ``lses[W, ...]`` (natural log).

    All ranks at -inf gives ``(0, -inf)``.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    mx = lses.max(axis=0)
    finite = np.isfinite(mx)
    safe_mx = np.where(finite, mx, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - safe_mx), 0.0)   # [W, ...]
    z = w.sum(axis=0)
    lse = np.where(finite, safe_mx + np.log(np.where(finite, z, 1.0)), -np.inf)
    zz = np.where(finite, z, 1.0)
    out = (w[..., None] * outs).sum(axis=0) / zz[..., None]
    out = np.where(finite[..., None], out, 0.0)
    return out, lse


def merge_segments_base2(outs: np.ndarray, lse2: np.ndarray):
    """Merge split-KV segment partials with base-2 statistics.

    ``outs[nseg, ..., 512]`` are each segment's normalised output and
    ``lse2[nseg, ...]`` its log2-sum-exp2 of base-2 scores.  Returns the
    merged output and the *natural-log* LSE (= ln 2 times the merged base-2
    value).  All segments at -inf gives ``(0, -inf)``.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lse2 = np.asarray(lse2, dtype=np.float64)
    mx = lse2.max(axis=0)
    finite = np.isfinite(mx)
    safe_mx = np.where(finite, mx, 0.0)
    w = np.where(np.isfinite(lse2), np.exp2(lse2 - safe_mx), 0.0)
    z = w.sum(axis=0)
    zz = np.where(finite, z, 1.0)
    l2 = np.where(finite, safe_mx + np.log2(zz), -np.inf)
    out = (w[..., None] * outs).sum(axis=0) / zz[..., None]
    out = np.where(finite[..., None], out, 0.0)
    return out, l2 * LN2


def base2_stats(q_rows: np.ndarray, keys: np.ndarray, softmax_scale: float):
    """One segment's normalised output and base-2 LSE (scores scaled by log2 e)."""
    out, lse = attend(q_rows, keys, softmax_scale)
    return out, lse / LN2
