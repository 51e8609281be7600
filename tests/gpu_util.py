"""Helpers for the GPU tests: device upload of seeded workloads and oracle views.

Inputs come from ``synth``; expected values come from ``oracle``; nothing here
computes any part of the method.
"""
import numpy as np
import torch

from oracle import attention as A
from oracle import formats, layout, parity

HAS_GPU = torch.cuda.is_available()


def geometry(w, groups=0, max_local_pages=None, num_blocks=None, row_boundary="causal", q_format="split",
             p_format="split"):
    from decode_context_parallelism_amd import ops
    return ops.Geometry(dcp_world=w.world, interleave=w.interleave, block_size=w.block_size,
                        qlen=w.qlen, num_heads=w.heads, batch=w.batch,
                        max_blocks_per_seq=w.block_table.shape[1],
                        max_local_pages=max_local_pages or w.max_local_pages,
                        kv_dtype=w.kv_format, num_blocks=num_blocks or w.num_blocks,
                        groups=groups, row_boundary=row_boundary, q_format=q_format,
                        p_format=p_format)


def device_inputs(w, device="cuda"):
    q = torch.from_numpy(w.q_bits.view(np.int16)).view(torch.bfloat16).to(device)
    if w.kv_format == "fp8_e4m3":
        lat = torch.from_numpy(w.kv).to(device)
    else:
        lat = torch.from_numpy(w.kv.view(np.int16)).view(torch.bfloat16).to(device)
    seq_ids, positions = w.token_arrays()
    return dict(q=q, latents=lat,
                seq_ids=torch.from_numpy(seq_ids).to(device),
                positions=torch.from_numpy(positions).to(device),
                block_table=torch.from_numpy(w.block_table).to(device),
                ctx_lens=torch.from_numpy(w.ctx_lens).to(device))


def run_group(w, groups=0, device="cuda", row_boundary="causal", q_format="split", p_format="split"):
    """Write the KV, build every rank's metadata, run every rank and the merge."""
    from decode_context_parallelism_amd.group import DcpGroup
    g = geometry(w, groups=groups, row_boundary=row_boundary, q_format=q_format, p_format=p_format)
    d = device_inputs(w, device)
    grp = DcpGroup(g, device)
    grp.write_kv(d["seq_ids"], d["positions"], d["latents"], d["block_table"])
    grp.forward(d["q"], d["ctx_lens"], d["block_table"], w.kv_scale, w.softmax_scale)
    torch.cuda.synchronize()
    return grp, d


def oracle_latents(w):
    def get(b, pos):
        rows = w.kv[w.seq_start[b] + np.asarray(pos, dtype=np.int64)]
        return formats.decode_cache(rows, w.kv_format, w.kv_scale)
    return get


def oracle_q(w, q_format="split"):
    """The query the method multiplies: the BF16 query, or with q_format "fp8"
    its per-row E4M3 quantisation (oracle.qsplit.quantize_rows)."""
    q = formats.decode_bf16(w.q_bits)
    if q_format == "fp8":
        from oracle import qsplit
        q = qsplit.quantize_rows(q)
    return q


def bf16_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def tolerance(w):
    """Arithmetic max-abs bar on outputs: 1.5e-2 with an FP8 cache, 5e-3 with BF16."""
    return 1.5e-2 if w.kv_format == "fp8_e4m3" else 5e-3


LSE_TOL = 1e-3


def bf16_half_ulp(x):
    """Half a BF16 ulp at |x| (the projection bound of the exchange tests)."""
    return formats.bf16_quantum(x) / 2


E4M3_REL = 2.0 ** -4        # E4M3 round-to-nearest, normal range: relative error
E4M3_SUB = 2.0 ** -17       # largest normalised weight error of one subnormal probability


def fp8_probability_bound(wabs, vsum):
    """Bound on the output change from rounding a row's probabilities to E4M3
    against power-of-two scales (p_format "fp8"), given
    ``wabs = sum_t w_t |v_t|`` and ``vsum = sum_t |v_t|`` over the row's
    visible tokens.

    The probabilities of each 32-token block are multiplied by 2^(8 - ms),
    2^ms a power of two at least the block's largest exp-score and below
    twice the row's largest, then rounded; the sum that normalises the row is
    taken before
    rounding.  A normal E4M3 value moves by at most 2^-4 of itself, so weight
    w_t by at most 2^-4 w_t; a subnormal one (below 2^-6) by at most
    min(p', 2^-10), which is min(w_t, 2^-17) after the scale and the
    normalisation.  Summed against |v_t|:

        |dO| <= 2^-4 wabs + min(wabs, 2^-17 vsum).
    """
    return E4M3_REL * wabs + np.minimum(wabs, E4M3_SUB * vsum)


def rank_expectations(w, rows, q_format="split", boundary=layout.verify_row_boundary, ranks=None,
                      p_bound=False):
    """Exact float64 per-rank partials ``(o[W, B, qlen, H, 512], l[W, B, qlen, H])``
    of the selected rows from the oracle (rows not selected, and ranks not in
    ``ranks``, are NaN).

    With ``p_bound`` a third array ``extra`` (shaped like ``o``) holds
    ``fp8_probability_bound`` of each rank's row: what rounding the
    probabilities to E4M3 (p_format "fp8") can add to the output on top of
    the arithmetic bar.

    The oracle attends row by row; the windows of one sequence's rows on one
    rank are prefixes of one another, so each (sequence, rank) is decoded once,
    for its longest window, and shorter windows read a prefix of it.
    """
    q = oracle_q(w, q_format)
    ranks = range(w.world) if ranks is None else ranks
    B, ql, H = w.batch, w.qlen, w.heads
    o = np.full((w.world, B, ql, H, 512), np.nan)
    l = np.full((w.world, B, ql, H), np.nan)
    extra = np.full((w.world, B, ql, H, 512), np.nan) if p_bound else None
    by_seq = {}
    for b, i in rows:
        by_seq.setdefault(int(b), []).append(int(i))
    for b, ilist in sorted(by_seq.items()):
        gmax = max(boundary(int(w.ctx_lens[b]), ql, i) for i in ilist)
        for r in ranks:
            pos_all = layout.rank_local_positions(max(gmax, 0), w.world, w.interleave, r)
            keys = formats.decode_cache(w.kv[w.seq_start[b] + pos_all], w.kv_format, w.kv_scale)

            def lat(bb, pos, keys=keys, pos_all=pos_all, b=b):
                n = len(pos)
                assert bb == b and np.array_equal(pos, pos_all[:n])
                return keys[:n]

            ro, rl = A.verify_attention(q, lat, w.ctx_lens, w.softmax_scale, world=w.world,
                                        interleave=w.interleave, rank=r,
                                        rows=[(b, i) for i in ilist], boundary=boundary)
            for i in ilist:
                o[r, b, i], l[r, b, i] = ro[b, i], rl[b, i]
            if p_bound:
                wv, _ = A.verify_attention(q, lat, w.ctx_lens, w.softmax_scale, world=w.world,
                                           interleave=w.interleave, rank=r,
                                           rows=[(b, i) for i in ilist], boundary=boundary,
                                           abs_values=True)
                for i in ilist:
                    n = len(layout.rank_local_positions(max(boundary(int(w.ctx_lens[b]), ql, i), 0),
                                                        w.world, w.interleave, r))
                    vsum = np.abs(keys[:n, :512]).sum(axis=0)
                    extra[r, b, i] = fp8_probability_bound(wv[b, i], vsum)
    return (o, l, extra) if p_bound else (o, l)


def _new_stats():
    return dict(elements=0, differ=0, one_step=0, beyond_bar=0, beyond_plain=0, max_abs=0.0,
                max_abs_no_flip=0.0, max_implied=0.0)


def _add_stats(st, v, e, implied, bar, plain):
    """Error of BF16 outputs ``v`` against their rounded expectation ``e``:
    elements that differ, those one BF16 step away (rounding-boundary flips),
    the largest |v - e| overall and over the elements that are not one-step
    flips, and the largest arithmetic error the outputs imply (the distance from
    the expected real to the reals that round to v); ``plain`` is the bar
    before any widening."""
    d = np.abs(v - e)
    one = (d > 0) & ((formats.bf16_step(e, 1) == v) | (formats.bf16_step(e, -1) == v))
    st["elements"] += v.size
    st["differ"] += int((d > 0).sum())
    st["one_step"] += int(one.sum())
    st["beyond_bar"] += int((d > bar).sum())
    st["beyond_plain"] += int((implied > plain).sum())
    st["max_abs"] = max(st["max_abs"], float(d.max(initial=0.0)))
    st["max_abs_no_flip"] = max(st["max_abs_no_flip"], float(d[~one].max(initial=0.0)))
    st["max_implied"] = max(st["max_implied"], float(implied.max(initial=0.0)))


def check_rank(w, gpu_o, gpu_l, o, l, rows, tag="", extra=None):
    """One rank's BF16 output and LSE against its exact partial (``o``, ``l`` for
    that rank).  Empty (row, rank): exactly 0 and -inf.  Otherwise each output
    element must be the BF16 rounding of a real within the bar of the exact value,
    and the LSE within 1e-3.  ``extra`` (that rank's, shaped like ``o``) widens
    the bar element by element.  Returns statistics of the error against the
    rounded exact value."""
    st = _new_stats()
    for b, i in rows:
        bar = tolerance(w) if extra is None else tolerance(w) + extra[b, i]
        emp = np.isneginf(l[b, i])
        assert np.all(np.isneginf(gpu_l[b, i][emp])), (tag, b, i)
        assert np.all(gpu_o[b, i][emp] == 0.0), (tag, b, i)
        assert np.all(np.isfinite(gpu_l[b, i][~emp])), (tag, b, i)
        if not (~emp).any():
            continue
        x, v = o[b, i][~emp], gpu_o[b, i][~emp]
        bar = bar if np.isscalar(bar) else bar[~emp]
        implied = parity.distance_to_rounding(v, x)
        assert (implied <= bar).all(), (tag, b, i, float((implied - bar).max()))
        err_l = float(np.abs(gpu_l[b, i][~emp] - l[b, i][~emp]).max())
        assert err_l <= LSE_TOL, (tag, b, i, err_l)
        _add_stats(st, v, formats.round_bf16(x), implied, bar, tolerance(w))
    return st


def check_merged(w, gpu_o, gpu_l, o, l, rows, tag="", extra=None):
    """The merged BF16 output against the two-rounding expectation of the exact
    per-rank partials ``o[W, ...]``, ``l[W, ...]``: each element must be the
    rounding of a real within the bar of a merge of admissible per-rank BF16
    values (the rounded exact value, or one step from it where the exact value
    lies within the bar of that rounding boundary); LSE within 1e-3 of the
    exact merged LSE.  Per-rank ``extra[W, ...]`` widens each rank's bar, and
    the merged bar by its LSE-weighted merge.  Returns error statistics
    against the expectation."""
    st = _new_stats()
    for b, i in rows:
        _, _, e, lse = parity.merged_expectation(o[:, b, i], l[:, b, i])
        v = gpu_o[b, i]
        emp = np.isneginf(lse)
        assert np.all(np.isneginf(gpu_l[b, i][emp])) and np.all(v[emp] == 0.0), (tag, b, i)
        if extra is None:
            bar_r = bar = tolerance(w)
        else:
            ex = np.where(np.isfinite(l[:, b, i])[..., None], extra[:, b, i], 0.0)
            bar_r = tolerance(w) + ex
            bar = tolerance(w) + A.merge_ranks(ex, l[:, b, i])[0]
        implied = parity.merged_gap(v, o[:, b, i], l[:, b, i], bar_r)
        ok = implied <= bar
        assert ok.all(), (tag, b, i, int((~ok).sum()), float(np.abs(v - e)[~ok].max()))
        assert np.abs(gpu_l[b, i][~emp] - lse[~emp]).max(initial=0.0) <= LSE_TOL, (tag, b, i)
        _add_stats(st, v, e, implied, bar, tolerance(w))
    return st


def count_rejected(w, gpu_o, o, l, rows):
    """Merged output elements the acceptance rule rejects (the negative control),
    and the largest |GPU - expectation| among the selected rows."""
    bar = tolerance(w)
    bad, total, worst = 0, 0, 0.0
    for b, i in rows:
        _, _, e, _ = parity.merged_expectation(o[:, b, i], l[:, b, i])
        v = gpu_o[b, i]
        ok = parity.accept_merged(v, o[:, b, i], l[:, b, i], bar)
        bad += int((~ok).sum())
        total += v.size
        worst = max(worst, float(np.abs(v - e).max()))
    return bad, total, worst


def fmt_stats(st):
    return (f"{st['elements']} elements: {st['differ']} differ from the rounded expectation "
            f"({st['one_step']} by one BF16 step), {st['beyond_bar']} by more than the bar; "
            f"max |d| {st['max_abs']:.3e}, {st['max_abs_no_flip']:.3e} without one-step flips; "
            f"largest implied arithmetic error {st['max_implied']:.3e} "
            f"({st['beyond_plain']} beyond the unwidened bar)")
