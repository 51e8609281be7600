"""Per-rank segmented attention, segment merge and cross-rank merge on the GPU
against the float64 oracle.

Expected values take the oracle's exact per-rank partials through the two
BF16 roundings the method applies (each rank's output, then the merged
output; ``oracle.parity``).  An output element passes when it is the BF16
rounding of a real within the bar of that expectation -- max-abs 1.5e-2 with
an FP8 cache, 5e-3 with a BF16 cache -- where a rank's exact value that lies
within the bar of a rounding boundary may reach the merge one BF16 step
away.  LSE abs 1e-3.  The oracle reads the same decoded cache values, so FP8
quantisation is not part of the error.
"""
import numpy as np
import pytest
import torch

from oracle import formats, layout
from synth import make_config, make_workload
from gpu_util import (bf16_to_f64, check_merged, check_rank, count_rejected, fmt_stats,
                      rank_expectations, run_group)

pytestmark = pytest.mark.gpu


def _check_all(w, grp, rows, boundary=layout.verify_row_boundary, q_format="split", ranks=None,
               merged=True, tag="", p_bound=False):
    """Every selected rank's output and LSE, then the merged output, on ``rows``.
    ``p_bound`` widens the bar by the bound on E4M3 probabilities
    (``gpu_util.fp8_probability_bound``)."""
    if p_bound:
        o, l, extra = rank_expectations(w, rows, q_format=q_format, boundary=boundary, p_bound=True)
    else:
        (o, l), extra = rank_expectations(w, rows, q_format=q_format, boundary=boundary), None
    ranks = range(w.world) if ranks is None else ranks
    worst = None
    for r in ranks:
        go = bf16_to_f64(grp.out_ranks[r])
        gl = grp.lse_ranks[r].cpu().numpy().astype(np.float64)
        st = check_rank(w, go, gl, o[r], l[r], rows, tag=f"{tag} rank {r}",
                        extra=None if extra is None else extra[r])
        if worst is None or st["max_implied"] > worst[1]["max_implied"]:
            worst = (r, st)
    if worst is not None:
        print(f"{tag} worst rank {worst[0]}: {fmt_stats(worst[1])}", flush=True)
    if merged:
        st = check_merged(w, bf16_to_f64(grp.out), grp.lse.cpu().numpy().astype(np.float64), o, l, rows,
                          tag=f"{tag} merged", extra=extra)
        print(f"{tag} merged: {fmt_stats(st)}", flush=True)
    return o, l


def _all_rows(w):
    return [(b, i) for b in range(w.batch) for i in range(w.qlen)]


@pytest.mark.parametrize("k,groups", [(1, 0), (1, 1), (1, 3), (2, 0), (2, 7), (2, 1)])
def test_small_configs_full(k, groups):
    w = make_config(k)
    print(f"config {k} groups {groups}", flush=True)
    grp, _ = run_group(w, groups=groups)
    assert grp.errors() == 0
    _check_all(w, grp, _all_rows(w), tag=f"config {k} groups {groups}")


def _sample_rows(w, n, seed):
    rng = np.random.default_rng(seed)
    bs = rng.choice(w.batch, size=min(n, w.batch), replace=False)
    return [(int(b), int(rng.integers(w.qlen))) for b in bs] + [(int(bs[0]), w.qlen - 1), (int(bs[0]), 0)]


@pytest.mark.parametrize("k", [3, 4, 5])
def test_large_configs_every_row(k):
    # every verify row of every sequence, every rank's partial and the merged
    # output, at full size in the launch configuration the bench times.  On
    # workload 4 (log-uniform contexts, interleave 16, qlen 5) empty (row, rank)
    # pairs occur and the shortest and longest sequences are among the rows
    w = make_config(k)
    print(f"config {k}: {w.name}", flush=True)
    grp, _ = run_group(w)
    assert grp.errors() == 0
    _check_all(w, grp, _all_rows(w), tag=f"config {k}")


@pytest.mark.parametrize("kv_format,q_format,p_format", [("bf16", "split", "split"),
                                                          ("fp8_e4m3", "split", "split"),
                                                          ("fp8_e4m3", "fp8", "split"),
                                                          ("fp8_e4m3", "split", "fp8"),
                                                          ("fp8_e4m3", "fp8", "fp8")])
def test_ragged_tiles_and_tiny_contexts(kv_format, q_format, p_format):
    # M = 3 * 40 = 120 (one ragged tile); contexts down to qlen (first row sees one token);
    # interleave 4 over 8 ranks leaves most ranks empty for short rows.  With an FP8 cache
    # the sequences' head-rows start inside the split query's 32-row blocks (120 b), so
    # a wave's query rows straddle two blocks
    ctx = np.array([3, 4, 5, 9, 33, 64, 65, 200, 1000])
    w = make_workload(name="ragged", world=8, interleave=4, batch=len(ctx), qlen=3, heads=40,
                      block_size=16, kv_format=kv_format, ctx=ctx, table="random",
                      max_local_pages=16, seed=77)
    print(f"ragged tiles {kv_format} q_format {q_format} p_format {p_format}", flush=True)
    for groups in (0, 5):
        grp, _ = run_group(w, groups=groups, q_format=q_format, p_format=p_format)
        assert grp.errors() == 0
        _check_all(w, grp, _all_rows(w), q_format=q_format, p_bound=p_format == "fp8",
                   tag=f"ragged {kv_format} q {q_format} p {p_format} groups {groups}")


@pytest.mark.parametrize("B,qlen,kv_format", [(1024, 3, "bf16"), (5000, 1, "fp8_e4m3")])
def test_partition_outside_lds(B, qlen, kv_format):
    # batches whose work partition and row lengths do not fit in LDS next to the stage tiles and
    # staging areas: the kernel reads them from global memory.  With more than 1024 verify rows
    # the metadata also takes its two-kernel path.  Short contexts keep the oracle cheap
    ctx = np.random.default_rng(5).integers(qlen, 120, B)
    w = make_workload(name="bigbatch", world=2, interleave=1, batch=B, qlen=qlen, heads=8,
                      block_size=16, kv_format=kv_format, ctx=ctx, table="shuffled",
                      max_local_pages=8, seed=91)
    print(f"partition outside LDS: B={B} qlen={qlen} {kv_format}", flush=True)
    grp, _ = run_group(w)
    assert grp.errors() == 0
    _check_all(w, grp, _sample_rows(w, 48, 93), tag=f"B={B}")


@pytest.mark.parametrize("world", [1, 2])
@pytest.mark.parametrize("q_format,p_format", [("split", "split"), ("split", "fp8"), ("fp8", "split")])
def test_windows_at_half_stage_edges(world, q_format, p_format):
    # With an FP8 cache each 32-token tile half has its own probability scale;
    # rows whose rank-local window ends just before, at and just after a
    # 32-token boundary leave a half wholly or partly masked (qlen 3: row i
    # of a sequence sees ctx - 2 + i tokens)
    ctx = np.array([33, 34, 35, 65, 66, 67, 97, 98, 130, 200]) * world
    w = make_workload(name="half_edges", world=world, interleave=1, batch=len(ctx), qlen=3, heads=16,
                      block_size=16, kv_format="fp8_e4m3", ctx=ctx, table="random",
                      max_local_pages=16, seed=99)
    print(f"half-stage edges W={world} q {q_format} p {p_format}", flush=True)
    for groups in (0, 5):
        grp, _ = run_group(w, groups=groups, q_format=q_format, p_format=p_format)
        assert grp.errors() == 0
        _check_all(w, grp, _all_rows(w), q_format=q_format, p_bound=p_format == "fp8",
                   tag=f"half edges W={world} q {q_format} p {p_format} groups {groups}")


@pytest.mark.parametrize("block_size", [1, 48, 512])
@pytest.mark.parametrize("kv_format", ["bf16", "fp8_e4m3"])
def test_block_sizes(block_size, kv_format):
    # subpage P = min(128, lowbit(block size)): P = 1 (a page per token, 32 page lookups per
    # stage), P = 16 with three subpages per block, and P = 128
    ctx = np.array([5, 300, 1100])
    w = make_workload(name=f"bs{block_size}", world=2, interleave=1, batch=3, qlen=3, heads=16,
                      block_size=block_size, kv_format=kv_format, ctx=ctx, table="random",
                      max_local_pages=600, seed=95)
    print(f"block size {block_size} {kv_format}", flush=True)
    grp, _ = run_group(w)
    assert grp.errors() == 0
    _check_all(w, grp, _all_rows(w), tag=f"block size {block_size} {kv_format}")


@pytest.mark.parametrize("world,interleave,heads,qlen,kv_format,p_format", [
    (1, 1, 16, 3, "bf16", "split"),      # no context parallelism: one rank owns every token
    (3, 2, 1, 1, "fp8_e4m3", "split"),   # M = 1: one valid head-row in the whole tile
    (3, 1, 3, 7, "fp8_e4m3", "split"),   # M = 21: odd world, rows straddle the split's 32-row blocks
    (2, 1, 7, 2, "bf16", "split"),
    (3, 2, 1, 1, "fp8_e4m3", "fp8"),
    (3, 1, 3, 7, "fp8_e4m3", "fp8"),
])
def test_degenerate_shapes(world, interleave, heads, qlen, kv_format, p_format):
    ctx = np.array([qlen, qlen + 1, 40, 257, 700])
    w = make_workload(name="degenerate", world=world, interleave=interleave, batch=len(ctx),
                      qlen=qlen, heads=heads, block_size=16, kv_format=kv_format, ctx=ctx,
                      table="random", max_local_pages=64, seed=97)
    print(f"W={world} S={interleave} H={heads} q={qlen} {kv_format} p {p_format}", flush=True)
    grp, _ = run_group(w, p_format=p_format)
    assert grp.errors() == 0
    _check_all(w, grp, _all_rows(w), p_bound=p_format == "fp8",
               tag=f"W={world} S={interleave} H={heads} q={qlen} p {p_format}")
    if world == 1:
        # the merge of a single rank returns that rank's result
        assert torch.equal(grp.out, grp.out_ranks[0]) and torch.equal(grp.lse, grp.lse_ranks[0])


def test_all_ranks_but_one_empty():
    # every context shorter than the interleave: only rank 0 owns tokens
    ctx = np.array([5, 8, 12, 16])
    w = make_workload(name="rank0only", world=8, interleave=16, batch=4, qlen=2, heads=16,
                      block_size=16, kv_format="fp8_e4m3", ctx=ctx, table="shuffled",
                      max_local_pages=2, seed=78)
    grp, _ = run_group(w)
    for r in range(1, 8):
        assert torch.all(grp.lse_ranks[r] == float("-inf"))
        assert torch.all(grp.out_ranks[r] == 0)
    _check_all(w, grp, _all_rows(w), ranks=[0], tag="rank 0 only")


@pytest.mark.parametrize("where,bad_page", [("interior", 1 << 30), ("interior", -5), ("last", 1 << 30)])
def test_page_outside_pool(where, bad_page):
    # a page id of a sequence's longest verify row points outside the pool:
    # its tokens read as the zero row (no read outside the pool), the kernel
    # raises the page-range bit, and no other sequence's output or LSE moves
    # (the rows of one sequence share the tiles that row's table loads).  An
    # interior page sits in a stage the one-block score phase loads; the last
    # page in the row's last stage.
    from decode_context_parallelism_amd import _lib, ops
    w = make_config(2)
    grp, _ = run_group(w)
    r = 0
    meta = grp.meta[r]
    P = ops.subpage_size(w.block_size)
    lens = meta.row_local_len.cpu().numpy()
    row = int(np.argmax(lens))
    npg = (int(lens[row]) + P - 1) // P
    assert npg >= 8
    idx = npg // 2 if where == "interior" else npg - 1
    out0, lse0 = grp.out_ranks[r].clone(), grp.lse_ranks[r].clone()
    assert int(meta.err.item()) == 0
    b = row // w.qlen
    meta.page_table[b * w.qlen:(b + 1) * w.qlen, idx] = bad_page   # whichever row's table loads
    grp.rank_attention_split(r, w.kv_scale, w.softmax_scale)
    torch.cuda.synchronize()
    assert int(meta.err.item()) & _lib.ERR_PAGE_RANGE
    out1, lse1 = grp.out_ranks[r], grp.lse_ranks[r]
    assert torch.isfinite(out1[b].float()).all() and torch.isfinite(lse1[b]).all()
    keep = torch.ones(w.batch, dtype=torch.bool, device=out1.device)
    keep[b] = False
    assert torch.equal(out1[keep], out0[keep])
    assert torch.equal(lse1[keep], lse0[keep])


@pytest.mark.parametrize("k", [1, 2, 4])
def test_negative_control_boundary(k):
    # "[ROCm][MLA][DCP] Support causal multi-token verification", "Validation":
    # with the row boundary reverted to the committed prefix, the causal
    # reference must fail.  The GPU result passes against the correct boundary
    # and the same acceptance rule rejects it against both mutated ones (every
    # row sees only the committed prefix; every row sees the whole context)
    w = make_config(k)
    grp, _ = run_group(w)
    assert grp.errors() == 0
    if k == 4:
        # the shortest sequences, where one token more or less moves the output
        rows = [(int(b), i) for b in np.argsort(w.ctx_lens)[:6] for i in range(w.qlen)]
    else:
        rows = _all_rows(w)
    _check_all(w, grp, rows, ranks=[], tag=f"config {k} correct boundary")
    go = bf16_to_f64(grp.out)
    for name, mutant in (("committed prefix", lambda c, q, i: c - q), ("whole context", lambda c, q, i: c)):
        o, l = rank_expectations(w, rows, boundary=mutant)
        bad, total, worst = count_rejected(w, go, o, l, rows)
        print(f"config {k} negative control ({name}): {bad} of {total} elements rejected, "
              f"max |d| {worst:.4f}", flush=True)
        assert bad > 0, (name, worst)


# ------------------------------------------------ bidirectional draft block ----

@pytest.mark.parametrize("k,groups", [(1, 0), (2, 0), (2, 7)])
def test_block_rows_full(k, groups):
    # every row of a sequence sees the whole cache ("Context Parallel Guide",
    # DSpark): same kernels, degenerate row boundary
    w = make_config(k)
    print(f"config {k} groups {groups} block rows", flush=True)
    grp, _ = run_group(w, groups=groups, row_boundary="block")
    assert grp.errors() == 0
    _check_all(w, grp, _all_rows(w), boundary=layout.block_row_boundary, tag=f"config {k} block rows")


@pytest.mark.parametrize("k,groups", [(2, 0), (2, 5)])
def test_fp8_query_full(k, groups):
    # the quantised-query variant against attention with the same E4M3 query
    w = make_config(k)
    print(f"config {k} groups {groups} q_format fp8", flush=True)
    grp, _ = run_group(w, groups=groups, q_format="fp8")
    assert grp.errors() == 0
    _check_all(w, grp, _all_rows(w), q_format="fp8", tag=f"config {k} groups {groups} fp8 query")


@pytest.mark.parametrize("k", [3, 4])
def test_fp8_query_sampled(k):
    w = make_config(k)
    print(f"config {k}: {w.name} q_format fp8", flush=True)
    grp, _ = run_group(w, q_format="fp8")
    assert grp.errors() == 0
    _check_all(w, grp, _sample_rows(w, 3, 60 + k), ranks=(0, w.world - 1), q_format="fp8",
               tag=f"config {k} fp8 query")


def _spiked_workload(seed, kv_format="fp8_e4m3"):
    """FP8 workload whose cache holds a few keys aligned with one head's query
    at full E4M3 magnitude: that head's scores jump by about 240 (base 2)
    at those tokens, far past any running maximum of ordinary N(0, 1) data.
    A spike inside a later stage makes the row move its reference mid-piece;
    one in the first stage leaves every later stage far below it."""
    w = make_workload(name="spiked", world=2, interleave=1, batch=2, qlen=3, heads=16, block_size=64,
                      kv_format=kv_format, ctx=("fixed", 2000), table="shuffled", max_local_pages=24,
                      seed=seed)
    q = formats.decode_bf16(w.q_bits)
    top = 0x7E   # E4M3 code of 448
    for b, pos, h in ((0, 1200, 3), (0, 10, 7), (1, 700, 0), (1, 1600, 0), (1, 1601, 12)):
        sign = q[b, 0, h] < 0
        w.kv[w.seq_start[b] + pos] = np.where(sign, top | 0x80, top).astype(np.uint8)
    return w


@pytest.mark.parametrize("groups", [0, 5])
@pytest.mark.parametrize("p_format", ["split", "fp8"])
def test_score_jumps(groups, p_format):
    w = _spiked_workload(3001)
    print(f"spiked workload groups {groups} p_format {p_format}", flush=True)
    grp, _ = run_group(w, groups=groups, p_format=p_format)
    assert grp.errors() == 0
    _check_all(w, grp, _all_rows(w), p_bound=p_format == "fp8",
               tag=f"spiked groups {groups} p {p_format}")


# ------------------------------------------------ E4M3 probabilities ----
#
# p_format "fp8" rounds each stage's probabilities to E4M3 against a per-stage
# power-of-two scale and multiplies them with the E4M3 cache on FP8 matrix
# units.  Each weight carries up to 2^-4 relative error, so a row's output
# error grows as its effective token count 1 / sum w^2 falls.  On the
# 1M-context workload (131,072 tokens a rank, effective counts in the
# hundreds at the least) the output stays within the standard 1.5e-2 bar of
# exact attention.  On the decode workload (16,384 tokens a rank) a row with
# an effective count near 80 already leaves it (1.7e-2 in a float64
# emulation of the same rounding), and shorter rows further: there, and on
# every smaller workload, the bar is widened by the rounding bound of
# gpu_util.fp8_probability_bound, and the count of elements past the
# unwidened bar is printed.

@pytest.mark.parametrize("q_format,groups", [("split", 0), ("split", 5), ("fp8", 0)])
def test_fp8_probabilities_full(q_format, groups):
    w = make_config(2)
    print(f"config 2 groups {groups} q_format {q_format} p_format fp8", flush=True)
    grp, _ = run_group(w, groups=groups, q_format=q_format, p_format="fp8")
    assert grp.errors() == 0
    _check_all(w, grp, _all_rows(w), q_format=q_format, p_bound=True,
               tag=f"config 2 groups {groups} q {q_format} p fp8")


@pytest.mark.parametrize("q_format", ["split", "fp8"])
def test_fp8_probabilities_long_rows(q_format):
    # the standard bar against exact attention, no widening
    w = make_config(5)
    print(f"config 5: {w.name} q_format {q_format} p_format fp8", flush=True)
    grp, _ = run_group(w, q_format=q_format, p_format="fp8")
    assert grp.errors() == 0
    _check_all(w, grp, _sample_rows(w, 3, 75), ranks=(0, w.world - 1), q_format=q_format,
               tag=f"config 5 q {q_format} p fp8")


@pytest.mark.parametrize("k", [3, 4])
def test_fp8_probabilities_sampled(k):
    # decode rows (16,384 tokens a rank; the sample holds sequence 15, whose
    # row leaves the unwidened bar) and log-uniform contexts from 8 tokens
    # with the shortest sequences among the rows
    w = make_config(k)
    print(f"config {k}: {w.name} p_format fp8", flush=True)
    grp, _ = run_group(w, p_format="fp8")
    assert grp.errors() == 0
    rows = _sample_rows(w, 3, 70 + k)
    if k == 4:
        rows += [(int(b), w.qlen - 1) for b in np.argsort(w.ctx_lens)[:2]]
    _check_all(w, grp, rows, ranks=(0, w.world - 1), p_bound=True, tag=f"config {k} p fp8")
