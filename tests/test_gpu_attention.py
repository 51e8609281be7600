"""Per-rank segmented attention, segment merge and cross-rank merge on the GPU
against the float64 oracle.

Tolerances: outputs max-abs 1.5e-2 with an FP8 cache and 5e-3 with a BF16
cache, on top of the BF16 output format's own rounding (half a BF16 ulp of the
exact value, and for the merged output also each rank's rounded partial
weighted by its merge weight); LSE abs 1e-3.  The oracle reads the same
decoded cache values, so FP8 quantisation is not part of the error; what
remains is BF16 rounding of the probabilities and of the outputs plus fp32
accumulation.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import layout
from synth import make_config, make_workload
from gpu_util import (LSE_TOL, bf16_to_f64, oracle_latents, oracle_q, output_bound,
                      run_group, tolerance)

pytestmark = pytest.mark.gpu


def _compare_rank(w, grp, r, rows, boundary=layout.verify_row_boundary, q_format="split"):
    o, l = A.verify_attention(oracle_q(w, q_format), oracle_latents(w), w.ctx_lens, w.softmax_scale,
                              world=w.world, interleave=w.interleave, rank=r, rows=rows,
                              boundary=boundary)
    go = bf16_to_f64(grp.out_ranks[r])
    gl = grp.lse_ranks[r].cpu().numpy().astype(np.float64)
    for b, i in rows:
        emp = np.isneginf(l[b, i])
        # empty (row, rank): exactly zero output and -inf LSE
        assert np.all(np.isneginf(gl[b, i][emp]))
        assert np.all(go[b, i][emp] == 0.0)
        assert np.all(np.isfinite(gl[b, i][~emp]))
        if (~emp).any():
            ex = o[b, i][~emp]
            err_o = np.abs(go[b, i][~emp] - ex)
            bad = err_o > output_bound(w, ex)
            assert not bad.any(), (r, b, i, err_o.max(), err_o[bad].max())
            err_l = np.abs(gl[b, i][~emp] - l[b, i][~emp]).max()
            assert err_l <= LSE_TOL, (r, b, i, err_l)


def _compare_merged(w, grp, rows, boundary=layout.verify_row_boundary, q_format="split"):
    q, lat = oracle_q(w, q_format), oracle_latents(w)
    o, l = A.verify_attention(q, lat, w.ctx_lens, w.softmax_scale, rows=rows, boundary=boundary)
    ro, rl = [], []
    for r in range(w.world):
        a, c = A.verify_attention(q, lat, w.ctx_lens, w.softmax_scale, world=w.world,
                                  interleave=w.interleave, rank=r, rows=rows, boundary=boundary)
        ro.append(a)
        rl.append(c)
    ro, rl = np.stack(ro), np.stack(rl)
    go = bf16_to_f64(grp.out)
    gl = grp.lse.cpu().numpy().astype(np.float64)
    worst = 0.0
    for b, i in rows:
        wts = np.where(np.isneginf(rl[:, b, i]), 0.0, np.exp(rl[:, b, i] - l[b, i][None, :]))
        err = np.abs(go[b, i] - o[b, i])
        bound = output_bound(w, o[b, i], ro[:, b, i], wts)
        assert not (err > bound).any(), (b, i, err.max())
        worst = max(worst, err.max())
        assert np.abs(gl[b, i] - l[b, i]).max() <= LSE_TOL
    return worst


@pytest.mark.parametrize("k,groups", [(1, 0), (1, 1), (1, 3), (2, 0), (2, 7), (2, 1)])
def test_small_configs_full(k, groups):
    w = make_config(k)
    print(f"config {k} groups {groups}", flush=True)
    grp, _ = run_group(w, groups=groups)
    assert grp.errors() == 0
    rows = [(b, i) for b in range(w.batch) for i in range(w.qlen)]
    for r in range(w.world):
        _compare_rank(w, grp, r, rows)
    _compare_merged(w, grp, rows)


def _sample_rows(w, n, seed):
    rng = np.random.default_rng(seed)
    bs = rng.choice(w.batch, size=min(n, w.batch), replace=False)
    return [(int(b), int(rng.integers(w.qlen))) for b in bs] + [(int(bs[0]), w.qlen - 1), (int(bs[0]), 0)]


def test_config4_verify_interleave16():
    # log-uniform contexts, interleave 16, qlen 5: empty (row, rank) pairs occur
    w = make_config(4)
    print(f"config 4: {w.name}", flush=True)
    grp, _ = run_group(w)
    assert grp.errors() == 0
    shortest = int(np.argmin(w.ctx_lens))
    longest = int(np.argmax(w.ctx_lens))
    rows = sorted(set(_sample_rows(w, 5, 44) + [(shortest, i) for i in range(w.qlen)]
                      + [(longest, w.qlen - 1)]))
    for r in (0, 3, 7):
        _compare_rank(w, grp, r, rows)
    _compare_merged(w, grp, rows)


@pytest.mark.parametrize("k", [3, 5])
def test_large_configs_sampled(k):
    w = make_config(k)
    print(f"config {k}: {w.name}", flush=True)
    grp, _ = run_group(w)
    assert grp.errors() == 0
    rows = _sample_rows(w, 2, 40 + k)
    for r in (0, w.world - 1):
        _compare_rank(w, grp, r, rows)
    _compare_merged(w, grp, rows)


@pytest.mark.parametrize("kv_format,q_format", [("bf16", "split"), ("fp8_e4m3", "split"),
                                                 ("fp8_e4m3", "fp8")])
def test_ragged_tiles_and_tiny_contexts(kv_format, q_format):
    # M = 3 * 40 = 120 (one ragged tile); contexts down to qlen (first row sees one token);
    # interleave 4 over 8 ranks leaves most ranks empty for short rows.  With an FP8 cache
    # the sequences' head-rows start inside the split query's 32-row blocks (120 b), so
    # a wave's query rows straddle two blocks
    ctx = np.array([3, 4, 5, 9, 33, 64, 65, 200, 1000])
    w = make_workload(name="ragged", world=8, interleave=4, batch=len(ctx), qlen=3, heads=40,
                      block_size=16, kv_format=kv_format, ctx=ctx, table="random",
                      max_local_pages=16, seed=77)
    print(f"ragged tiles {kv_format} q_format {q_format}", flush=True)
    for groups in (0, 5):
        grp, _ = run_group(w, groups=groups, q_format=q_format)
        assert grp.errors() == 0
        rows = [(b, i) for b in range(w.batch) for i in range(w.qlen)]
        for r in range(w.world):
            _compare_rank(w, grp, r, rows, q_format=q_format)
        _compare_merged(w, grp, rows, q_format=q_format)


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
    rows = _sample_rows(w, 48, 93)
    for r in range(w.world):
        _compare_rank(w, grp, r, rows)
    _compare_merged(w, grp, rows)


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
    rows = [(b, i) for b in range(w.batch) for i in range(w.qlen)]
    for r in range(w.world):
        _compare_rank(w, grp, r, rows)
    _compare_merged(w, grp, rows)


@pytest.mark.parametrize("world,interleave,heads,qlen,kv_format", [
    (1, 1, 16, 3, "bf16"),       # no context parallelism: one rank owns every token
    (3, 2, 1, 1, "fp8_e4m3"),    # M = 1: one valid head-row in the whole tile
    (3, 1, 3, 7, "fp8_e4m3"),    # M = 21: odd world, rows straddle the split's 32-row blocks
    (2, 1, 7, 2, "bf16"),
])
def test_degenerate_shapes(world, interleave, heads, qlen, kv_format):
    ctx = np.array([qlen, qlen + 1, 40, 257, 700])
    w = make_workload(name="degenerate", world=world, interleave=interleave, batch=len(ctx),
                      qlen=qlen, heads=heads, block_size=16, kv_format=kv_format, ctx=ctx,
                      table="random", max_local_pages=64, seed=97)
    print(f"W={world} S={interleave} H={heads} q={qlen} {kv_format}", flush=True)
    grp, _ = run_group(w)
    assert grp.errors() == 0
    rows = [(b, i) for b in range(w.batch) for i in range(w.qlen)]
    for r in range(w.world):
        _compare_rank(w, grp, r, rows)
    _compare_merged(w, grp, rows)
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
    rows = [(b, i) for b in range(w.batch) for i in range(w.qlen)]
    _compare_rank(w, grp, 0, rows)
    _compare_merged(w, grp, rows)


def test_negative_control_boundary():
    # the GPU result matches the correct boundary and misses both mutated ones
    w = make_config(2)
    grp, _ = run_group(w)
    rows = [(0, i) for i in range(w.qlen)] + [(1, i) for i in range(w.qlen)]
    _compare_merged(w, grp, rows)
    go = bf16_to_f64(grp.out)
    for mutant in (lambda c, q, i: c - q, lambda c, q, i: c):
        outs, lses = [], []
        for r in range(w.world):
            o, l = A.verify_attention(oracle_q(w), oracle_latents(w), w.ctx_lens, w.softmax_scale,
                                      world=w.world, interleave=w.interleave, rank=r, rows=rows,
                                      boundary=mutant)
            outs.append(o)
            lses.append(l)
        mo, _ = A.merge_ranks(np.stack(outs), np.stack(lses))
        diff = max(np.abs(go[b, i] - mo[b, i]).max() for b, i in rows)
        assert diff > tolerance(w), diff


# ------------------------------------------------ bidirectional draft block ----

@pytest.mark.parametrize("k,groups", [(1, 0), (2, 0), (2, 7)])
def test_block_rows_full(k, groups):
    # every row of a sequence sees the whole cache ("Context Parallel Guide",
    # DSpark): same kernels, degenerate row boundary
    w = make_config(k)
    print(f"config {k} groups {groups} block rows", flush=True)
    grp, _ = run_group(w, groups=groups, row_boundary="block")
    assert grp.errors() == 0
    rows = [(b, i) for b in range(w.batch) for i in range(w.qlen)]
    for r in range(w.world):
        _compare_rank(w, grp, r, rows, boundary=layout.block_row_boundary)
    _compare_merged(w, grp, rows, boundary=layout.block_row_boundary)


@pytest.mark.parametrize("k,groups", [(2, 0), (2, 5)])
def test_fp8_query_full(k, groups):
    # the quantised-query variant against attention with the same E4M3 query
    w = make_config(k)
    print(f"config {k} groups {groups} q_format fp8", flush=True)
    grp, _ = run_group(w, groups=groups, q_format="fp8")
    assert grp.errors() == 0
    rows = [(b, i) for b in range(w.batch) for i in range(w.qlen)]
    for r in range(w.world):
        _compare_rank(w, grp, r, rows, q_format="fp8")
    _compare_merged(w, grp, rows, q_format="fp8")


@pytest.mark.parametrize("k", [3, 4])
def test_fp8_query_sampled(k):
    w = make_config(k)
    print(f"config {k}: {w.name} q_format fp8", flush=True)
    grp, _ = run_group(w, q_format="fp8")
    assert grp.errors() == 0
    rows = _sample_rows(w, 3, 60 + k)
    for r in (0, w.world - 1):
        _compare_rank(w, grp, r, rows, q_format="fp8")
    _compare_merged(w, grp, rows, q_format="fp8")
