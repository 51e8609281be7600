"""The verification step captured as a HIP graph and replayed.

The bench times the step as graph replays, so the captured step must give
exactly the eager result on every replay: the kernels are deterministic (no
atomics on the data path, fixed merge orders), so each replay is compared bit
for bit with an eager forward, with eager work and synchronisations between
the replays.
"""
import numpy as np
import pytest
import torch

from synth import make_config, make_workload
from gpu_util import run_group

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("k", [1, 2])
def test_step_graph_replays_match_eager(k):
    w = make_config(k)
    print(f"config {k}: {w.name} graph replay", flush=True)
    grp, d = run_group(w)
    ref = [t.clone() for t in (grp.out, grp.lse, grp.out_ranks, grp.lse_ranks)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        grp.forward(d["q"], d["ctx_lens"], d["block_table"], w.kv_scale, w.softmax_scale)
    for i in range(3):
        for t in (grp.out, grp.out_ranks):
            t.fill_(float("nan"))
        grp.lse.zero_()
        grp.lse_ranks.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip((grp.out, grp.lse, grp.out_ranks, grp.lse_ranks), ref):
            assert torch.equal(got, want), (k, i)
        # an eager step between replays, then the same check on its output
        grp.forward(d["q"], d["ctx_lens"], d["block_table"], w.kv_scale, w.softmax_scale)
        torch.cuda.synchronize()
        assert torch.equal(grp.out, ref[0]) and torch.equal(grp.lse, ref[1])
    assert grp.errors() == 0


def _odd_world(kv_format):
    """Three ranks (two on the first stream, one on the second), interleave 2, ragged heads."""
    ctx = np.array([5, 6, 40, 257, 700, 1500])
    return make_workload(name=f"w3_{kv_format}", world=3, interleave=2, batch=len(ctx), qlen=5,
                         heads=21, block_size=16, kv_format=kv_format, ctx=ctx, table="random",
                         max_local_pages=64, seed=131)


@pytest.mark.parametrize("k", [1, 2, 4, "w3_bf16", "w3_fp8"])
def test_two_stream_step_matches_one_stream(k):
    """The ranks issued over two streams (the query split and the odd ranks on a second
    stream with its own split-KV workspace), eagerly and as replays of a captured graph,
    give the one-stream forward's result bit for bit: the launches and their inputs are the
    same, only their order across streams differs."""
    if isinstance(k, str):
        w = _odd_world("bf16" if k.endswith("bf16") else "fp8_e4m3")
    else:
        w = make_config(k)
    print(f"config {k}: {w.name} two-stream step", flush=True)
    grp, d = run_group(w)
    ref = [t.clone() for t in (grp.out, grp.lse, grp.out_ranks, grp.lse_ranks)]
    side = torch.cuda.Stream()
    args = (d["q"], d["ctx_lens"], d["block_table"], w.kv_scale, w.softmax_scale)

    def clear():
        for t in (grp.out, grp.out_ranks):
            t.fill_(float("nan"))
        grp.lse.zero_()
        grp.lse_ranks.zero_()
        torch.cuda.synchronize()

    def check(tag):
        for got, want in zip((grp.out, grp.lse, grp.out_ranks, grp.lse_ranks), ref):
            assert torch.equal(got, want), (k, tag)

    clear()
    grp.forward_two_streams(*args, side)
    torch.cuda.synchronize()
    check("eager")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        grp.forward_two_streams(*args, side)
    for i in range(3):
        clear()
        graph.replay()
        torch.cuda.synchronize()
        check(f"replay {i}")
        # a one-stream eager step between replays
        grp.forward(*args)
        torch.cuda.synchronize()
        check(f"eager after replay {i}")
    assert grp.errors() == 0
