"""Verify-view metadata and KV write on the GPU: bit-exact against the oracle.

Expected values come from ``oracle.layout`` (brute-force enumeration of global
positions); inputs from ``synth``.  Every call goes through the C ABI.
"""
import numpy as np
import pytest
import torch

from oracle import layout
from synth import make_config, make_workload
from gpu_util import device_inputs, geometry

pytestmark = pytest.mark.gpu


def _ops():
    from decode_context_parallelism_amd import ops
    return ops


def _gpu_meta(w, rank, **geo):
    ops = _ops()
    g = geometry(w, **geo)
    meta = ops.RankMetadata(g)
    ops.build_metadata(g, rank, torch.from_numpy(w.ctx_lens).cuda(),
                       torch.from_numpy(w.block_table).cuda(), meta)
    torch.cuda.synchronize()
    return meta


def _check_rank(w, rank, meta, max_local_pages=None):
    lens, table, last = layout.row_metadata(
        w.ctx_lens, w.block_table, world=w.world, interleave=w.interleave,
        block_size=w.block_size, qlen=w.qlen, rank=rank,
        max_local_pages=max_local_pages or w.max_local_pages)
    assert np.array_equal(meta.row_local_len.cpu().numpy(), lens)
    assert np.array_equal(meta.page_table.cpu().numpy(), table)
    assert np.array_equal(meta.last_page_len.cpu().numpy(), last)
    assert int(meta.err.item()) == 0


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_metadata_configs_all_ranks(k):
    w = make_config(k, with_kv=False)
    print(f"config {k}: {w.name}", flush=True)
    for r in range(w.world):
        _check_rank(w, r, _gpu_meta(w, r))


SWEEP = [(bs, W, S, q) for bs in (1, 16, 48, 64, 128, 192, 256, 512)
         for (W, S) in ((2, 1), (8, 1), (4, 4), (8, 16), (3, 2))
         for q in (1, 3, 5) if bs % S == 0 and S <= bs]


@pytest.mark.parametrize("bs,W,S,q", SWEEP)
def test_metadata_sweep(bs, W, S, q):
    rng = np.random.default_rng(bs * 1000 + W * 100 + S * 10 + q)
    B = 4
    ctx = rng.integers(q, 5 * bs * W + 50, size=B)
    P = layout.subpage_size(bs)
    w = make_workload(name="sweep", world=W, interleave=S, batch=B, qlen=q, heads=4, block_size=bs,
                      kv_format="fp8_e4m3", ctx=ctx, table="random", max_local_pages=1,
                      seed=int(rng.integers(1 << 30)), extra_cols=2, with_kv=False)
    mlp = w.block_table.shape[1] * (bs // P) + 3     # room to spare: unused entries must be -1
    for r in range(W):
        _check_rank(w, r, _gpu_meta(w, r, max_local_pages=mlp), max_local_pages=mlp)


def test_metadata_error_bits_and_clamps():
    ops = _ops()
    w = make_workload(name="err", world=2, interleave=1, batch=3, qlen=3, heads=4, block_size=16,
                      kv_format="bf16", ctx=np.array([100, 2, 300]), table="shuffled",
                      max_local_pages=64, seed=5, with_kv=False)
    bt = w.block_table.copy()
    bt[2, 3] = -1                      # hole inside sequence 2's used range
    w2 = w
    w2.block_table = bt
    g = geometry(w2, max_local_pages=5)   # too small for sequence 2 (needs 10 pages)
    meta = ops.RankMetadata(g)
    ops.build_metadata(g, 0, torch.from_numpy(w2.ctx_lens).cuda(), torch.from_numpy(bt).cuda(), meta)
    torch.cuda.synchronize()
    err = int(meta.err.item())
    assert err & _lib().ERR_CTX_LT_QLEN
    assert err & _lib().ERR_LOCAL_PAGES
    lens = meta.row_local_len.cpu().numpy()
    pt = meta.page_table.cpu().numpy()
    # sequence 1 (ctx 2 < qlen 3): row 0 would have boundary 0 -> no tokens
    assert lens[3] == 0
    # sequence 2: clamped to the static bound, then cut at the hole (page 3 -> 3 pages)
    assert np.all(lens[6:9] <= 3 * 16)
    assert np.all(pt[6:9, 3:] == -1)
    g2 = geometry(w2, max_local_pages=64)
    meta2 = ops.RankMetadata(g2)
    ops.build_metadata(g2, 0, torch.from_numpy(w2.ctx_lens).cuda(), torch.from_numpy(bt).cuda(), meta2)
    torch.cuda.synchronize()
    assert int(meta2.err.item()) & _lib().ERR_BLOCK_ID
    assert np.all(meta2.row_local_len.cpu().numpy()[6:9] == 3 * 16)


def _lib():
    from decode_context_parallelism_amd import _lib as L
    return L


@pytest.mark.parametrize("k", [1, 2, 4])
def test_write_kv_slots_and_pool(k):
    from decode_context_parallelism_amd.group import DcpGroup
    w = make_config(k)
    g = geometry(w)
    d = device_inputs(w)
    grp = DcpGroup(g)
    slots = grp.write_kv(d["seq_ids"], d["positions"], d["latents"], d["block_table"]).cpu().numpy()
    torch.cuda.synchronize()
    assert grp.errors() == 0
    seq_ids, positions = w.token_arrays()
    for r in range(w.world):
        want = layout.token_slots(seq_ids, positions, w.block_table, world=w.world,
                                  interleave=w.interleave, block_size=w.block_size, rank=r)
        assert np.array_equal(slots[r], want)
        pool = grp.pools[r].view(-1, 576)
        owned = np.nonzero(want >= 0)[0]
        got = pool[torch.from_numpy(want[owned]).cuda().long()]
        src = d["latents"][torch.from_numpy(owned).cuda().long()]
        assert torch.equal(got.view(torch.uint8) if got.dtype == torch.uint8 else got.view(torch.int16),
                           src.view(torch.uint8) if src.dtype == torch.uint8 else src.view(torch.int16))


@pytest.mark.parametrize("k", [1, 2, 4])
def test_metadata_block_rows(k):
    # bidirectional draft block: every row gets the whole cache ("Context
    # Parallel Guide", DSpark), bit-exact against the brute-force oracle
    w = make_config(k, with_kv=False)
    print(f"config {k}: {w.name} block rows", flush=True)
    for r in range(w.world):
        meta = _gpu_meta(w, r, row_boundary="block")
        lens, table, last = layout.row_metadata(
            w.ctx_lens, w.block_table, world=w.world, interleave=w.interleave,
            block_size=w.block_size, qlen=w.qlen, rank=r, max_local_pages=w.max_local_pages,
            boundary=layout.block_row_boundary)
        assert np.array_equal(meta.row_local_len.cpu().numpy(), lens)
        assert np.array_equal(meta.page_table.cpu().numpy(), table)
        assert np.array_equal(meta.last_page_len.cpu().numpy(), last)
        assert int(meta.err.item()) == 0
