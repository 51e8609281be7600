"""Pins for ``oracle.layout`` (CPU only).

The oracle enumerates global positions and counts; these tests hold it to the
closed forms and the worked example the pages print, which it never uses.
"""
import math
import os

import numpy as np
import pytest

from oracle import layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_layout_golden():
    ranks = {}
    with open(os.path.join(GOLDEN, "dcp2_token_layout.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("world"):
                parts = line.split()
                world, interleave, n = int(parts[1]), int(parts[3]), int(parts[5])
            else:
                head, toks = line.split(":")
                ranks[int(head.split()[1])] = [int(t) for t in toks.split()]
    return world, interleave, n, ranks


def test_printed_dcp2_example():
    # "Context Parallel Guide (PCP & DCP)", DCP Guide diagram: tokens 0..5 over 2 ranks
    world, interleave, n, ranks = _read_layout_golden()
    for r, toks in ranks.items():
        got = layout.rank_local_positions(n, world, interleave, r).tolist()
        assert got == toks


# --- closed forms the pages print (the oracle never evaluates them) -------------

def _page_local_index(i, S, W):
    # "Context Parallel Guide", interleave_size constraints: local index math
    return (i // (S * W)) * S + i % S


def _page_local_rows_s1(L, rank, dcp):
    # "Context Parallel Guide", DSpark bullet: L global tokens give ceil((L - rank)/dcp) local rows
    return max(0, math.ceil((L - rank) / dcp))


def _page_slot_s1(p, block_table_row, bs, dcp):
    # "Context Parallel Guide", DSpark bullet: slot of global position p on its owner rank
    return block_table_row[p // (bs * dcp)] * bs + (p % (bs * dcp)) // dcp


def _page_row_len(g, rank, W, S):
    # "[Spec decode] Support Kimi-K3 DCP with DSpark", review: per-query global lengths
    span = W * S
    rem = min(max(g % span - rank * S, 0), S)
    return g // span * S + rem


WS = [(w, s) for w in range(1, 9) for s in (1, 2, 4, 8, 16) if not (s > 1 and w == 1)]


@pytest.mark.parametrize("W,S", WS)
def test_local_length_matches_page_formula(W, S):
    for g in range(0, 4 * W * S + 3):
        for r in range(W):
            brute = layout.rank_local_positions(g, W, S, r).shape[0]
            assert brute == _page_row_len(g, r, W, S), (g, r)


@pytest.mark.parametrize("W,S", WS)
def test_windows_partition_prefix(W, S):
    # union of rank windows is exactly [0, g) and they are disjoint
    for g in (0, 1, 2, W * S - 1, W * S, W * S + 1, 3 * W * S + 5):
        allpos = np.concatenate([layout.rank_local_positions(g, W, S, r) for r in range(W)])
        assert allpos.shape[0] == g
        assert np.array_equal(np.sort(allpos), np.arange(g))


@pytest.mark.parametrize("W,S", WS)
def test_local_index_matches_page_formula(W, S):
    n = 5 * W * S + 7
    for r in range(W):
        owned = layout.rank_local_positions(n, W, S, r)
        for li, p in enumerate(owned):
            assert _page_local_index(int(p), S, W) == li


def test_local_rows_s1_closed_form():
    for dcp in range(1, 9):
        for L in range(0, 200):
            for r in range(dcp):
                assert layout.rank_local_positions(L, dcp, 1, r).shape[0] == _page_local_rows_s1(L, r, dcp)


def test_length_step_property():
    # len_r(g+1) - len_r(g) == [r owns position g]
    for W, S in [(2, 1), (8, 16), (3, 4), (8, 1)]:
        for g in range(0, 3 * W * S):
            for r in range(W):
                d = layout.rank_local_positions(g + 1, W, S, r).shape[0] - \
                    layout.rank_local_positions(g, W, S, r).shape[0]
                assert d == int(layout.owner_rank(g, W, S) == r)


def test_slots_match_page_formula_s1():
    rng = np.random.default_rng(5)
    for dcp in (1, 2, 4, 8):
        for bs in (1, 4, 16, 64):
            nblk = 6
            bt = rng.permutation(50)[:nblk].astype(np.int64)
            n = nblk * bs * dcp
            pos = np.arange(n)
            seq = np.zeros(n, dtype=np.int64)
            for r in range(dcp):
                slots = layout.token_slots(seq, pos, bt[None, :], world=dcp, interleave=1,
                                           block_size=bs, rank=r)
                for p in range(n):
                    want = _page_slot_s1(p, bt, bs, dcp) if p % dcp == r else -1
                    assert slots[p] == want


def test_slots_interleaved_consistent_with_local_index():
    # S > 1: slot = block_table[li // bs]*bs + li % bs with li from the page's local-index formula
    rng = np.random.default_rng(6)
    for W, S, bs in [(2, 2, 4), (8, 16, 64), (4, 8, 16), (3, 4, 8)]:
        bt = rng.permutation(100)[:8].astype(np.int64)
        n = 7 * bs * W + 3
        pos = np.arange(n)
        seq = np.zeros(n, dtype=np.int64)
        for r in range(W):
            slots = layout.token_slots(seq, pos, bt[None, :], world=W, interleave=S, block_size=bs, rank=r)
            for p in range(n):
                if (p // S) % W != r:
                    assert slots[p] == -1
                else:
                    li = _page_local_index(p, S, W)
                    assert slots[p] == bt[li // bs] * bs + li % bs


def test_subpage_size_rule():
    # "[ROCm][MLA][DCP] Support causal multi-token verification", review thread on
    # _segmented_mla_page_size: min(128, largest power-of-two divisor of block size).
    hand = {1: 1, 2: 2, 3: 1, 6: 2, 12: 4, 16: 16, 48: 16, 64: 64, 96: 32, 128: 128,
            192: 64, 256: 128, 512: 128, 640: 128, 1000: 8}
    for bs, P in hand.items():
        assert layout.subpage_size(bs) == P
    for bs in range(1, 2049):
        assert layout.subpage_size(bs) == min(128, bs & -bs)


def test_verify_boundary_is_causal_on_positions():
    # The verify tokens occupy the last qlen positions [ctx-qlen, ctx); causal attention
    # lets the token at position t see positions <= t, i.e. t + 1 of them.
    for ctx in (3, 4, 64, 1000):
        for qlen in (1, 2, 3, 5):
            if qlen > ctx:
                continue
            for i in range(qlen):
                t = ctx - qlen + i
                assert layout.verify_row_boundary(ctx, qlen, i) == t + 1
            assert layout.verify_row_boundary(ctx, qlen, qlen - 1) == ctx


def _brute_pages_by_token(ctx, bt_row, W, S, bs, qlen, rank):
    """Independent page list: walk tokens, map every owned one to its (block, subpage)."""
    P = min(128, bs & -bs)
    rows = []
    for i in range(qlen):
        g = ctx - qlen + 1 + i
        li = 0
        pages = []
        counts = []
        for p in range(g):
            if (p // S) % W != rank:
                continue
            pg = (int(bt_row[li // bs]) * bs + li % bs) // P
            if not pages or pages[-1] != pg:
                pages.append(pg)
                counts.append(0)
            counts[-1] += 1
            li += 1
        rows.append((li, pages, counts[-1] if counts else 0))
    return rows


@pytest.mark.parametrize("bs", [1, 16, 48, 64, 128, 192, 256, 512])
def test_row_metadata_small_sweep(bs):
    rng = np.random.default_rng(bs)
    for W, S in [(2, 1), (4, 1), (8, 1), (2, 2), (4, 4), (8, 16)]:
        if bs % S:
            continue
        for qlen in (1, 3, 5):
            B = 3
            ctx = rng.integers(qlen, 6 * bs * W + 40, size=B)
            span = bs * W
            width = int(((ctx + span - 1) // span).max()) + 1
            bt = np.full((B, width), -1, dtype=np.int64)
            ids = rng.permutation(B * width * 2)
            for b in range(B):
                n = (ctx[b] + span - 1) // span
                bt[b, :n] = ids[b * width: b * width + n]
            P = min(128, bs & -bs)
            mlp = width * (bs // P) + 1
            for r in range(W):
                lens, table, last = layout.row_metadata(ctx, bt, world=W, interleave=S,
                                                        block_size=bs, qlen=qlen, rank=r,
                                                        max_local_pages=mlp)
                for b in range(B):
                    brute = _brute_pages_by_token(int(ctx[b]), bt[b], W, S, bs, qlen, r)
                    for i, (n, pages, lastc) in enumerate(brute):
                        row = b * qlen + i
                        assert lens[row] == n
                        assert table[row, : len(pages)].tolist() == pages
                        assert np.all(table[row, len(pages):] == -1)
                        assert last[row] == lastc


# -------------------------------------------------- bidirectional draft block ----

@pytest.mark.parametrize("W,S", [(1, 1), (2, 1), (8, 1), (4, 4), (8, 16)])
def test_block_rows_see_whole_cache(W, S):
    # "Context Parallel Guide", DSpark: the draft block attends the whole block,
    # so every row of a sequence gets the same window [0, ctx); with S = 1 the
    # rank-local length is the printed ceil((L - rank) / dcp)
    rng = np.random.default_rng(W * 100 + S)
    B, q, bs = 3, 4, 16 * S
    ctx = rng.integers(q, 6 * bs * W, size=B)
    ncol = int(max(-(-c // (bs * W)) for c in ctx)) + 1
    bt = rng.permutation(B * ncol).reshape(B, ncol).astype(np.int64)
    for r in range(W):
        lens, table, last = layout.row_metadata(ctx, bt, world=W, interleave=S, block_size=bs, qlen=q,
                                                rank=r, max_local_pages=4 * ncol,
                                                boundary=layout.block_row_boundary)
        causal = layout.row_metadata(ctx, bt, world=W, interleave=S, block_size=bs, qlen=q, rank=r,
                                     max_local_pages=4 * ncol)
        for b in range(B):
            rows = slice(b * q, (b + 1) * q)
            # every row equals the last causal row, whose window is [0, ctx)
            assert np.all(lens[rows] == causal[0][b * q + q - 1])
            assert np.all(table[rows] == causal[1][b * q + q - 1])
            assert np.all(last[rows] == causal[2][b * q + q - 1])
            if S == 1:
                assert np.all(lens[rows] == _page_local_rows_s1(int(ctx[b]), r, W))
