"""DCP cache layout and per-row metadata by brute-force enumeration (exact ints).

Test infrastructure only (see ``oracle/__init__``).

Everything here is derived from two definitions on the pages and nothing else:

* Ownership.  "Context Parallel Guide (PCP & DCP)", ``--dcp-config`` table,
  row ``interleave_size``: with interleave S and DCP world W, global token i
  lives on rank (i // S) % W.  S = 1 is the token round-robin of the
  "Decode Context Parallel (DCP) Guide" diagram.
* Virtual blocks.  Same page, "How it works" item 1: one block-table entry
  (shared by all ranks) names, on every rank, that rank's own physical block
  of ``block_size`` consecutive *rank-local* tokens.  So rank-local token
  number ``li`` sits in physical row ``block_table[li // bs] * bs + li % bs``
  of that rank's pool.

The rank-local index of a token is found by *counting* the owned positions
before it, never by the closed forms the pages also print; those closed forms
are what the tests compare this module against.

The verify-row boundary follows "[ROCm][MLA][DCP] Support causal multi-token
verification" (vLLM PR #51705), "Implementation" item 1: each verification
row has its own global causal boundary.  Reading used here (the verify tokens'
own KV is already in the cache, so the last row sees the whole context):
row i of a sequence with ``ctx`` cached tokens and ``qlen`` verify rows sees
global positions [0, ctx - qlen + 1 + i).

Subpages follow the review thread on ``_segmented_mla_page_size`` in the same
PR: the segmented kernel reads subpages of the largest power of two that
divides the block size, capped at 128.
"""
import numpy as np


def owner_rank(p, world: int, interleave: int):
    """Rank that stores global position(s) ``p``."""
    return (np.asarray(p) // interleave) % world


def verify_row_boundary(ctx: int, qlen: int, i: int) -> int:
    """Number of global positions visible to verify row ``i`` (exclusive end)."""
    return ctx - qlen + 1 + i


def block_row_boundary(ctx: int, qlen: int, i: int) -> int:
    """Row boundary of a bidirectional draft block: every row sees the whole cache.

    "Context Parallel Guide (PCP & DCP)", "DSpark (Kimi-K3)": the draft block
    is not causal -- each draft position attends the whole block -- so no row
    gets a boundary of its own.
    """
    return ctx


def rank_local_positions(g: int, world: int, interleave: int, rank: int) -> np.ndarray:
    """Global positions < g owned by ``rank``, ascending (the rank-local order)."""
    p = np.arange(max(g, 0), dtype=np.int64)
    return p[owner_rank(p, world, interleave) == rank]


def subpage_size(block_size: int) -> int:
    """Largest power of two dividing ``block_size``, capped at 128 (by search)."""
    if block_size <= 0:
        raise ValueError("block_size must be positive")
    best = 1
    cand = 1
    while cand <= block_size:
        if block_size % cand == 0:
            best = cand
        cand *= 2
    return min(best, 128)


def physical_rows(local_index: np.ndarray, block_table_row: np.ndarray, block_size: int) -> np.ndarray:
    """Physical pool row of each rank-local token index (virtual-block rule)."""
    li = np.asarray(local_index, dtype=np.int64)
    blocks = np.asarray(block_table_row, dtype=np.int64)[li // block_size]
    return blocks * block_size + li % block_size


def row_metadata(ctx_lens, block_table, *, world, interleave, block_size, qlen, rank,
                 max_local_pages, boundary=verify_row_boundary):
    """Expected verify view for one rank.

    Returns ``(row_local_len[B*q], page_table[B*q, max_local_pages],
    last_page_len[B*q])`` as int32 arrays; row index is ``b*qlen + i``.
    The page list of a row is the sequence of distinct subpages its local
    tokens occupy, in local-token order; unused entries are -1.
    """
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    block_table = np.asarray(block_table, dtype=np.int64)
    P = subpage_size(block_size)
    B = ctx_lens.shape[0]
    n_rows = B * qlen
    lens = np.zeros(n_rows, dtype=np.int32)
    table = np.full((n_rows, max_local_pages), -1, dtype=np.int32)
    last = np.zeros(n_rows, dtype=np.int32)
    for b in range(B):
        for i in range(qlen):
            row = b * qlen + i
            g = boundary(int(ctx_lens[b]), qlen, i)
            pos = rank_local_positions(g, world, interleave, rank)
            n = pos.shape[0]
            lens[row] = n
            if n == 0:
                continue
            li = np.arange(n, dtype=np.int64)
            pages = physical_rows(li, block_table[b], block_size) // P
            # distinct pages in order of first appearance along the token list
            starts = np.ones(n, dtype=bool)
            starts[1:] = pages[1:] != pages[:-1]
            distinct = pages[starts]
            if distinct.shape[0] > max_local_pages:
                raise ValueError("row needs more subpages than max_local_pages")
            table[row, : distinct.shape[0]] = distinct
            # tokens in the final run of equal pages
            run_start = np.nonzero(starts)[0][-1]
            last[row] = n - run_start
    return lens, table, last


def token_slots(seq_ids, positions, block_table, *, world, interleave, block_size, rank):
    """Pool row on ``rank`` of every (sequence, global position) token, or -1.

    The rank-local index is the count of owned positions before the token.
    """
    seq_ids = np.asarray(seq_ids, dtype=np.int64)
    positions = np.asarray(positions, dtype=np.int64)
    block_table = np.asarray(block_table, dtype=np.int64)
    out = np.full(positions.shape[0], -1, dtype=np.int64)
    for b in np.unique(seq_ids):
        sel = np.nonzero(seq_ids == b)[0]
        p = positions[sel]
        owned_all = rank_local_positions(int(p.max()) + 1, world, interleave, rank)
        mine = owner_rank(p, world, interleave) == rank
        li = np.searchsorted(owned_all, p[mine])  # owned positions strictly before p
        out[sel[mine]] = physical_rows(li, block_table[b], block_size)
    return out
