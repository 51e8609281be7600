"""Seeded synthetic workloads shaped like the pages' DCP verification runs.

Recipe (numpy ``Generator(PCG64)``; workload seed ``s``):
  * stream ``SeedSequence(s, spawn_key=(0,))`` draws the context lengths,
    ``(1,)`` the block-table ids, ``(2,)`` the query, and ``(3, b, c)`` the
    latent rows of sequence b, chunk c (65,536 tokens per chunk), so any
    sequence can be regenerated on its own and chunks fill in parallel;
  * query: N(0, 1) float32 rounded to BF16 (round-to-nearest-even);
  * latents: N(0, 1) float32; BF16 caches round to BF16 with scale 1; FP8
    caches use one per-tensor scale ``amax / 448`` over every generated
    latent value, and store the OCP E4M3 code of ``x / scale`` (clipped to
    +-448 first);
  * block tables: every sequence receives ``ceil(ctx / (block_size * world))``
    virtual block ids (one entry covers ``block_size * world`` global tokens),
    either a seeded sample without replacement from ``[0, 2N)`` ("random") or
    a permutation of ``[0, N)`` ("shuffled"), N = total entries; every row
    gets at least one extra column and every unused entry is -1.

Layouts handed out: ``q_bits[B, qlen, H, 576]`` uint16; ``kv[T, 576]`` uint8
(FP8 codes) or uint16 (BF16 bits), the global latent rows of all sequences
back to back, sequence b occupying rows ``seq_start[b] : seq_start[b+1]`` in
global-position order.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np
import torch

D_QK = 576
CHUNK_TOKENS = 65536
FP8_MAX = 448.0

#: The five workloads (sizes as the pages' runs are described).
CONFIGS = {
    1: dict(name="tiny_dcp2_q3_h16_bf16", world=2, interleave=1, batch=1, qlen=3, heads=16,
            block_size=16, kv_format="bf16", ctx=("fixed", 64), table="random",
            max_local_pages=4, seed=1001),
    2: dict(name="dcp2_q3_h96_b8_ctxU1k-8k_fp8", world=2, interleave=1, batch=8, qlen=3,
            heads=96, block_size=64, kv_format="fp8_e4m3", ctx=("uniform", 1024, 8192),
            table="shuffled", max_local_pages=64, seed=1002),
    3: dict(name="dcp8_decode_q1_h128_b32_ctx128k_fp8", world=8, interleave=1, batch=32,
            qlen=1, heads=128, block_size=64, kv_format="fp8_e4m3", ctx=("fixed", 131072),
            table="shuffled", max_local_pages=256, seed=1003),
    4: dict(name="dcp8_S16_q5_h128_b32_ctxlogU8-256k_fp8", world=8, interleave=16, batch=32,
            qlen=5, heads=128, block_size=64, kv_format="fp8_e4m3",
            ctx=("loguniform", 8, 262144), table="shuffled", max_local_pages=512, seed=1004),
    5: dict(name="dcp8_q3_h128_b4_ctx1M_fp8", world=8, interleave=1, batch=4, qlen=3,
            heads=128, block_size=64, kv_format="fp8_e4m3", ctx=("fixed", 1048576),
            table="shuffled", max_local_pages=2048, seed=1005),
}


@dataclass
class Workload:
    name: str
    world: int
    interleave: int
    batch: int
    qlen: int
    heads: int
    block_size: int
    kv_format: str            # "bf16" | "fp8_e4m3"
    ctx_lens: np.ndarray      # int32 [B]
    block_table: np.ndarray   # int32 [B, width], -1 = unused
    num_blocks: int           # physical blocks in each rank's pool
    max_local_pages: int      # static bound on subpages per verify row
    q_bits: np.ndarray        # uint16 [B, qlen, H, 576]
    kv: np.ndarray            # uint8/uint16 [T, 576] global latent rows
    seq_start: np.ndarray     # int64 [B+1]
    kv_scale: float
    softmax_scale: float
    seed: int

    @property
    def elem_bytes(self) -> int:
        return 1 if self.kv_format == "fp8_e4m3" else 2

    def token_arrays(self):
        """Flat ``(seq_ids, positions)`` int32 arrays matching ``kv`` rows."""
        lens = np.diff(self.seq_start)
        seq_ids = np.repeat(np.arange(self.batch, dtype=np.int32), lens)
        positions = (np.arange(self.seq_start[-1], dtype=np.int64)
                     - np.repeat(self.seq_start[:-1], lens)).astype(np.int32)
        return seq_ids, positions


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _to_e4m3_codes(x: np.ndarray, inv_scale: np.float32) -> np.ndarray:
    y = np.clip(x * inv_scale, -FP8_MAX, FP8_MAX)
    return torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _draw_ctx(spec, batch: int, rng: np.random.Generator) -> np.ndarray:
    kind = spec[0]
    if kind == "fixed":
        return np.full(batch, spec[1], dtype=np.int64)
    if kind == "uniform":
        return rng.integers(spec[1], spec[2], size=batch, endpoint=True).astype(np.int64)
    if kind == "loguniform":
        lo, hi = spec[1], spec[2]
        v = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=batch)))
        return np.clip(v, lo, hi).astype(np.int64)
    raise ValueError(f"unknown context spec {spec!r}")


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_workload(*, name: str, world: int, interleave: int, batch: int, qlen: int, heads: int,
                  block_size: int, kv_format: str, ctx, table: str, max_local_pages: int,
                  seed: int, extra_cols: int = 1, softmax_scale: float | None = None,
                  with_kv: bool = True) -> Workload:
    """Build one seeded workload.  ``ctx`` is a spec tuple or explicit lengths.

    ``with_kv=False`` skips the latent rows (``kv`` is an empty array and
    ``kv_scale`` is 1): enough for metadata-only work.
    """
    if isinstance(ctx, tuple) and isinstance(ctx[0], str):
        ctx_lens = _draw_ctx(ctx, batch, _rng(seed, 0))
    else:
        ctx_lens = np.asarray(ctx, dtype=np.int64)
        assert ctx_lens.shape == (batch,)

    # block table: one virtual block id per block_size*world global tokens
    span = block_size * world
    nblk = (ctx_lens + span - 1) // span
    total = int(nblk.sum())
    width = int(nblk.max()) + extra_cols
    rng_bt = _rng(seed, 1)
    if table == "random":
        num_blocks = max(2 * total, 1)
        ids = rng_bt.choice(num_blocks, size=total, replace=False)
    elif table == "shuffled":
        num_blocks = max(total, 1)
        ids = rng_bt.permutation(total)
    else:
        raise ValueError(table)
    block_table = np.full((batch, width), -1, dtype=np.int32)
    off = 0
    for b in range(batch):
        block_table[b, : nblk[b]] = ids[off: off + nblk[b]]
        off += nblk[b]

    q = _rng(seed, 2).standard_normal((batch, qlen, heads, D_QK), dtype=np.float32)
    q_bits = _to_bf16_bits(q)

    seq_start = np.zeros(batch + 1, dtype=np.int64)
    seq_start[1:] = np.cumsum(ctx_lens)
    T = int(seq_start[-1])
    if not with_kv:
        return Workload(name=name, world=world, interleave=interleave, batch=batch, qlen=qlen,
                        heads=heads, block_size=block_size, kv_format=kv_format,
                        ctx_lens=ctx_lens.astype(np.int32), block_table=block_table,
                        num_blocks=int(num_blocks), max_local_pages=int(max_local_pages),
                        q_bits=q_bits, kv=np.zeros((0, D_QK), dtype=np.uint8),
                        seq_start=seq_start, kv_scale=1.0,
                        softmax_scale=float(softmax_scale if softmax_scale is not None
                                            else 1.0 / math.sqrt(192.0)),
                        seed=seed)
    jobs = []
    for b in range(batch):
        for c in range((int(ctx_lens[b]) + CHUNK_TOKENS - 1) // CHUNK_TOKENS):
            lo = int(seq_start[b]) + c * CHUNK_TOKENS
            hi = min(int(seq_start[b + 1]), lo + CHUNK_TOKENS)
            jobs.append((b, c, lo, hi))

    raw = np.empty((T, D_QK), dtype=np.float32)

    def fill(job):
        b, c, lo, hi = job
        _rng(seed, 3, b, c).standard_normal((hi - lo, D_QK), dtype=np.float32, out=raw[lo:hi])
        return float(np.abs(raw[lo:hi]).max()) if hi > lo else 0.0

    with ThreadPoolExecutor(_workers()) as ex:
        amaxes = list(ex.map(fill, jobs))

    if kv_format == "bf16":
        kv = np.empty((T, D_QK), dtype=np.uint16)
        kv_scale = 1.0

        def conv(job):
            _, _, lo, hi = job
            kv[lo:hi] = _to_bf16_bits(raw[lo:hi])
    elif kv_format == "fp8_e4m3":
        amax = max(amaxes) if amaxes else 1.0
        kv_scale = float(np.float32(amax / FP8_MAX))
        inv = np.float32(1.0) / np.float32(kv_scale)
        kv = np.empty((T, D_QK), dtype=np.uint8)

        def conv(job):
            _, _, lo, hi = job
            kv[lo:hi] = _to_e4m3_codes(raw[lo:hi], inv)
    else:
        raise ValueError(kv_format)
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(conv, jobs))
    del raw

    return Workload(name=name, world=world, interleave=interleave, batch=batch, qlen=qlen,
                    heads=heads, block_size=block_size, kv_format=kv_format,
                    ctx_lens=ctx_lens.astype(np.int32), block_table=block_table,
                    num_blocks=int(num_blocks), max_local_pages=int(max_local_pages),
                    q_bits=q_bits, kv=kv, seq_start=seq_start, kv_scale=kv_scale,
                    softmax_scale=float(softmax_scale if softmax_scale is not None
                                        else 1.0 / math.sqrt(192.0)),
                    seed=seed)


def make_config(k: int, **overrides) -> Workload:
    """Workload for configuration ``k`` (1..5) with optional overrides."""
    cfg = dict(CONFIGS[k])
    cfg.update(overrides)
    return make_workload(**cfg)


def random_rank_partials(world: int, n: int, seed: int, frac_empty: float = 0.2):
    """Synthetic per-rank partials for the cross-rank merge.

    Returns ``(out_bits uint16 [W, n, 512] BF16, lse float32 [W, n])``; a
    fraction of (rank, row) pairs is empty (LSE -inf, output 0) and some rows
    are empty on every rank.
    """
    rng = _rng(seed, 7)
    out = rng.standard_normal((world, n, 512), dtype=np.float32)
    lse = rng.uniform(-20.0, 40.0, size=(world, n)).astype(np.float32)
    empty = rng.uniform(size=(world, n)) < frac_empty
    if n >= 4:
        empty[:, n // 3] = True        # a row that no rank can see
    lse[empty] = -np.inf
    out[empty] = 0.0
    return _to_bf16_bits(out), lse


def random_segment_partials(nseg: int, n: int, seed: int, frac_empty: float = 0.2):
    """Synthetic split-KV segment partials: ``(o float32 [nseg, n, 512], lse2 float32 [nseg, n])``."""
    rng = _rng(seed, 8)
    o = rng.standard_normal((nseg, n, 512), dtype=np.float32)
    lse2 = rng.uniform(-30.0, 60.0, size=(nseg, n)).astype(np.float32)
    empty = rng.uniform(size=(nseg, n)) < frac_empty
    if n >= 4:
        empty[:, n // 2] = True
    lse2[empty] = -np.inf
    o[empty] = 0.0
    return o, lse2
