"""One GPU playing every rank of a DCP group.

Each rank keeps its own KV pool and verify-view buffers in HBM; ``forward``
runs the ranks one after another on one stream (KV write, metadata, segmented
attention and segment merge per rank), and the cross-rank LSE merge then reads
all W partials from HBM.  ``ranks_two_streams`` issues the same launches over
two streams, so independent work overlaps.  In a real deployment each rank is a different GPU and the
merge input arrives through an all-to-all; the per-rank work is identical.

Buffer layout (all contiguous, allocated once):
  pools[r]     [num_blocks, block_size, 576]  cache elements (uint8 FP8 codes
               or bfloat16), filled with a NaN pattern until written, so a
               read of an unwritten slot cannot go unnoticed
  meta[r]      verify view of rank r (see ``ops.RankMetadata``)
  workspace    split-KV partials, shared by the ranks in turn (workspace2: the
               second stream's, for ``ranks_two_streams``)
  q_split      FP8 cache: the query split once per forward into two E4M3
  q_scale      terms and its per-row scale, read by every rank
  out_ranks    [W, B, qlen, H, 512] bfloat16, lse_ranks [W, B, qlen, H] float
  out, lse     merged result
"""
from __future__ import annotations

import torch

from . import ops

_NAN_FILL = {"fp8_e4m3": 0x7F, "bf16": float("nan")}


class DcpGroup:
    def __init__(self, geom: ops.Geometry, device="cuda"):
        self.geom = geom
        self.device = device
        W, B, q, H = geom.dcp_world, geom.batch, geom.qlen, geom.num_heads
        self.pools = []
        for _ in range(W):
            pool = torch.empty(geom.num_blocks, geom.block_size, ops.D_QK,
                               dtype=geom.kv_torch_dtype, device=device)
            pool.fill_(_NAN_FILL[geom.kv_dtype])
            self.pools.append(pool)
        self.meta = [ops.RankMetadata(geom, device) for _ in range(W)]
        self.workspace = ops.alloc_workspace(geom, device)
        self.workspace2 = ops.alloc_workspace(geom, device)
        self.out_ranks = torch.empty(W, B, q, H, ops.D_V, dtype=torch.bfloat16, device=device)
        self.lse_ranks = torch.empty(W, B, q, H, dtype=torch.float32, device=device)
        self.out = torch.empty(B, q, H, ops.D_V, dtype=torch.bfloat16, device=device)
        self.lse = torch.empty(B, q, H, dtype=torch.float32, device=device)
        self.kv_err = torch.zeros(1, dtype=torch.int32, device=device)
        self.q_split = self.q_scale = None
        if geom.kv_dtype == "fp8_e4m3":
            rows = B * q * H
            self.q_split = torch.empty(ops.split_q_bytes(rows), dtype=torch.uint8, device=device)
            self.q_scale = torch.empty(rows, dtype=torch.float32, device=device)

    def write_kv(self, seq_ids, positions, latents, block_table, stream=None):
        """Scatter global latent rows into every rank's pool; returns slot mappings [W, T]."""
        T = seq_ids.shape[0]
        slots = torch.empty(self.geom.dcp_world, T, dtype=torch.int32, device=self.device)
        for r in range(self.geom.dcp_world):
            ops.write_kv(self.geom, r, seq_ids, positions, latents, block_table, self.pools[r],
                         slots[r], self.kv_err, stream)
        return slots

    def build_metadata(self, ctx_lens, block_table, stream=None):
        for r in range(self.geom.dcp_world):
            ops.build_metadata(self.geom, r, ctx_lens, block_table, self.meta[r], stream)

    def rank_attention(self, r, q, kv_scale, softmax_scale, stream=None):
        ops.rank_attention(self.geom, q, self.pools[r], kv_scale, softmax_scale, self.meta[r],
                           self.workspace, self.out_ranks[r], self.lse_ranks[r], stream)

    def merge(self, stream=None):
        ops.merge_ranks(self.out_ranks, self.lse_ranks, self.out, self.lse, stream)

    def rank_attention_split(self, r, kv_scale, softmax_scale, stream=None):
        """Rank r's attention and segment merge on the query split by ``split_query``."""
        ops.partial_attention_split(self.geom, self.q_split, self.q_scale, self.pools[r], kv_scale,
                                    softmax_scale, self.meta[r], self.workspace, self.out_ranks[r],
                                    self.lse_ranks[r], stream)
        ops.merge_segments(self.geom, self.meta[r], self.workspace, self.out_ranks[r],
                           self.lse_ranks[r], stream)

    def split_query(self, q, stream=None):
        ops.split_q(q, self.q_split, self.q_scale, stream)

    def forward(self, q, ctx_lens, block_table, kv_scale, softmax_scale, stream=None):
        """One verification step: metadata, every rank's attention, cross-rank merge.  With an
        FP8 cache the query is split once and every rank reads the split."""
        self.build_metadata(ctx_lens, block_table, stream)
        if self.q_split is not None:
            self.split_query(q, stream)
        for r in range(self.geom.dcp_world):
            if self.q_split is not None:
                self.rank_attention_split(r, kv_scale, softmax_scale, stream)
            else:
                self.rank_attention(r, q, kv_scale, softmax_scale, stream)
        self.merge(stream)
        return self.out, self.lse

    def ranks_two_streams(self, q, ctx_lens, block_table, kv_scale, softmax_scale, side,
                          pools=None):
        """Metadata, query split, attention and segment merge of every rank, issued over two
        streams: the current stream takes the even ranks, ``side`` the query split and the odd
        ranks, each stream with its own split-KV workspace.  The launches and their inputs are
        those of ``forward``; only independent work overlaps (the query split beside rank 0's
        metadata, one stream's attention beside the other's, a segment merge beside the other
        stream's attention).  On return the current stream waits for ``side``, so what is
        issued next on it (the cross-rank merge) sees every rank's result.  Capturable into a
        HIP graph (the fork and the join become graph edges).  ``pools`` replaces the KV pools
        (the bench rotates input copies)."""
        main = torch.cuda.current_stream()
        pools = self.pools if pools is None else pools
        streams = (main, side)
        work = (self.workspace, self.workspace2)
        W = self.geom.dcp_world
        side.wait_stream(main)
        split_done = None
        if self.q_split is not None:
            ops.split_q(q, self.q_split, self.q_scale, side)
            split_done = torch.cuda.Event()
            split_done.record(side)
        for r in range(W):
            ops.build_metadata(self.geom, r, ctx_lens, block_table, self.meta[r], streams[r % 2])
        if split_done is not None:
            main.wait_event(split_done)
        for r in range(W):
            s, ws = streams[r % 2], work[r % 2]
            if self.q_split is not None:
                ops.partial_attention_split(self.geom, self.q_split, self.q_scale, pools[r],
                                            kv_scale, softmax_scale, self.meta[r], ws,
                                            self.out_ranks[r], self.lse_ranks[r], s)
            else:
                ops.partial_attention(self.geom, q, pools[r], kv_scale, softmax_scale,
                                      self.meta[r], ws, self.out_ranks[r], self.lse_ranks[r], s)
            ops.merge_segments(self.geom, self.meta[r], ws, self.out_ranks[r], self.lse_ranks[r], s)
        main.wait_stream(side)

    def forward_two_streams(self, q, ctx_lens, block_table, kv_scale, softmax_scale, side):
        """``forward`` with the ranks issued by ``ranks_two_streams``."""
        self.ranks_two_streams(q, ctx_lens, block_table, kv_scale, softmax_scale, side)
        self.merge()
        return self.out, self.lse

    def errors(self):
        """OR of every device error word (synchronises)."""
        e = int(self.kv_err.item())
        for m in self.meta:
            e |= int(m.err.item())
        return e
