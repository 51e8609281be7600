"""Tensor-level wrappers over the dcpmla C ABI (PyTorch for memory and streams).

Each function checks dtypes, shapes and contiguity of the tensors it hands
over, passes raw device pointers and the current HIP stream to the library,
and raises ``DcpMlaError`` on a non-zero status.  All arithmetic happens in
the HIP kernels.  Names follow ``include/dcpmla.h``.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import lib

D_QK = 576
D_V = 512


class DcpMlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {_lib.strerror(status)} (status {status})")
        self.status = status


def _check(status: int, what: str) -> None:
    if status != _lib.OK:
        raise DcpMlaError(status, what)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, dtype, shape, name: str):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")


@dataclass(frozen=True)
class Geometry:
    """One DCP group and one verification batch (``dcpmla_geom``)."""
    dcp_world: int
    interleave: int
    block_size: int
    qlen: int
    num_heads: int
    batch: int
    max_blocks_per_seq: int
    max_local_pages: int
    kv_dtype: str              # "bf16" | "fp8_e4m3"
    num_blocks: int
    groups: int = 0
    row_boundary: str = "causal"   # "causal" verify rows | "block" (bidirectional draft block)
    q_format: str = "split"        # FP8 cache: "split" (exact BF16 query) | "fp8" (quantised query)
    p_format: str = "split"        # FP8 cache: "split" (two-term probabilities) | "fp8" (one E4M3 term)

    def c(self) -> _lib.Geom:
        return _lib.Geom(self.dcp_world, self.interleave, self.block_size, self.qlen,
                         self.num_heads, self.batch, self.max_blocks_per_seq,
                         self.max_local_pages, self.kv_code, self.groups, self.num_blocks,
                         {"causal": _lib.BOUNDARY_CAUSAL, "block": _lib.BOUNDARY_BLOCK}[self.row_boundary],
                         {"split": _lib.Q_SPLIT, "fp8": _lib.Q_FP8}[self.q_format],
                         {"split": _lib.P_SPLIT, "fp8": _lib.P_FP8}[self.p_format])

    @property
    def kv_code(self) -> int:
        return {"bf16": _lib.KV_BF16, "fp8_e4m3": _lib.KV_FP8_E4M3}[self.kv_dtype]

    @property
    def kv_torch_dtype(self):
        return torch.uint8 if self.kv_dtype == "fp8_e4m3" else torch.bfloat16

    @property
    def rows(self) -> int:
        return self.batch * self.qlen

    @property
    def head_rows(self) -> int:
        return self.batch * self.qlen * self.num_heads


def validate(geom: Geometry) -> int:
    g = geom.c()
    return lib.dcpmla_validate(ctypes.byref(g))


def subpage_size(block_size: int) -> int:
    return lib.dcpmla_subpage_size(block_size)


def work_ints(geom: Geometry) -> int:
    g = geom.c()
    n = lib.dcpmla_work_ints(ctypes.byref(g))
    _check(int(min(n, 0)), "dcpmla_work_ints")
    return int(n)


def workspace_bytes(geom: Geometry) -> int:
    g = geom.c()
    n = lib.dcpmla_workspace_bytes(ctypes.byref(g))
    _check(int(min(n, 0)), "dcpmla_workspace_bytes")
    return int(n)


class RankMetadata:
    """Device buffers of one rank's verify view (``dcpmla_meta``), allocated once."""

    def __init__(self, geom: Geometry, device="cuda"):
        rows = geom.rows
        self.row_local_len = torch.zeros(rows, dtype=torch.int32, device=device)
        self.page_table = torch.zeros(rows, geom.max_local_pages, dtype=torch.int32, device=device)
        self.last_page_len = torch.zeros(rows, dtype=torch.int32, device=device)
        self.err = torch.zeros(1, dtype=torch.int32, device=device)
        self.work = torch.zeros(work_ints(geom), dtype=torch.int32, device=device)

    def c(self) -> _lib.Meta:
        return _lib.Meta(self.row_local_len.data_ptr(), self.page_table.data_ptr(),
                         self.last_page_len.data_ptr(), self.err.data_ptr(), self.work.data_ptr())


def alloc_workspace(geom: Geometry, device="cuda") -> torch.Tensor:
    return torch.empty(workspace_bytes(geom), dtype=torch.uint8, device=device)


def write_kv(geom: Geometry, rank: int, seq_ids, positions, latents, block_table, kv_pool,
             slot_mapping, err, stream=None) -> None:
    T = seq_ids.shape[0]
    _need(seq_ids, torch.int32, (T,), "seq_ids")
    _need(positions, torch.int32, (T,), "positions")
    _need(latents, geom.kv_torch_dtype, (T, D_QK), "latents")
    _need(block_table, torch.int32, (geom.batch, geom.max_blocks_per_seq), "block_table")
    _need(kv_pool, geom.kv_torch_dtype, (geom.num_blocks, geom.block_size, D_QK), "kv_pool")
    _need(slot_mapping, torch.int32, (T,), "slot_mapping")
    _need(err, torch.int32, (1,), "err")
    g = geom.c()
    _check(lib.dcpmla_write_kv(ctypes.byref(g), rank, T, _ptr(seq_ids), _ptr(positions),
                               _ptr(latents), _ptr(block_table), _ptr(kv_pool),
                               _ptr(slot_mapping), _ptr(err), _stream(stream)),
           "dcpmla_write_kv")


def build_metadata(geom: Geometry, rank: int, ctx_lens, block_table, meta: RankMetadata,
                   stream=None) -> None:
    _need(ctx_lens, torch.int32, (geom.batch,), "ctx_lens")
    _need(block_table, torch.int32, (geom.batch, geom.max_blocks_per_seq), "block_table")
    g = geom.c()
    m = meta.c()
    _check(lib.dcpmla_build_metadata(ctypes.byref(g), rank, _ptr(ctx_lens), _ptr(block_table),
                                     ctypes.byref(m), _stream(stream)),
           "dcpmla_build_metadata")


def _attn_shapes(geom, q, kv_pool, out, lse):
    _need(q, torch.bfloat16, (geom.batch, geom.qlen, geom.num_heads, D_QK), "q")
    _need(kv_pool, geom.kv_torch_dtype, (geom.num_blocks, geom.block_size, D_QK), "kv_pool")
    _need(out, torch.bfloat16, (geom.batch, geom.qlen, geom.num_heads, D_V), "out")
    _need(lse, torch.float32, (geom.batch, geom.qlen, geom.num_heads), "lse")


def partial_attention(geom: Geometry, q, kv_pool, kv_scale: float, softmax_scale: float,
                      meta: RankMetadata, workspace, out, lse, stream=None) -> None:
    _attn_shapes(geom, q, kv_pool, out, lse)
    g = geom.c()
    m = meta.c()
    _check(lib.dcpmla_partial_attention(ctypes.byref(g), _ptr(q), _ptr(kv_pool), kv_scale,
                                        softmax_scale, ctypes.byref(m), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _ptr(out),
                                        _ptr(lse), _stream(stream)),
           "dcpmla_partial_attention")


def partial_attention_split(geom: Geometry, q_split, q_inv_scale, kv_pool, kv_scale: float,
                            softmax_scale: float, meta: RankMetadata, workspace, out, lse,
                            stream=None) -> None:
    """``partial_attention`` with the query already split (``split_q`` output); FP8 cache only."""
    rows = geom.batch * geom.qlen * geom.num_heads
    _need(kv_pool, geom.kv_torch_dtype, (geom.num_blocks, geom.block_size, D_QK), "kv_pool")
    _need(q_split, torch.uint8, (split_q_bytes(rows),), "q_split")
    _need(q_inv_scale, torch.float32, (rows,), "q_inv_scale")
    _need(out, torch.bfloat16, (geom.batch, geom.qlen, geom.num_heads, D_V), "out")
    _need(lse, torch.float32, (geom.batch, geom.qlen, geom.num_heads), "lse")
    g = geom.c()
    m = meta.c()
    _check(lib.dcpmla_partial_attention_split(ctypes.byref(g), _ptr(q_split), _ptr(q_inv_scale),
                                              _ptr(kv_pool), kv_scale, softmax_scale, ctypes.byref(m),
                                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                                              _ptr(out), _ptr(lse), _stream(stream)),
           "dcpmla_partial_attention_split")


def merge_segments(geom: Geometry, meta: RankMetadata, workspace, out, lse, stream=None) -> None:
    _need(out, torch.bfloat16, (geom.batch, geom.qlen, geom.num_heads, D_V), "out")
    _need(lse, torch.float32, (geom.batch, geom.qlen, geom.num_heads), "lse")
    g = geom.c()
    m = meta.c()
    _check(lib.dcpmla_merge_segments(ctypes.byref(g), ctypes.byref(m), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _ptr(out),
                                     _ptr(lse), _stream(stream)),
           "dcpmla_merge_segments")


def rank_attention(geom: Geometry, q, kv_pool, kv_scale: float, softmax_scale: float,
                   meta: RankMetadata, workspace, out, lse, stream=None) -> None:
    _attn_shapes(geom, q, kv_pool, out, lse)
    g = geom.c()
    m = meta.c()
    _check(lib.dcpmla_rank_attention(ctypes.byref(g), _ptr(q), _ptr(kv_pool), kv_scale,
                                     softmax_scale, ctypes.byref(m), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _ptr(out),
                                     _ptr(lse), _stream(stream)),
           "dcpmla_rank_attention")


def rank_attention_static(geom: Geometry, q, kv_pool, kv_scale: float, softmax_scale: float,
                          meta: RankMetadata, out, lse, stream=None) -> None:
    """``rank_attention`` with the library's static scratch array as its
    workspace: allocates nothing.  Calls that overlap on one GPU race."""
    _attn_shapes(geom, q, kv_pool, out, lse)
    g = geom.c()
    m = meta.c()
    _check(lib.dcpmla_rank_attention_static(ctypes.byref(g), _ptr(q), _ptr(kv_pool), kv_scale,
                                            softmax_scale, ctypes.byref(m), _ptr(out), _ptr(lse),
                                            _stream(stream)),
           "dcpmla_rank_attention_static")


def static_scratch_bytes() -> int:
    return int(lib.dcpmla_static_scratch_bytes())


def merge_ranks(out_ranks, lse_ranks, out, lse, stream=None) -> None:
    """``out_ranks [W, ..., 512]`` bf16, ``lse_ranks [W, ...]`` f32 -> ``out``, ``lse``."""
    W = out_ranks.shape[0]
    rows = lse_ranks[0].numel()
    _need(out_ranks, torch.bfloat16, (W, *lse_ranks.shape[1:], D_V), "out_ranks")
    _need(lse_ranks, torch.float32, (W, *lse_ranks.shape[1:]), "lse_ranks")
    _need(out, torch.bfloat16, (*lse_ranks.shape[1:], D_V), "out")
    _need(lse, torch.float32, tuple(lse_ranks.shape[1:]), "lse")
    _check(lib.dcpmla_merge_ranks(W, rows, _ptr(out_ranks), _ptr(lse_ranks), _ptr(out), _ptr(lse),
                                  _stream(stream)),
           "dcpmla_merge_ranks")


def merge_segments_dense(o_seg, lse2_seg, out, lse, stream=None) -> None:
    """``o_seg [rows, nseg, 512]`` f32, ``lse2_seg [rows, nseg]`` f32 -> bf16 ``out``, ``lse``."""
    rows, nseg = lse2_seg.shape
    _need(o_seg, torch.float32, (rows, nseg, D_V), "o_seg")
    _need(lse2_seg, torch.float32, (rows, nseg), "lse2_seg")
    _need(out, torch.bfloat16, (rows, D_V), "out")
    _need(lse, torch.float32, (rows,), "lse")
    _check(lib.dcpmla_merge_segments_dense(rows, nseg, _ptr(o_seg), _ptr(lse2_seg), _ptr(out),
                                           _ptr(lse), _stream(stream)),
           "dcpmla_merge_segments_dense")


def device_info(device: int = 0) -> dict:
    """CU count, clocks and memory interface of a HIP device (host query)."""
    info = _lib.DeviceInfo()
    _check(_lib.lib.dcpmla_get_device_info(int(device), ctypes.byref(info)), "dcpmla_get_device_info")
    return {"compute_units": info.compute_units, "clock_khz": info.clock_khz,
            "memory_clock_khz": info.memory_clock_khz, "memory_bus_bits": info.memory_bus_bits,
            "lds_bytes_per_block": info.lds_bytes_per_block, "arch": info.arch.decode()}


def a2a_message_elems(dim: int) -> int:
    n = int(lib.dcpmla_a2a_message_elems(int(dim)))
    _check(min(n, 0), "dcpmla_a2a_message_elems")
    return n


def split_q_bytes(rows: int) -> int:
    """Bytes of the tiled split of ``rows`` head-rows (``dcpmla_split_q_bytes``)."""
    n = int(lib.dcpmla_split_q_bytes(int(rows)))
    _check(min(n, 0), "dcpmla_split_q_bytes")
    return n


def split_q(q, q_split, inv_scale, stream=None) -> None:
    """``q [..., 576]`` bf16 -> ``q_split [split_q_bytes(rows)]`` uint8 (hi and lo codes, tiled as
    ``include/dcpmla.h`` describes), ``inv_scale [rows]`` f32."""
    rows = q.numel() // D_QK
    _need(q, torch.bfloat16, (*q.shape[:-1], D_QK), "q")
    _need(q_split, torch.uint8, (split_q_bytes(rows),), "q_split")
    _need(inv_scale, torch.float32, (rows,), "inv_scale")
    _check(lib.dcpmla_split_q(rows, _ptr(q), _ptr(q_split), _ptr(inv_scale), _stream(stream)), "dcpmla_split_q")


def a2a_pack(world: int, out_rank, lse_rank, send, stream=None) -> None:
    """``out_rank [T, H, D]`` bf16, ``lse_rank [T, H]`` f32 -> ``send [W, T, H/W, D + 8]`` bf16."""
    T, H, D = out_rank.shape
    _need(out_rank, torch.bfloat16, (T, H, D), "out_rank")
    _need(lse_rank, torch.float32, (T, H), "lse_rank")
    _need(send, torch.bfloat16, (world, T, H // world, a2a_message_elems(D)), "send")
    _check(lib.dcpmla_a2a_pack(world, T, H, D, _ptr(out_rank), _ptr(lse_rank), _ptr(send), _stream(stream)),
           "dcpmla_a2a_pack")


def a2a_combine(recv, out, lse, stream=None) -> None:
    """``recv [W, T, Hl, D + 8]`` bf16 -> ``out [T, Hl, D]`` bf16, ``lse [T, Hl]`` f32."""
    W, T, Hl, _ = recv.shape
    D = out.shape[-1]
    _need(recv, torch.bfloat16, (W, T, Hl, a2a_message_elems(D)), "recv")
    _need(out, torch.bfloat16, (T, Hl, D), "out")
    _need(lse, torch.float32, (T, Hl), "lse")
    _check(lib.dcpmla_a2a_combine(W, T, Hl, D, _ptr(recv), _ptr(out), _ptr(lse), _stream(stream)),
           "dcpmla_a2a_combine")


def project_heads(o, w_v_t, out, stream=None) -> None:
    """``o [T, H, 512]`` bf16, ``w_v_t [H, DV, 512]`` bf16 -> ``out [T, H, DV]`` bf16."""
    T, H, _ = o.shape
    DV = w_v_t.shape[1]
    _need(o, torch.bfloat16, (T, H, D_V), "o")
    _need(w_v_t, torch.bfloat16, (H, DV, D_V), "w_v_t")
    _need(out, torch.bfloat16, (T, H, DV), "out")
    _check(lib.dcpmla_project_heads(T, H, DV, _ptr(o), _ptr(w_v_t), _ptr(out), _stream(stream)),
           "dcpmla_project_heads")
