"""The C-ABI library on the host: it loads, exports every declared symbol, and
its host-only logic (validation, sizes, aliasing and argument checks) behaves.

No kernel is launched here; every call below either needs no device or is
refused before any HIP call.
"""
import ctypes
import os
import re

import pytest

from oracle import layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dcpmla.h")

ops = pytest.importorskip("decode_context_parallelism_amd.ops",
                          reason="libdcpmla.so not built (run __graft_entry__.build())")
from decode_context_parallelism_amd import _lib  # noqa: E402


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dcpmla_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    syms = declared_symbols()
    assert len(syms) >= 12
    for s in syms:
        assert hasattr(_lib.lib, s), s
    assert set(syms) == set(_lib.SIGNATURES)


def test_header_is_plain_c():
    text = open(HEADER).read()
    assert 'extern "C"' in text
    assert "torch" not in text and "at::" not in text


def _geom(**kw):
    base = dict(dcp_world=2, interleave=1, block_size=16, qlen=3, num_heads=16, batch=1,
                max_blocks_per_seq=3, max_local_pages=4, kv_dtype="bf16", num_blocks=8, groups=4)
    base.update(kw)
    return ops.Geometry(**base)


def test_validate_interleave_rules():
    # "Context Parallel Guide (PCP & DCP)", interleave_size: 1 <= S <= block_size,
    # block_size % S == 0 when S > 1, S > 1 needs dcp > 1
    assert ops.validate(_geom()) == _lib.OK
    assert ops.validate(_geom(interleave=16, dcp_world=8, block_size=64)) == _lib.OK
    assert ops.validate(_geom(interleave=0)) == _lib.E_INVALID
    assert ops.validate(_geom(interleave=32, block_size=16)) == _lib.E_INVALID
    assert ops.validate(_geom(interleave=3, block_size=16)) == _lib.E_INVALID
    assert ops.validate(_geom(interleave=2, dcp_world=1)) == _lib.E_INVALID
    assert ops.validate(_geom(interleave=1, dcp_world=1)) == _lib.OK


@pytest.mark.parametrize("field,value", [("dcp_world", 0), ("block_size", 0), ("qlen", 0),
                                         ("num_heads", 0), ("batch", 0), ("max_local_pages", 0),
                                         ("max_blocks_per_seq", 0), ("num_blocks", 0),
                                         ("groups", -1), ("groups", 5000)])
def test_validate_rejects(field, value):
    assert ops.validate(_geom(**{field: value})) == _lib.E_INVALID


@pytest.mark.parametrize("ok,bad", [
    # pool token rows (num_blocks x block_size) stay below 2^31: the kernels
    # index token rows and pages with 32-bit integers
    (dict(block_size=64, num_blocks=(1 << 25) - 1), dict(block_size=64, num_blocks=1 << 25)),
    # a row's local capacity (max_local_pages x subpage size) stays below 2^31 tokens
    (dict(max_local_pages=(1 << 27) - 1), dict(max_local_pages=1 << 27)),
    # work units (sequences x head-row tiles x 32-token stages of that capacity)
    (dict(batch=256, qlen=8, num_heads=128, max_local_pages=(1 << 21) - 2),
     dict(batch=256, qlen=8, num_heads=128, max_local_pages=1 << 21)),
    # head-rows x 576 query elements
    (dict(batch=3728269, qlen=1, num_heads=1), dict(batch=3728270, qlen=1, num_heads=1)),
    # block-table entries
    (dict(batch=1 << 16, max_blocks_per_seq=(1 << 15) - 1), dict(batch=1 << 16, max_blocks_per_seq=1 << 15)),
])
def test_validate_size_limits(ok, bad):
    # each limit of 32-bit device index arithmetic: the largest geometry below
    # it is accepted, the first one at it refused before any launch
    assert ops.validate(_geom(**ok)) == _lib.OK
    assert ops.validate(_geom(**bad)) == _lib.E_INVALID


def test_validate_rejects_bad_dtype():
    g = _geom().c()
    g.kv_dtype = 7
    assert _lib.lib.dcpmla_validate(ctypes.byref(g)) == _lib.E_INVALID


def test_validate_q_format():
    assert ops.validate(_geom(kv_dtype="fp8_e4m3", q_format="fp8")) == _lib.OK
    assert ops.validate(_geom(kv_dtype="bf16", q_format="fp8")) == _lib.E_INVALID   # FP8 cache only
    g = _geom().c()
    g.q_format = 2
    assert _lib.lib.dcpmla_validate(ctypes.byref(g)) == _lib.E_INVALID


def test_validate_row_boundary():
    assert ops.validate(_geom(row_boundary="block")) == _lib.OK
    g = _geom().c()
    g.row_boundary = 2
    assert _lib.lib.dcpmla_validate(ctypes.byref(g)) == _lib.E_INVALID


def test_subpage_size_matches_oracle():
    for bs in range(1, 1100):
        assert ops.subpage_size(bs) == layout.subpage_size(bs)
    assert ops.subpage_size(0) == _lib.E_INVALID


def test_sizes():
    g = _geom(batch=5)
    # partition (4B + 2 ints), padded to 64 ints, then one zero latent row
    assert ops.work_ints(g) == 64 + 576 * 2 // 4
    ws = ops.workspace_bytes(g)
    # per group: 2 slots x 128 rows x (512 partial values + 1 lse2) floats; then a 16-byte scale
    # slot; then, 256-byte aligned, the split query (1152 bytes per head-row in blocks of 32
    # rows, the last block padded) and a float scale per head-row
    part = 4 * 2 * 128 * (512 + 1) * 4 + 16
    rows = 5 * 3 * 16
    split = (rows + 31) // 32 * 32 * 1152
    assert ws == (part + 255) // 256 * 256 + split + rows * 4
    part1 = 1 * 2 * 128 * (512 + 1) * 4 + 16
    assert ops.workspace_bytes(_geom(groups=1, batch=5)) == (part1 + 255) // 256 * 256 + split + rows * 4


def test_split_q_bytes():
    # whole 32-row blocks of 36 KiB
    assert [ops.split_q_bytes(r) for r in (0, 1, 31, 32, 33, 96, 97)] == \
        [0, 36864, 36864, 36864, 73728, 110592, 147456]
    assert _lib.lib.dcpmla_split_q_bytes(-1) == _lib.E_INVALID
    assert _lib.lib.dcpmla_split_q_bytes(1 << 40) == _lib.E_INVALID


def test_split_q_checks():
    L = _lib.lib
    assert L.dcpmla_split_q(-1, FAKE, FAKE + 10 ** 7, FAKE + 2 * 10 ** 7, None) == _lib.E_INVALID
    assert L.dcpmla_split_q(4, None, FAKE + 10 ** 7, FAKE + 2 * 10 ** 7, None) == _lib.E_INVALID
    assert L.dcpmla_split_q(4, FAKE, FAKE + 100, FAKE + 2 * 10 ** 7, None) == _lib.E_ALIAS     # split over q
    assert L.dcpmla_split_q(4, FAKE, FAKE + 10 ** 7, FAKE + 10 ** 7 + 64, None) == _lib.E_ALIAS  # scale over split
    assert L.dcpmla_split_q(0, None, None, None, None) == _lib.OK


def test_strerror():
    for code in (0, -1, -2, -3, -4, -5):
        assert _lib.strerror(code)
    assert "overlap" in _lib.strerror(_lib.E_ALIAS)


FAKE = 1 << 40   # host-only checks run before any device access


def test_partial_attention_split_checks():
    L = _lib.lib
    m = _meta(FAKE + 10 ** 9)
    wsb = ops.workspace_bytes(_geom(kv_dtype="fp8_e4m3"))
    args = lambda g, **o: [ctypes.byref(g), o.get("qs", FAKE), o.get("qsc", FAKE + 10 ** 6), FAKE + 10 ** 7,
                           1.0, 0.07, ctypes.byref(m), FAKE + 2 * 10 ** 7, wsb, FAKE + 4 * 10 ** 7,
                           FAKE + 5 * 10 ** 7, None]
    g8 = _geom(kv_dtype="fp8_e4m3").c()
    assert L.dcpmla_partial_attention_split(*args(_geom(kv_dtype="bf16").c())) == _lib.E_INVALID  # FP8 only
    assert L.dcpmla_partial_attention_split(*args(g8, qs=None)) == _lib.E_INVALID
    assert L.dcpmla_partial_attention_split(*args(g8, qsc=FAKE + 4 * 10 ** 7 + 8)) == _lib.E_ALIAS  # scale in out


def test_merge_ranks_alias_and_args():
    L = _lib.lib
    rows = 100
    ins = FAKE
    # output overlapping the input partials
    assert L.dcpmla_merge_ranks(2, rows, ins, ins + 10 ** 6, ins + 1024, ins + 10 ** 8, None) == _lib.E_ALIAS
    assert L.dcpmla_merge_ranks(0, rows, ins, ins + 10 ** 6, ins + 10 ** 7, ins + 10 ** 8, None) == _lib.E_INVALID
    assert L.dcpmla_merge_ranks(2, rows, None, ins, ins, ins, None) == _lib.E_INVALID
    # out and lse overlapping each other
    assert L.dcpmla_merge_ranks(2, rows, ins, ins + 10 ** 6, ins + 10 ** 7, ins + 10 ** 7 + 64, None) == _lib.E_ALIAS


def test_merge_segments_dense_args():
    L = _lib.lib
    assert L.dcpmla_merge_segments_dense(10, 0, FAKE, FAKE + 10 ** 6, FAKE + 10 ** 7, FAKE + 10 ** 8, None) == _lib.E_INVALID
    assert L.dcpmla_merge_segments_dense(10, 3, FAKE, FAKE + 10 ** 6, FAKE + 100, FAKE + 10 ** 8, None) == _lib.E_ALIAS


def _meta(base):
    return _lib.Meta(base, base + 10 ** 5, base + 2 * 10 ** 5, base + 3 * 10 ** 5, base + 4 * 10 ** 5)


def test_attention_checks_before_launch():
    L = _lib.lib
    g = _geom().c()
    m = _meta(FAKE + 10 ** 9)
    q, pool, ws, out, lse = FAKE, FAKE + 10 ** 7, FAKE + 2 * 10 ** 7, FAKE + 4 * 10 ** 7, FAKE + 5 * 10 ** 7
    wsb = ops.workspace_bytes(_geom())
    args = lambda **o: [ctypes.byref(g), o.get("q", q), o.get("pool", pool), o.get("kvs", 1.0),
                        o.get("sms", 0.07), ctypes.byref(o.get("m", m)), o.get("ws", ws),
                        o.get("wsb", wsb), o.get("out", out), o.get("lse", lse), None]
    assert L.dcpmla_partial_attention(*args(wsb=wsb - 1)) == _lib.E_WORKSPACE
    assert L.dcpmla_partial_attention(*args(out=q + 64)) == _lib.E_ALIAS            # out over q
    assert L.dcpmla_partial_attention(*args(ws=pool + 128)) == _lib.E_ALIAS         # workspace over pool
    assert L.dcpmla_partial_attention(*args(lse=FAKE + 10 ** 9 + 8)) == _lib.E_ALIAS  # lse over metadata
    assert L.dcpmla_partial_attention(*args(kvs=0.0)) == _lib.E_INVALID
    assert L.dcpmla_partial_attention(*args(sms=float("inf"))) == _lib.E_INVALID
    assert L.dcpmla_partial_attention(*args(q=None)) == _lib.E_INVALID
    bad = _lib.Meta(0, 1, 2, 3, 4)
    assert L.dcpmla_partial_attention(*args(m=bad)) == _lib.E_INVALID
    g.qlen = 0
    assert L.dcpmla_partial_attention(*args()) == _lib.E_INVALID


def test_build_metadata_checks_before_launch():
    L = _lib.lib
    g = _geom().c()
    m = _meta(FAKE)
    assert L.dcpmla_build_metadata(ctypes.byref(g), 2, FAKE + 10 ** 8, FAKE + 10 ** 9, ctypes.byref(m), None) == _lib.E_INVALID
    assert L.dcpmla_build_metadata(ctypes.byref(g), -1, FAKE + 10 ** 8, FAKE + 10 ** 9, ctypes.byref(m), None) == _lib.E_INVALID
    # block table aliasing the page table output
    assert L.dcpmla_build_metadata(ctypes.byref(g), 0, FAKE + 10 ** 8, FAKE + 10 ** 5, ctypes.byref(m), None) == _lib.E_ALIAS


def test_write_kv_checks_before_launch():
    L = _lib.lib
    g = _geom().c()
    T = 64
    assert L.dcpmla_write_kv(ctypes.byref(g), 5, T, FAKE, FAKE + 10 ** 6, FAKE + 2 * 10 ** 6, FAKE + 3 * 10 ** 6,
                             FAKE + 4 * 10 ** 6, FAKE + 6 * 10 ** 6, FAKE + 7 * 10 ** 6, None) == _lib.E_INVALID
    # pool overlapping the latents
    assert L.dcpmla_write_kv(ctypes.byref(g), 0, T, FAKE, FAKE + 10 ** 6, FAKE + 2 * 10 ** 6, FAKE + 3 * 10 ** 6,
                             FAKE + 2 * 10 ** 6 + 64, FAKE + 6 * 10 ** 6, FAKE + 7 * 10 ** 6, None) == _lib.E_ALIAS
