"""dcpmla_rank_attention_static -- the per-rank attention with the library's
static scratch array as its workspace -- against dcpmla_rank_attention with a
caller workspace, through the C ABI.

Both run the same kernels over the same persistent grid, so their outputs and
LSEs agree bit for bit; the static variant is also checked against the oracle
on the smaller call.  Two calls in a row on one GPU, the second with a smaller
input (and the other cache format), show that the array's leftover contents
from the first call do not leak into the second.  The size limit is checked on
the host.
"""
import ctypes

import numpy as np
import pytest
import torch

from synth import make_config
from gpu_util import (bf16_to_f64, check_rank, device_inputs, fmt_stats, geometry,
                      rank_expectations)


def _ops():
    from decode_context_parallelism_amd import ops
    return ops


def test_static_scratch_size_limit_on_host():
    # a request whose workspace exceeds the array is refused before any launch
    from decode_context_parallelism_amd import _lib
    ops = _ops()
    limit = ops.static_scratch_bytes()
    assert limit == 160 << 20
    w = make_config(1)
    g = geometry(w, groups=1024)            # 1024 groups x 0.5 MB of partials > 160 MiB
    assert _lib.lib.dcpmla_workspace_bytes(ctypes.byref(g.c())) > limit
    fake = ctypes.c_void_p(4096)            # never dereferenced: the call returns first
    meta = _lib.Meta(fake, fake, fake, fake, fake)
    st = _lib.lib.dcpmla_rank_attention_static(ctypes.byref(g.c()), fake, fake, 1.0, 0.07,
                                               ctypes.byref(meta), fake, fake, None)
    assert st == -6 and "static scratch" in _lib.strerror(st)


@pytest.mark.gpu
def test_static_matches_workspace_entry_point_two_calls():
    ops = _ops()
    from decode_context_parallelism_amd.group import DcpGroup
    # the larger FP8-cache call first, then a smaller BF16-cache call
    for k in (2, 1):
        w = make_config(k)
        print(f"static scratch: config {k} {w.name}", flush=True)
        g = geometry(w)
        d = device_inputs(w)
        grp = DcpGroup(g, "cuda")
        grp.write_kv(d["seq_ids"], d["positions"], d["latents"], d["block_table"])
        grp.build_metadata(d["ctx_lens"], d["block_table"])
        assert ops.workspace_bytes(g) <= ops.static_scratch_bytes()
        out_s = torch.empty_like(grp.out_ranks)
        lse_s = torch.empty_like(grp.lse_ranks)
        for r in range(w.world):
            grp.rank_attention(r, d["q"], w.kv_scale, w.softmax_scale)
            ops.rank_attention_static(g, d["q"], grp.pools[r], w.kv_scale, w.softmax_scale, grp.meta[r],
                                      out_s[r], lse_s[r])
        torch.cuda.synchronize()
        assert grp.errors() == 0
        assert torch.equal(out_s.view(torch.int16), grp.out_ranks.view(torch.int16))
        assert torch.equal(lse_s.view(torch.int32), grp.lse_ranks.view(torch.int32))
        if k == 1:
            rows = [(b, i) for b in range(w.batch) for i in range(w.qlen)]
            o, l = rank_expectations(w, rows)
            for r in range(w.world):
                st = check_rank(w, bf16_to_f64(out_s[r]), lse_s[r].cpu().numpy().astype(np.float64),
                                o[r], l[r], rows, tag=f"static rank {r}")
                print(f"static scratch config {k} rank {r}: {fmt_stats(st)}", flush=True)
