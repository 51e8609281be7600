"""Oracle self-checks on the seeded configurations (CPU only).

On the actual configuration inputs: the per-rank windows partition every
row's causal prefix, and the LSE-merge of the float64 per-rank partials
reproduces float64 global causal attention ("[ROCm][MLA][DCP] Support causal
multi-token verification", "Validation": both ranks' partials merged by LSE
are compared against global causal attention).
"""
import numpy as np
import pytest

from oracle import attention as A
from oracle import formats, layout
from synth import make_config


def latents_fn(w):
    def get(b, pos):
        rows = w.kv[w.seq_start[b] + np.asarray(pos, dtype=np.int64)]
        return formats.decode_cache(rows, w.kv_format, w.kv_scale)
    return get


def q64(w):
    return formats.decode_bf16(w.q_bits)


@pytest.mark.parametrize("k", [1, 2])
def test_rank_merge_equals_global_on_config(k):
    w = make_config(k)
    q = q64(w)
    lat = latents_fn(w)
    rows = [(b, i) for b in range(min(w.batch, 3)) for i in range(w.qlen)]
    g_out, g_lse = A.verify_attention(q, lat, w.ctx_lens, w.softmax_scale, rows=rows)
    outs, lses = [], []
    for r in range(w.world):
        o, l = A.verify_attention(q, lat, w.ctx_lens, w.softmax_scale, world=w.world,
                                  interleave=w.interleave, rank=r, rows=rows)
        outs.append(o)
        lses.append(l)
    m_out, m_lse = A.merge_ranks(np.stack(outs), np.stack(lses))
    sel = np.zeros((w.batch, w.qlen), dtype=bool)
    for b, i in rows:
        sel[b, i] = True
    assert np.abs(m_out[sel] - g_out[sel]).max() < 1e-12
    assert np.abs(m_lse[sel] - g_lse[sel]).max() < 1e-12


def test_config4_has_empty_rank_rows():
    # log-uniform contexts with interleave 16 leave some (row, rank) pairs with no KV
    w = make_config(4)
    empty = 0
    for r in range(w.world):
        lens, _, _ = layout.row_metadata(w.ctx_lens, w.block_table, world=w.world,
                                         interleave=w.interleave, block_size=w.block_size,
                                         qlen=w.qlen, rank=r, max_local_pages=w.max_local_pages)
        empty += int((lens == 0).sum())
    assert empty > 0
