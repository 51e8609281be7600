"""The two-term E4M3 split of the query on the GPU, through the C ABI.

The codes are integer output of the split: hi, lo and the per-row 2^-k must
equal the float64 oracle's bit for bit (oracle/qsplit.py: round to nearest
E4M3, ties to even, residual of the same, k the largest exponent that fits
448).  The library stores the codes tiled for its attention kernel
(include/dcpmla.h, dcpmla_split_q); the test undoes the tiling on the host
before comparing.  The attention parity tests cover the split's use inside
the FP8-cache attention on every workload.
"""
import numpy as np
import pytest
import torch

from oracle import formats, qsplit

pytestmark = pytest.mark.gpu


def _ops():
    from decode_context_parallelism_amd import ops
    return ops


def _bf16_bits(v):
    v = np.ascontiguousarray(v, dtype=np.float32)
    u = v.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _rows(seed):
    rng = np.random.default_rng(seed)
    rows = [rng.standard_normal((300, 576)).astype(np.float32),
            (rng.standard_normal((200, 576)) * np.exp2(rng.uniform(-14, 6, (200, 576)))).astype(np.float32)]
    edge = np.zeros((12, 576), dtype=np.float32)
    edge[1, 7] = 3.0                                   # one non-zero element
    edge[2] = 448.0; edge[2, 1::2] = -448.0            # at the top of the range, scale 1
    # amax = 448 (k = 0) and E4M3 midpoints that BF16 holds exactly: ties to even
    edge[3] = 1.0625; edge[3, 0] = 448.0; edge[3, 1] = 2.125; edge[3, 2] = -1.1875; edge[3, 3] = 0.0078125 * 3
    edge[4] = 1.75 * 2.0 ** 3                         # mantissa at the 1.75 threshold
    edge[5] = 1.7578125 * 2.0 ** -5                   # just above it
    edge[6] = 2.0 ** -130                             # BF16 subnormals (amax tiny)
    edge[7] = -0.0; edge[7, 5] = 1.0                  # negative zeros
    edge[8] = rng.standard_normal(576) * 1e-30
    edge[9] = rng.standard_normal(576) * 1e30
    edge[10, ::3] = 5.0; edge[10, 1::3] = 5.0 * 2.0 ** -12   # elements far below the row maximum
    edge[11] = -edge[3]
    rows.append(edge)
    return np.concatenate(rows)


def _untile(flat, R):
    """Tiled split bytes -> (hi [R, 576], lo [R, 576]).  Block n, chunk c = 4t + 2 term + half,
    bytes 16 (32 g + i) + e hold row 32 n + i, dim 64t + 32g + 16 half + e of that term."""
    nb = (R + 31) // 32
    a = flat.reshape(nb, 9, 2, 2, 2, 32, 16)          # n, t, term, half, g, i, e
    a = a.transpose(0, 5, 2, 1, 4, 3, 6)              # n, i, term, t, g, half, e
    a = a.reshape(nb * 32, 2, 576)[:R]
    return a[:, 0], a[:, 1]


def _padding_rows(flat, R):
    """Bytes of the last block that belong to rows R .. (padding)."""
    nb = (R + 31) // 32
    a = flat.reshape(nb, 9, 2, 2, 2, 32, 16)
    return a[nb - 1, :, :, :, :, R - 32 * (nb - 1):, :]


@pytest.mark.parametrize("take", [None, 45])
def test_split_q_matches_oracle_bit_exact(take):
    # all 512 rows (whole blocks), and the first 45 (a ragged last block)
    ops = _ops()
    bits = _bf16_bits(_rows(3))
    if take is not None:
        bits = bits[np.r_[0:33, 500:512]]
    R = bits.shape[0]
    q = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    split = torch.full((ops.split_q_bytes(R),), 0x5A, dtype=torch.uint8, device="cuda")
    inv = torch.full((R,), -1.0, dtype=torch.float32, device="cuda")
    ops.split_q(q, split, inv)
    torch.cuda.synchronize()
    hi_r, lo_r, inv_r = qsplit.split_rows(formats.decode_bf16(bits))
    flat = split.cpu().numpy()
    hi, lo = _untile(flat, R)
    assert np.array_equal(hi, hi_r), np.argwhere(hi != hi_r)[:5]
    assert np.array_equal(lo, lo_r), np.argwhere(lo != lo_r)[:5]
    assert np.array_equal(inv.cpu().numpy().view(np.uint32), inv_r.astype(np.float32).view(np.uint32))
    if R % 32:
        assert (_padding_rows(flat, R) == 0x5A).all()   # padding rows are not written


def test_split_q_zero_rows_is_a_no_op():
    ops = _ops()
    q = torch.zeros((0, 576), dtype=torch.bfloat16, device="cuda")
    split = torch.zeros((0,), dtype=torch.uint8, device="cuda")
    inv = torch.zeros((0,), dtype=torch.float32, device="cuda")
    ops.split_q(q, split, inv)
    torch.cuda.synchronize()


def test_presplit_attention_equals_internal_split():
    # dcpmla_partial_attention (splits the query itself) and
    # dcpmla_partial_attention_split (reads the group's split) run the same
    # arithmetic: their outputs must be identical
    from synth import make_config
    from gpu_util import run_group
    ops = _ops()
    w = make_config(2)
    grp, d = run_group(w)
    for r in range(w.world):
        out = torch.empty_like(grp.out_ranks[r])
        lse = torch.empty_like(grp.lse_ranks[r])
        ops.rank_attention(grp.geom, d["q"], grp.pools[r], w.kv_scale, w.softmax_scale, grp.meta[r],
                           grp.workspace, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out, grp.out_ranks[r]) and torch.equal(lse, grp.lse_ranks[r]), r
