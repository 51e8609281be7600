"""Float64 / bit-level oracle of the exchange around the cross-rank merge.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"Context Parallel Guide (PCP & DCP)" (ATOM docs):
  * comm_backend, a2a: each rank sends every peer that peer's slice of heads
    of its partial output with the LSE packed alongside, in one all-to-all,
    and the combine is done locally; the fp32 LSE travels through two 16-bit
    halves of the bf16 buffer.
  * enable_project_before_merge: the merge is a per-(token, head) scalar
    weighting plus a cross-rank sum and W_V is a per-head linear map, so the
    two commute; projecting first shrinks the payload from the latent width
    to v_head_dim per head.

Message row (reading of the pages, which fix only "LSE packed alongside"):
``dim`` bf16 values, then the LSE's low and high 16 bits, then six zeros.
"""
import numpy as np


def lse_halves(lse):
    """fp32 LSE -> (low 16 bits, high 16 bits) as uint16 arrays."""
    bits = np.ascontiguousarray(np.asarray(lse, dtype=np.float32)).view(np.uint32)
    return (bits & 0xFFFF).astype(np.uint16), (bits >> 16).astype(np.uint16)


def join_halves(lo, hi):
    """Inverse of ``lse_halves``."""
    bits = np.asarray(lo, dtype=np.uint32) | (np.asarray(hi, dtype=np.uint32) << 16)
    return bits.astype(np.uint32).view(np.float32)


def a2a_pack(out_bits, lse, world):
    """One rank's send buffer: out_bits [T, H, D] uint16 (bf16 patterns), lse
    [T, H] fp32 -> [W, T, H/W, D + 8] uint16; block p holds heads of slice p."""
    out_bits = np.asarray(out_bits, dtype=np.uint16)
    T, H, D = out_bits.shape
    Hl = H // world
    send = np.zeros((world, T, Hl, D + 8), dtype=np.uint16)
    lo, hi = lse_halves(lse)
    for p in range(world):
        heads = slice(p * Hl, (p + 1) * Hl)
        send[p, :, :, :D] = out_bits[:, heads]
        send[p, :, :, D] = lo[:, heads]
        send[p, :, :, D + 1] = hi[:, heads]
    return send


def all_to_all(sends):
    """The collective between packing and combining: block p of rank r's send
    buffer becomes block r of rank p's receive buffer."""
    W = len(sends)
    return [np.stack([sends[r][p] for r in range(W)]) for p in range(W)]


def unpack(recv):
    """recv [W, T, Hl, D + 8] -> (out_bits [W, T, Hl, D], lse [W, T, Hl])."""
    D = recv.shape[-1] - 8
    return recv[..., :D], join_halves(recv[..., D], recv[..., D + 1])


def project_heads(o, w_v):
    """Per-head projection: o [T, H, 512] times W_V[h] [512, DV] -> [T, H, DV]."""
    return np.einsum("thk,hkn->thn", np.asarray(o, dtype=np.float64), np.asarray(w_v, dtype=np.float64))
