"""Helpers for the GPU tests: device upload of seeded workloads and oracle views.

Inputs come from ``synth``; expected values come from ``oracle``; nothing here
computes any part of the method.
"""
import numpy as np
import torch

from oracle import formats

HAS_GPU = torch.cuda.is_available()


def geometry(w, groups=0, max_local_pages=None, num_blocks=None, row_boundary="causal", q_format="split"):
    from decode_context_parallelism_amd import ops
    return ops.Geometry(dcp_world=w.world, interleave=w.interleave, block_size=w.block_size,
                        qlen=w.qlen, num_heads=w.heads, batch=w.batch,
                        max_blocks_per_seq=w.block_table.shape[1],
                        max_local_pages=max_local_pages or w.max_local_pages,
                        kv_dtype=w.kv_format, num_blocks=num_blocks or w.num_blocks,
                        groups=groups, row_boundary=row_boundary, q_format=q_format)


def device_inputs(w, device="cuda"):
    q = torch.from_numpy(w.q_bits.view(np.int16)).view(torch.bfloat16).to(device)
    if w.kv_format == "fp8_e4m3":
        lat = torch.from_numpy(w.kv).to(device)
    else:
        lat = torch.from_numpy(w.kv.view(np.int16)).view(torch.bfloat16).to(device)
    seq_ids, positions = w.token_arrays()
    return dict(q=q, latents=lat,
                seq_ids=torch.from_numpy(seq_ids).to(device),
                positions=torch.from_numpy(positions).to(device),
                block_table=torch.from_numpy(w.block_table).to(device),
                ctx_lens=torch.from_numpy(w.ctx_lens).to(device))


def run_group(w, groups=0, device="cuda", row_boundary="causal", q_format="split"):
    """Write the KV, build every rank's metadata, run every rank and the merge."""
    from decode_context_parallelism_amd.group import DcpGroup
    g = geometry(w, groups=groups, row_boundary=row_boundary, q_format=q_format)
    d = device_inputs(w, device)
    grp = DcpGroup(g, device)
    grp.write_kv(d["seq_ids"], d["positions"], d["latents"], d["block_table"])
    grp.forward(d["q"], d["ctx_lens"], d["block_table"], w.kv_scale, w.softmax_scale)
    torch.cuda.synchronize()
    return grp, d


def oracle_latents(w):
    def get(b, pos):
        rows = w.kv[w.seq_start[b] + np.asarray(pos, dtype=np.int64)]
        return formats.decode_cache(rows, w.kv_format, w.kv_scale)
    return get


def oracle_q(w, q_format="split"):
    """The query the method multiplies: the BF16 query, or with q_format "fp8"
    its per-row E4M3 quantisation (oracle.qsplit.quantize_rows)."""
    q = formats.decode_bf16(w.q_bits)
    if q_format == "fp8":
        from oracle import qsplit
        q = qsplit.quantize_rows(q)
    return q


def bf16_to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def tolerance(w):
    """Arithmetic max-abs tolerance: 1.5e-2 with an FP8 cache, 5e-3 with BF16."""
    return 1.5e-2 if w.kv_format == "fp8_e4m3" else 5e-3


def bf16_half_ulp(x):
    """Half a BF16 ulp at |x|: the error of a correctly rounded BF16 value.

    BF16 keeps 8 significant bits, so a value in [2^e, 2^(e+1)) is stored to
    within 2^(e-8).  For |x| >= 2 that is 7.8e-3 or more, above the 5e-3 bar
    itself; the output tolerance is therefore the arithmetic bar plus the
    output format's own rounding.
    """
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def output_bound(w, exact, rank_exact=None, rank_weights=None):
    """Per-element bound for a BF16 output against the exact float64 value.

    ``rank_exact``/``rank_weights`` ([W, ...]): for a merged output, each rank's
    BF16-rounded partial adds its half-ulp times its merge weight.
    """
    bound = tolerance(w) + bf16_half_ulp(exact)
    if rank_exact is not None:
        bound = bound + (np.asarray(rank_weights)[..., None] * bf16_half_ulp(rank_exact)).sum(axis=0)
    return bound


LSE_TOL = 1e-3
