"""The exchange around the cross-rank merge on the GPU, through the C ABI.

* a2a pack: bit-exact against the oracle's message layout (the bf16 values
  move unchanged and the fp32 LSE is split into its two 16-bit halves);
* local combine after the all-to-all: bit-identical to the direct rank merge
  kernel (same arithmetic and order) and within the merge tolerance of the
  float64 oracle;
* project-before-merge: the per-head W_V projection against float64, and the
  whole PBM route (project each rank's partial, pack, exchange, combine) on
  seeded partials shaped like a verify step, against projecting the oracle's
  merge of the same partials.

The all-to-all itself is a collective: here one GPU plays every rank and the
exchange is a copy between the ranks' buffers.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import exchange as X
from oracle import formats
from gpu_util import bf16_half_ulp

pytestmark = pytest.mark.gpu


def _ops():
    from decode_context_parallelism_amd import ops
    return ops


def _partials(seed, W, T, H, D):
    rng = np.random.default_rng(seed)
    bits = (rng.standard_normal((W, T, H, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    lse = (rng.standard_normal((W, T, H)) * 3).astype(np.float32)
    lse[0, 0, :] = -np.inf
    lse[:, min(1, T - 1), 0] = -np.inf
    return bits, lse


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _exchange(sends):
    W = len(sends)
    return [torch.stack([sends[r][p] for r in range(W)]).contiguous() for p in range(W)]


@pytest.mark.parametrize("W,T,H,D", [(2, 3, 32, 512), (8, 40, 128, 512), (8, 7, 64, 128), (4, 5, 16, 64)])
def test_pack_bit_exact(W, T, H, D):
    ops = _ops()
    bits, lse = _partials(W * 100 + T, W, T, H, D)
    for r in range(W):
        send = torch.empty(W, T, H // W, D + 8, dtype=torch.bfloat16, device="cuda")
        send.fill_(7.0)   # every element must be written
        ops.a2a_pack(W, _dev_bf16(bits[r]), torch.from_numpy(lse[r]).cuda(), send)
        torch.cuda.synchronize()
        got = send.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, X.a2a_pack(bits[r], lse[r], W))


@pytest.mark.parametrize("W,T,H,D", [(2, 3, 32, 512), (8, 40, 128, 512), (8, 7, 64, 128)])
def test_combine_equals_rank_merge(W, T, H, D):
    ops = _ops()
    bits, lse = _partials(W * 7 + T, W, T, H, D)
    sends = []
    for r in range(W):
        send = torch.empty(W, T, H // W, D + 8, dtype=torch.bfloat16, device="cuda")
        ops.a2a_pack(W, _dev_bf16(bits[r]), torch.from_numpy(lse[r]).cuda(), send)
        sends.append(send)
    recvs = _exchange(sends)
    Hl = H // W
    outs, lses = [], []
    for p in range(W):
        o = torch.empty(T, Hl, D, dtype=torch.bfloat16, device="cuda")
        l = torch.empty(T, Hl, dtype=torch.float32, device="cuda")
        ops.a2a_combine(recvs[p], o, l)
        outs.append(o)
        lses.append(l)
    torch.cuda.synchronize()
    comb_o = torch.cat(outs, dim=1).view(torch.int16).cpu().numpy()
    comb_l = torch.cat(lses, dim=1).cpu().numpy()
    ref_o, ref_l = A.merge_ranks(formats.decode_bf16(bits), lse.astype(np.float64))
    got_o = formats.decode_bf16(comb_o.view(np.uint16))
    emp = np.isneginf(ref_l)
    assert np.all(np.isneginf(comb_l[emp])) and np.all(got_o[emp] == 0.0)
    assert np.all(np.abs(got_o - ref_o) <= 2.0 ** -8 * np.abs(ref_o) + 1e-5)
    assert np.all(np.abs(comb_l[~emp] - ref_l[~emp]) <= 1e-4)
    if D == 512:
        # the direct rank merge on the same partials gives the same bits
        mo = torch.empty(T, H, D, dtype=torch.bfloat16, device="cuda")
        ml = torch.empty(T, H, dtype=torch.float32, device="cuda")
        ops.merge_ranks(_dev_bf16(bits), torch.from_numpy(lse).cuda(), mo, ml)
        torch.cuda.synchronize()
        assert np.array_equal(mo.view(torch.int16).cpu().numpy(), comb_o)
        assert np.array_equal(ml.cpu().numpy().view(np.uint32), comb_l.view(np.uint32))


def _w_v(H, DV, seed):
    w = (np.random.default_rng(seed).standard_normal((H, DV, 512)) / np.sqrt(512)).astype(np.float32)
    bits = (w.view(np.uint32) >> 16).astype(np.uint16)          # bf16 W_V^T patterns
    return bits, formats.decode_bf16(bits).transpose(0, 2, 1)    # [H, 512, DV] float64


def _projection_bound(o, w, exact):
    # BF16 rounding of the result (half an ulp of the binade above the exact
    # value covers a sum that crossed a power of two) plus fp32 accumulation
    # over 512 products
    acc = np.einsum("thk,hkn->thn", np.abs(o), np.abs(w))
    return 2 * bf16_half_ulp(exact) + 2.0 ** -20 * acc


@pytest.mark.parametrize("T,H,DV", [(1, 4, 128), (37, 16, 128), (160, 128, 128), (5, 3, 256)])
def test_project_heads(T, H, DV):
    ops = _ops()
    rng = np.random.default_rng(T * H)
    obits = (rng.standard_normal((T, H, 512)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    wbits, w = _w_v(H, DV, T + H)
    out = torch.empty(T, H, DV, dtype=torch.bfloat16, device="cuda")
    ops.project_heads(_dev_bf16(obits), _dev_bf16(wbits), out)
    torch.cuda.synchronize()
    o = formats.decode_bf16(obits)
    exact = X.project_heads(o, w)
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - exact) <= _projection_bound(o, w, exact))


@pytest.mark.parametrize("W,B,q,H", [(2, 1, 3, 16), (2, 8, 3, 96), (8, 4, 3, 128)])
def test_project_before_merge_route(W, B, q, H):
    # seeded BF16 partials and LSEs with the shapes of a DCP verify step (the
    # workloads' world, rows and heads); PBM route on the GPU against
    # projecting the float64 merge of the same partials
    ops = _ops()
    T = B * q
    DV = 128
    bits, lse_np = _partials(1000 * W + H, W, T, H, 512)
    wbits, wv = _w_v(H, DV, 11 * W + H)
    wdev = _dev_bf16(wbits)
    Hl = H // W
    sends, proj_bits = [], []
    for r in range(W):
        pr = torch.empty(T, H, DV, dtype=torch.bfloat16, device="cuda")
        ops.project_heads(_dev_bf16(bits[r]), wdev, pr)
        send = torch.empty(W, T, Hl, DV + 8, dtype=torch.bfloat16, device="cuda")
        ops.a2a_pack(W, pr, torch.from_numpy(lse_np[r]).cuda(), send)
        sends.append(send)
        proj_bits.append(pr)
    recvs = _exchange(sends)
    outs, lses = [], []
    for p in range(W):
        o = torch.empty(T, Hl, DV, dtype=torch.bfloat16, device="cuda")
        l = torch.empty(T, Hl, dtype=torch.float32, device="cuda")
        ops.a2a_combine(recvs[p], o, l)
        outs.append(o)
        lses.append(l)
    torch.cuda.synchronize()
    got = torch.cat(outs, dim=1).float().cpu().numpy().astype(np.float64)
    got_l = torch.cat(lses, dim=1).cpu().numpy().astype(np.float64)
    o_r = formats.decode_bf16(bits)
    l_r = lse_np.astype(np.float64)
    mo, ml = A.merge_ranks(o_r, l_r)
    exact = X.project_heads(mo, wv)
    # bound: the final BF16 rounding, plus each rank's projected partial --
    # BF16-rounded and accumulated in fp32 -- weighted by its merge weight
    # (the weights sum to 1); 1e-6 covers the fp32 combine itself
    # The final rounding acts on the fp32 value, which may sit just past a
    # power of two from the exact one: charge half an ulp of the larger binade
    with np.errstate(invalid="ignore"):
        wts = np.where(np.isneginf(l_r), 0.0, np.exp(l_r - ml[None]))
    bound = np.maximum(bf16_half_ulp(exact), bf16_half_ulp(got)) + 1e-6
    for r in range(W):
        proj_exact = X.project_heads(o_r[r], wv)
        bound = bound + wts[r][..., None] * _projection_bound(o_r[r], wv, proj_exact)
    emp = np.isneginf(ml)
    assert np.all(np.isneginf(got_l[emp])) and np.all(got[emp] == 0.0)
    bad = np.abs(got - exact) > bound
    if bad.any():
        t, h, n = np.argwhere(bad)[np.argmax((np.abs(got - exact) - bound)[bad])]
        detail = {"t": int(t), "h": int(h), "n": int(n), "got": float(got[t, h, n]),
                  "exact": float(exact[t, h, n]), "bound": float(bound[t, h, n]),
                  "bad_count": int(bad.sum()), "bad_heads": sorted(set(np.argwhere(bad)[:, 1].tolist()))[:20],
                  "bad_tokens": sorted(set(np.argwhere(bad)[:, 0].tolist()))[:30],
                  "proj_r": [float(X.project_heads(o_r[r], wv)[t, h, n]) for r in range(W)],
                  "gpu_proj_r": [float(proj_bits[r][t, h, n].float()) for r in range(W)],
                  "w_r": [float(wts[r][t, h]) for r in range(W)], "lse_r": [float(l_r[r][t, h]) for r in range(W)]}
        raise AssertionError(detail)
    assert np.all(np.abs(got_l[~emp] - ml[~emp]) <= 1e-4)
