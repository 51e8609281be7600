"""LSE merges on the GPU against the float64 oracle, on synthetic partials.

The GPU output is BF16, so the bound is half a BF16 ulp of the exact value
(2^-8 relative) plus fp32 accumulation; LSE to 1e-4 absolute (fp32 exp/log
on values below 100).
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import formats
from synth import random_rank_partials, random_segment_partials

pytestmark = pytest.mark.gpu


def _bf16_dev(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("W,n", [(1, 7), (2, 1000), (8, 4096), (8, 3)])
def test_merge_ranks(W, n):
    from decode_context_parallelism_amd import ops
    bits, lse = random_rank_partials(W, n, seed=W * 1000 + n)
    out = torch.empty(n, 512, dtype=torch.bfloat16, device="cuda")
    lout = torch.empty(n, dtype=torch.float32, device="cuda")
    ops.merge_ranks(_bf16_dev(bits), torch.from_numpy(lse).cuda(), out, lout)
    torch.cuda.synchronize()
    ref_o, ref_l = A.merge_ranks(formats.decode_bf16(bits), lse.astype(np.float64))
    go = out.float().cpu().numpy().astype(np.float64)
    gl = lout.cpu().numpy().astype(np.float64)
    emp = np.isneginf(ref_l)
    assert np.all(np.isneginf(gl[emp])) and np.all(go[emp] == 0.0)
    assert np.all(np.abs(go - ref_o) <= 2.0 ** -8 * np.abs(ref_o) + 1e-5)
    assert np.all(np.abs(gl[~emp] - ref_l[~emp]) <= 1e-4)


@pytest.mark.parametrize("nseg,n", [(1, 9), (3, 500), (16, 2048)])
def test_merge_segments_dense(nseg, n):
    from decode_context_parallelism_amd import ops
    o, l2 = random_segment_partials(nseg, n, seed=nseg * 100 + n)
    o_dev = torch.from_numpy(np.ascontiguousarray(o.transpose(1, 0, 2))).cuda()
    l_dev = torch.from_numpy(np.ascontiguousarray(l2.T)).cuda()
    out = torch.empty(n, 512, dtype=torch.bfloat16, device="cuda")
    lout = torch.empty(n, dtype=torch.float32, device="cuda")
    ops.merge_segments_dense(o_dev, l_dev, out, lout)
    torch.cuda.synchronize()
    ref_o, ref_l = A.merge_segments_base2(o.astype(np.float64), l2.astype(np.float64))
    go = out.float().cpu().numpy().astype(np.float64)
    gl = lout.cpu().numpy().astype(np.float64)
    emp = np.isneginf(ref_l)
    assert np.all(np.isneginf(gl[emp])) and np.all(go[emp] == 0.0)
    assert np.all(np.abs(go - ref_o) <= 2.0 ** -8 * np.abs(ref_o) + 1e-5)
    assert np.all(np.abs(gl[~emp] - ref_l[~emp]) <= 1e-4)
