#!/usr/bin/env python
"""Throughput of DCP MLA causal verification on one MI355X.

One step = the whole hot path for one batch, every DCP rank played in turn on
this GPU: verify-view metadata for each rank, each rank's segmented split-KV
attention and segment merge, then the cross-rank LSE merge.  Inputs (query,
per-rank KV pools, block tables, contexts) are resident in HBM before the
timed region; the KV pools are written once, untimed, by the library's
interleaved KV write.

Prints one JSON line.  ``value`` = KV tokens attended per second on this GPU
(every global cached token is read once per step, by its owner rank).
``roofline`` describes the dominant kernel (segmented attention), timed with
HIP events around each of its launches on the stream it runs on.
``cpu_baseline`` times the float64 oracle on a bounded sample of the same
workload (rank 0, first sequences) on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1..5]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense BF16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2,
                    help="workload 1..5 (default 2: dcp=2, qlen=3, 96 heads, batch 8, FP8 KV)")
    ap.add_argument("--groups", type=int, default=0,
                    help="persistent workgroups of the attention kernel (0: one per compute unit)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the oracle's timed CPU sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    return ap.parse_args()


def copy_calibration(mib):
    import torch
    n = mib * (1 << 20)
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 5}))


def cpu_baseline(w, seconds):
    """Time the float64 oracle on rank 0 of the same workload (a bounded sample)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention as A
    from oracle import formats, layout

    q = formats.decode_bf16(w.q_bits)
    lat = lambda b, pos: formats.decode_cache(w.kv[w.seq_start[b] + pos], w.kv_format, w.kv_scale)
    tokens = 0
    seqs = 0
    t0 = time.perf_counter()
    for b in range(w.batch):
        rows = [(b, i) for i in range(w.qlen)]
        A.verify_attention(q, lat, w.ctx_lens, w.softmax_scale, world=w.world,
                           interleave=w.interleave, rank=0, rows=rows)
        g_last = layout.verify_row_boundary(int(w.ctx_lens[b]), w.qlen, w.qlen - 1)
        tokens += layout.rank_local_positions(g_last, w.world, w.interleave, 0).shape[0]
        seqs += 1
        if time.perf_counter() - t0 > seconds:
            break
    dt = time.perf_counter() - t0
    threads = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    return {"value": tokens / dt, "unit": "KV tokens/s", "cores": int(max(threads) if threads else 1),
            "kind": "oracle",
            "sample": f"float64 oracle, rank 0 of {w.world}, sequences 0..{seqs - 1} of {w.batch}, "
                      f"all {w.qlen} verify rows x {w.heads} heads ({tokens} rank-local KV tokens, "
                      f"{dt:.1f} s)"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: every DCP rank is played in turn on a single MI355X; "
              "runs on more than one GPU are not part of this build", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import numpy as np
    import torch

    from decode_context_parallelism_amd import ops
    from decode_context_parallelism_amd.group import DcpGroup
    from synth import make_config

    torch.cuda.set_device(0)
    w = make_config(args.config)
    g = ops.Geometry(dcp_world=w.world, interleave=w.interleave, block_size=w.block_size,
                     qlen=w.qlen, num_heads=w.heads, batch=w.batch,
                     max_blocks_per_seq=w.block_table.shape[1], max_local_pages=w.max_local_pages,
                     kv_dtype=w.kv_format, num_blocks=w.num_blocks, groups=args.groups)
    dev = "cuda"
    q = torch.from_numpy(w.q_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    if w.kv_format == "fp8_e4m3":
        lat = torch.from_numpy(w.kv).to(dev)
    else:
        lat = torch.from_numpy(w.kv.view(np.int16)).view(torch.bfloat16).to(dev)
    seq_ids, positions = w.token_arrays()
    bt = torch.from_numpy(w.block_table).to(dev)
    ctx = torch.from_numpy(w.ctx_lens).to(dev)
    grp = DcpGroup(g, dev)
    grp.write_kv(torch.from_numpy(seq_ids).to(dev), torch.from_numpy(positions).to(dev), lat, bt)
    del lat
    torch.cuda.synchronize()

    W = w.world
    stream = torch.cuda.current_stream()

    def step(events=None):
        for r in range(W):
            ops.build_metadata(g, r, ctx, bt, grp.meta[r], stream)
        for r in range(W):
            if events is not None:
                events[r][0].record(stream)
            ops.partial_attention(g, q, grp.pools[r], w.kv_scale, w.softmax_scale, grp.meta[r],
                                  grp.workspace, grp.out_ranks[r], grp.lse_ranks[r], stream)
            if events is not None:
                events[r][1].record(stream)
            ops.merge_segments(g, grp.meta[r], grp.workspace, grp.out_ranks[r], grp.lse_ranks[r],
                               stream)
        ops.merge_ranks(grp.out_ranks, grp.lse_ranks, grp.out, grp.lse, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if grp.errors() != 0:
        raise RuntimeError(f"device error word {grp.errors():#x}")

    # algorithmic work per rank launch, from the verify view the kernels consume
    E = 1 if w.kv_format == "fp8_e4m3" else 2
    flops, kv_bytes = [], []
    for r in range(W):
        lens = grp.meta[r].row_local_len.cpu().numpy().astype(np.int64).reshape(w.batch, w.qlen)
        flops.append(2 * (576 + 512) * w.heads * int(lens.sum()))
        kv_bytes.append(int(lens.max(axis=1).sum()) * 576 * E)
    io_bytes = w.batch * w.qlen * w.heads * (576 * 2 + 512 * 2 + 4)

    events = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
               for _ in range(W)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kern_ms = [[events[k][r][0].elapsed_time(events[k][r][1]) for r in range(W)]
               for k in range(args.steps)]
    kern_total_ms = float(np.sum(kern_ms))
    launches = args.steps * W
    avg_kernel_ms = kern_total_ms / launches
    total_flops = args.steps * sum(flops)
    total_bytes = args.steps * (sum(kv_bytes) + W * io_bytes)
    tflops = total_flops / (kern_total_ms * 1e-3) / 1e12
    gbs = total_bytes / (kern_total_ms * 1e-3) / 1e9
    t_mfma = sum(flops) / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    t_hbm = (sum(kv_bytes) + W * io_bytes) / (HBM_PEAK_GBS * 1e9)
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": None}
    else:
        roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS, "traffic": None}
    roof.update({"kernel": "attention_kernel (segmented split-KV MLA, one rank)",
                 "avg_launch_ms": avg_kernel_ms, "launches": launches,
                 "algorithmic_flops_per_launch": sum(flops) / W,
                 "algorithmic_bytes_per_launch": (sum(kv_bytes) + W * io_bytes) / W,
                 "hbm_achieved_GBs": gbs})

    kv_tokens = int(w.ctx_lens.astype(np.int64).sum())
    value = kv_tokens / (ms_per_step * 1e-3)
    out = {
        "metric": "DCP-MLA verify: KV tokens/s per GPU and % of binding roofline (HBM or MFMA)",
        "value": value,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "dcp_world": W, "interleave": w.interleave,
                   "batch": w.batch, "qlen": w.qlen, "heads": w.heads,
                   "block_size": w.block_size, "kv_cache": w.kv_format,
                   "kv_tokens_per_step": kv_tokens, "ranks_per_step": W},
        "verify_rows_per_s": w.batch * w.qlen / (ms_per_step * 1e-3),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
