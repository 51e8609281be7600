#!/usr/bin/env python
"""Throughput of DCP MLA causal verification on one MI355X.

One step = one pass of the whole hot path over one batch, every DCP rank
played in turn on this GPU: the verify-view metadata of each rank (row
boundary, rank-local length, subpage table), each rank's segmented split-KV
attention and segment merge, then the cross-rank LSE merge.  Inputs (query,
per-rank KV pools, block table, contexts) are resident in HBM before the
timed region; the pools are written once, untimed, by the library's
interleaved KV write.  When the pools of all ranks together fit in the
256 MB Infinity Cache, the step rotates over enough copies of the inputs
that every step reads its KV from HBM.

Prints one JSON line:
  value       global KV tokens attended per second (every cached token of
              every sequence is read once per step, by its owner rank)
  roofline    the dominant kernel (segmented attention), timed with HIP
              events around each launch on the stream it runs on, against
              the binding published MI355X peak (BF16 MFMA or HBM); traffic
              = HBM bytes per launch from the rocprofv3 counter summary under
              profiles/ when that summary was taken from the current kernel
              source, else null
  cpu_baseline  the float64 oracle timed on this host over a bounded sample
              of the same workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1..5]
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# published MI355X peaks (dense)
PEAK_HBM_GBS = 8000.0
PEAK_MFMA_BF16_TFLOPS = 2500.0
PEAK_MFMA_FP8_TFLOPS = 5000.0
# flops per clock per CU of dense BF16 MFMA on gfx950 (4 SIMDs x 1024)
BF16_FLOPS_PER_CLK_CU = 4096
# the chip's peak engine clock
MAX_CLOCK_GHZ = 2.4
INFINITY_CACHE_BYTES = 256 << 20
# sources that fix the attention kernel's code and work partition: the counter
# summaries under profiles/ record their digest
KERNEL_SOURCES = [os.path.join(ROOT, "decode_context_parallelism_amd", "csrc", f)
                  for f in ("attention.hip", "attention_fp8.hip", "attention_common.h", "common.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5,
                    help="workload 1..5 (default 5, the largest: dcp=8, 1,048,576-token contexts, "
                         "batch 4, qlen 3, 128 heads, FP8 KV)")
    ap.add_argument("--groups", type=int, default=0,
                    help="persistent workgroups of the attention kernel (0: one per compute unit)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target length of the oracle's timed CPU sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--q-format", choices=("split", "fp8"), default="split",
                    help="FP8 cache: the exact two-term split of the BF16 query (default) or the "
                         "quantised FP8 query variant")
    ap.add_argument("--p-format", choices=("split", "fp8"), default="split",
                    help="FP8 cache: probabilities as two FP8 terms (E4M3 + E5M2 remainder, default) or "
                         "one E4M3 term against a per-stage power-of-two scale")
    ap.add_argument("--row-boundary", choices=("causal", "block"), default="causal",
                    help="causal verify rows (default) or a bidirectional draft block "
                         "(every row sees the whole cache)")
    ap.add_argument("--merge", choices=("direct", "a2a", "pbm"), default="direct",
                    help="cross-rank combine: direct LSE merge of all partials (default); a2a pack, "
                         "exchange and local combine; or pbm (project each partial through a "
                         "synthetic W_V [H, 512 -> 128] before the a2a)")
    ap.add_argument("--streams", type=int, choices=(1, 2), default=2,
                    help="streams of the replayed step: 2 issues the query split and the odd ranks on a "
                         "second stream, each stream with its own split-KV workspace, so independent "
                         "launches overlap (default); 1 issues everything in order on one stream")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of replaying the step as a captured HIP graph")
    ap.add_argument("--no-rotate", action="store_true",
                    help="reuse one input set every step (cache-warm KV)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    return ap.parse_args()


def dtype_name(kv_format, q_format, p_format):
    """Arithmetic type of the attention products: "bf16" where each runs as
    BF16 or as two FP8 terms carrying BF16's precision, "fp8e4m3" where both
    take one FP8 term, "fp8e4m3+bf16" where one does."""
    if kv_format != "fp8_e4m3":
        return "bf16"
    n = (q_format == "fp8") + (p_format == "fp8")
    return ("bf16", "fp8e4m3+bf16", "fp8e4m3")[n]


def dtype_detail(kv_format, q_format, p_format):
    if kv_format != "fp8_e4m3":
        return "BF16 cache: q.k and p.v on the BF16 units, fp32 accumulation"
    qk = ("q.k on the FP8 units as two E4M3 terms that sum exactly to the BF16 query"
          if q_format == "split" else "q.k with the per-row E4M3-quantised query on the FP8 units")
    pv = ("p.v on the FP8 units with the probabilities as an E4M3 term plus its E5M2 remainder"
          if p_format == "split" else
          "p.v with E4M3 probabilities against a per-stage power-of-two scale on the FP8 units")
    return f"{qk}; {pv}; fp32 accumulation"


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


def code_only(text):
    """C/C++ source without its comments, whitespace runs collapsed: edits to comments or layout
    leave it unchanged, edits to code do not."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_digest():
    """sha256 over the code (not the comments) of the attention kernel's sources."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, encoding="utf-8") as f:
            h.update(os.path.basename(path).encode() + b"\0" + code_only(f.read()).encode())
    return h.hexdigest()


def read_traffic(workload, digest):
    """HBM bytes per attention launch from the committed counter summary, or None."""
    kv, src = read_summary(os.path.join(ROOT, "profiles", f"attention_kernel_{workload}_hbm.md"), digest)
    if kv is None:
        return None, src
    try:
        fetch = float(kv["fetch_kib_per_launch"]) * 1024 * float(kv["fetch_scale"])
        write = float(kv["write_kib_per_launch"]) * 1024 * float(kv["write_scale"])
    except KeyError:
        return None, "counter summary incomplete"
    return fetch + write, src


def read_summary(path, digest):
    """key: value lines of a committed counter summary, or (None, reason)."""
    if not os.path.exists(path):
        return None, "no counter summary"
    kv = {}
    for line in open(path):
        m = re.match(r"^\s*[-*]?\s*`?([a-z_0-9]+)`?\s*[:=]\s*`?([0-9a-fA-F.e+-]+)`?\s*$", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("kernel_source_sha256") != digest:
        return None, "kernel changed since the counters were taken"
    return kv, os.path.relpath(path, ROOT)


def read_mfma_busy(workload, digest):
    """Matrix-unit busy share and clock of the attention launch from the
    committed counter summary (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE),
    or None."""
    kv, src = read_summary(os.path.join(ROOT, "profiles", f"attention_kernel_{workload}_mfma.md"), digest)
    if kv is None:
        return None, src
    try:
        busy = {"mfma_busy_frac": float(kv["mfma_busy_frac"]), "clock_ghz": float(kv["clock_ghz"])}
    except KeyError:
        return None, "counter summary incomplete"
    if "mfma_busy_frac_at_2_4_ghz" in kv:
        busy["mfma_busy_frac_at_2_4_ghz"] = float(kv["mfma_busy_frac_at_2_4_ghz"])
    if busy["clock_ghz"] > MAX_CLOCK_GHZ:
        # the GPU-active counter's window outlasts a launch of a few tens of
        # microseconds, so a clock above the chip's peak marks both figures
        # derived from it as unusable; the busy share at the peak clock
        # divides by the launch's own duration and stands
        busy["clock_ghz"] = busy["mfma_busy_frac"] = None
        busy["note"] = (f"counted clock {float(kv['clock_ghz']):.3f} GHz exceeds the chip's "
                        f"{MAX_CLOCK_GHZ} GHz: launch shorter than the counter window")
    busy["source"] = src
    return busy, src


def host_cpu():
    """Host cores this process may run on, the machine's count, and the CPU model."""
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return usable, os.cpu_count() or usable, model


def cpu_baseline(w, seconds):
    """Time the float64 oracle on this host, as it stands: verify rows taken in
    order (sequence-major), each computed twice -- global causal attention over
    the whole visible prefix, and the per-rank split (every rank's partial
    over the positions it owns) plus the LSE merge -- until the time budget is
    spent (at least one row).  A row is credited ctx/qlen of its sequence's KV
    tokens, so the rates are in the metric's unit: global KV tokens of a full
    step per second."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention as A
    from oracle import formats

    q = formats.decode_bf16(w.q_bits)
    lat = lambda b, pos: formats.decode_cache(w.kv[w.seq_start[b] + pos], w.kv_format, w.kv_scale)
    t_glob = t_split = 0.0
    credited = 0.0
    done = []
    for b in range(w.batch):
        for i in range(w.qlen):
            rows = [(b, i)]
            t0 = time.perf_counter()
            A.verify_attention(q, lat, w.ctx_lens, w.softmax_scale, rows=rows)
            t1 = time.perf_counter()
            parts = [A.verify_attention(q, lat, w.ctx_lens, w.softmax_scale, world=w.world,
                                        interleave=w.interleave, rank=r, rows=rows)
                     for r in range(w.world)]
            A.merge_ranks(np.stack([p[0][b, i] for p in parts]), np.stack([p[1][b, i] for p in parts]))
            t2 = time.perf_counter()
            t_glob += t1 - t0
            t_split += t2 - t1
            credited += float(w.ctx_lens[b]) / w.qlen
            done.append((b, i))
            if t_glob + t_split > seconds:
                break
        if t_glob + t_split > seconds:
            break
    threads = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    usable, machine, model = host_cpu()
    return {"value": credited / t_split, "unit": "KV tokens/s",
            "cores": int(max(threads) if threads else 1), "kind": "oracle",
            "host_cores_usable": usable, "host_cores_machine": machine, "cpu_model": model,
            "global_attention": {"value": credited / t_glob, "unit": "KV tokens/s", "seconds": t_glob},
            "split_and_merge": {"value": credited / t_split, "unit": "KV tokens/s", "seconds": t_split},
            "sample": f"float64 oracle (numpy, BLAS threads = cores), {len(done)} verify row(s) of "
                      f"{w.name} taken in order from (sequence {done[0][0]}, row {done[0][1]}), all "
                      f"{w.heads} heads each: global causal attention {t_glob:.1f} s, the {w.world} ranks' "
                      f"partials plus the LSE merge {t_split:.1f} s; each row credited ctx/qlen KV tokens; "
                      f"value = the split-and-merge rate"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: every DCP rank is played in turn on a single MI355X; "
              "--gpus above 1 is not supported", file=sys.stderr)
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
    dev_info = ops.device_info(0)
    w = make_config(args.config)
    if w.kv_format != "fp8_e4m3" and (args.q_format == "fp8" or args.p_format == "fp8"):
        print(f"--q-format fp8 and --p-format fp8 need an FP8 cache; {w.name} holds {w.kv_format}",
              file=sys.stderr)
        sys.exit(2)
    g = ops.Geometry(dcp_world=w.world, interleave=w.interleave, block_size=w.block_size,
                     qlen=w.qlen, num_heads=w.heads, batch=w.batch,
                     max_blocks_per_seq=w.block_table.shape[1], max_local_pages=w.max_local_pages,
                     kv_dtype=w.kv_format, num_blocks=w.num_blocks, groups=args.groups,
                     row_boundary=args.row_boundary, q_format=args.q_format, p_format=args.p_format)
    dev = "cuda"
    q0 = torch.from_numpy(w.q_bits.view(np.int16)).view(torch.bfloat16).to(dev)
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
    if grp.errors() != 0:
        raise RuntimeError(f"device error word {grp.errors():#x} after the KV write")

    # input sets: the step reads set k % n_sets, so the KV of a step is not
    # left in the Infinity Cache by the previous one
    W = w.world
    pool_bytes = sum(p.numel() * p.element_size() for p in grp.pools)
    n_sets = 1 if args.no_rotate else min(16, max(1, math.ceil(2 * INFINITY_CACHE_BYTES / pool_bytes)))
    sets = [(grp.pools, q0)]
    for _ in range(n_sets - 1):
        sets.append(([p.clone() for p in grp.pools], q0.clone()))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    # exchange buffers for the a2a / pbm combines: the all-to-all between
    # ranks is one transposing copy here (block p of rank r -> block r of p)
    T, H = w.batch * w.qlen, w.heads
    Hl = H // W
    if args.merge != "direct":
        D = 128 if args.merge == "pbm" else 512
        msg = ops.a2a_message_elems(D)
        send = torch.empty(W, W, T, Hl, msg, dtype=torch.bfloat16, device=dev)
        recv = torch.empty_like(send)
        comb_o = torch.empty(W, T, Hl, D, dtype=torch.bfloat16, device=dev)
        comb_l = torch.empty(W, T, Hl, dtype=torch.float32, device=dev)
        if args.merge == "pbm":
            gw = torch.Generator().manual_seed(7)
            wvt = (torch.randn(H, D, 512, generator=gw) / 512 ** 0.5).to(torch.bfloat16).to(dev)
            proj = torch.empty(W, T, H, D, dtype=torch.bfloat16, device=dev)

    def combine():
        stream = torch.cuda.current_stream()
        if args.merge == "direct":
            ops.merge_ranks(grp.out_ranks, grp.lse_ranks, grp.out, grp.lse, stream)
            return
        for r in range(W):
            src = grp.out_ranks[r].view(T, H, 512)
            if args.merge == "pbm":
                ops.project_heads(src, wvt, proj[r], stream)
                src = proj[r]
            ops.a2a_pack(W, src, grp.lse_ranks[r].view(T, H), send[r], stream)
        recv.copy_(send.transpose(0, 1))
        for p in range(W):
            ops.a2a_combine(recv[p], comb_o[p], comb_l[p], stream)

    def attention_launches(k):
        stream = torch.cuda.current_stream()
        pools, q = sets[k % n_sets]
        for r in range(W):
            if grp.q_split is not None:
                ops.partial_attention_split(g, grp.q_split, grp.q_scale, pools[r], w.kv_scale,
                                            w.softmax_scale, grp.meta[r], grp.workspace,
                                            grp.out_ranks[r], grp.lse_ranks[r], stream)
            else:
                ops.partial_attention(g, q, pools[r], w.kv_scale, w.softmax_scale, grp.meta[r],
                                      grp.workspace, grp.out_ranks[r], grp.lse_ranks[r], stream)

    def step(k, events=None):
        # launches go to the current stream (a capture stream while a graph is recorded)
        stream = torch.cuda.current_stream()
        pools, q = sets[k % n_sets]
        for r in range(W):
            ops.build_metadata(g, r, ctx, bt, grp.meta[r], stream)
        if grp.q_split is not None:
            # once per forward: each rank splits its own head slice before the query gather
            ops.split_q(q, grp.q_split, grp.q_scale, stream)
        for r in range(W):
            if events is not None:
                events[r][0].record(stream)
            if grp.q_split is not None:
                ops.partial_attention_split(g, grp.q_split, grp.q_scale, pools[r], w.kv_scale,
                                            w.softmax_scale, grp.meta[r], grp.workspace,
                                            grp.out_ranks[r], grp.lse_ranks[r], stream)
            else:
                ops.partial_attention(g, q, pools[r], w.kv_scale, w.softmax_scale, grp.meta[r],
                                      grp.workspace, grp.out_ranks[r], grp.lse_ranks[r], stream)
            if events is not None:
                events[r][1].record(stream)
            ops.merge_segments(g, grp.meta[r], grp.workspace, grp.out_ranks[r], grp.lse_ranks[r],
                               stream)
            if events is not None:
                events[r][2].record(stream)
        combine()

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    if grp.errors() != 0:
        raise RuntimeError(f"device error word {grp.errors():#x}")

    # algorithmic work of each rank's attention launch, from the verify view
    E = 1 if w.kv_format == "fp8_e4m3" else 2
    flops, kv_bytes, lmax_tokens = [], [], []
    for r in range(W):
        lens = grp.meta[r].row_local_len.cpu().numpy().astype(np.int64).reshape(w.batch, w.qlen)
        flops.append(2 * (576 + 512) * w.heads * int(lens.sum()))
        lmax_tokens.append(int(lens.max(axis=1).sum()))
        kv_bytes.append(lmax_tokens[-1] * 576 * E)
    io_bytes = w.batch * w.qlen * w.heads * (576 * 2 + 512 * 2 + 4) + w.batch * w.qlen * 4
    alg_bytes = [kb + io_bytes for kb in kv_bytes]

    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(W)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(args.warmup + k, events[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if grp.errors() != 0:
        raise RuntimeError(f"device error word {grp.errors():#x}")

    ms_per_step_eager = (t1 - t0) * 1e3 / args.steps
    ms_per_step = ms_per_step_eager
    step_mode = "eager launches"
    if not args.no_graph:
        # The same steps replayed as captured HIP graphs (one per input set):
        # the work is identical, the host launch overhead between the short
        # kernels is gone.  The per-launch kernel durations above come from
        # the eager pass.
        side = torch.cuda.Stream()

        def step_replayed(k):
            if args.streams == 1:
                step(k)
                return
            pools, q = sets[k % n_sets]
            grp.ranks_two_streams(q, ctx, bt, w.kv_scale, w.softmax_scale, side, pools=pools)
            combine()

        graphs = []
        for i in range(n_sets):
            gph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gph):
                step_replayed(i)
            graphs.append(gph)
        for k in range(args.warmup):
            graphs[k % n_sets].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            graphs[(args.warmup + k) % n_sets].replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        if grp.errors() != 0:
            raise RuntimeError(f"device error word {grp.errors():#x}")
        ms_per_step = (t1 - t0) * 1e3 / args.steps
        step_mode = ("HIP graph replay (one captured graph per input set); " +
                     ("two streams: the query split and the odd ranks on the second, each stream "
                      "with its own split-KV workspace" if args.streams == 2 else "one stream"))
    attn_ms = np.array([[events[k][r][0].elapsed_time(events[k][r][1]) for r in range(W)]
                        for k in range(args.steps)])
    attn_merge_ms = np.array([[events[k][r][0].elapsed_time(events[k][r][2]) for r in range(W)]
                              for k in range(args.steps)])
    avg_launch_ms = float(attn_ms.mean())
    per_rank_ms = attn_ms.mean(axis=0)
    attn_timing = "HIP events around each eager launch"
    if not args.no_graph:
        # The roofline's launch duration: every rank's attention launch of a
        # step captured back to back in one graph per input set, K replays
        # bracketed by HIP events on the stream -- no host launch gap can
        # stretch it (as the eager events can under a slow host).
        attn_graphs = []
        for i in range(n_sets):
            gph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gph):
                attention_launches(i)
            attn_graphs.append(gph)
        for k in range(args.warmup):
            attn_graphs[k % n_sets].replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for k in range(args.steps):
            attn_graphs[(args.warmup + k) % n_sets].replay()
        e1.record()
        torch.cuda.synchronize()
        avg_launch_ms = e0.elapsed_time(e1) / (args.steps * W)
        # per-rank shares as measured by the eager events, scaled to this total
        per_rank_ms = per_rank_ms * (avg_launch_ms * W / float(per_rank_ms.sum()))
        attn_timing = ("HIP events around K replays of a graph of every rank's attention launch, "
                       "back to back; per-rank split from the eager pass")

    # roofline of the attention kernel against the published peaks.  With an
    # FP8 cache the default path runs q.k and p.v each as two FP8 products
    # (the query, and the probabilities, split into two FP8 terms): twice the
    # flops at twice the rate, so its MFMA time is that of an all-BF16 kernel
    # and the BF16 peak is the roofline.  The FP8-query variant runs q.k once
    # at the FP8 rate, the FP8-probability variant p.v; the roofline of a
    # product taken once is the FP8 peak, and of the kernel the time-weighted
    # mix of its two products' peaks.
    fp8_cache = w.kv_format == "fp8_e4m3"
    peak_qk = PEAK_MFMA_FP8_TFLOPS if fp8_cache and args.q_format == "fp8" else PEAK_MFMA_BF16_TFLOPS
    peak_pv = PEAK_MFMA_FP8_TFLOPS if fp8_cache and args.p_format == "fp8" else PEAK_MFMA_BF16_TFLOPS
    f_qk = sum(flops) * 576.0 / (576 + 512)
    f_pv = sum(flops) - f_qk
    peak_mfma = sum(flops) / (f_qk / peak_qk + f_pv / peak_pv)
    t_mfma = sum(flops) / (peak_mfma * 1e12)
    t_hbm = sum(alg_bytes) / (PEAK_HBM_GBS * 1e9)
    tflops = sum(flops) / (float(per_rank_ms.sum()) * 1e-3) / 1e12
    gbs = sum(alg_bytes) / (float(per_rank_ms.sum()) * 1e-3) / 1e9
    digest = source_digest()
    variant = ("fp8_query_" if args.q_format == "fp8" else "") + ("fp8_p_" if args.p_format == "fp8" else "")
    traffic, traffic_src = read_traffic(variant + w.name, digest)
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": tflops, "peak": peak_mfma, "unit": "TFLOP/s",
                "frac": tflops / peak_mfma}
    else:
        roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": gbs / PEAK_HBM_GBS}
    roof["traffic"] = traffic
    roof.update({
        "kernel": (("attention_fp8_kernel" if fp8_cache else "attention_kernel") +
                   " (segmented split-KV MLA, one rank per launch)"),
        "peak_qk_tflops": peak_qk, "peak_pv_tflops": peak_pv,
        "avg_launch_ms": avg_launch_ms, "launches": int(attn_ms.size), "launch_timing": attn_timing,
        "algorithmic_flops_per_launch": sum(flops) / W,
        "algorithmic_bytes_per_launch": sum(alg_bytes) / W,
        "algorithmic_hbm_GBs": gbs,
        "traffic_source": traffic_src,
        "kernel_source_sha256": digest,
    })
    # the matrix units' measured busy share of the launch, at the clock they ran
    busy, busy_src = read_mfma_busy(variant + w.name, digest)
    roof["mfma_busy_counters"] = busy if busy is not None else busy_src

    clk_ghz = dev_info["clock_khz"] / 1e6
    device = dict(dev_info)
    device["mfma_bf16_peak_tflops_from_clock"] = (dev_info["compute_units"] * clk_ghz * 1e9 *
                                                  BF16_FLOPS_PER_CLK_CU / 1e12)
    device["peaks_used"] = {"mfma_bf16_tflops": PEAK_MFMA_BF16_TFLOPS, "mfma_fp8_tflops": PEAK_MFMA_FP8_TFLOPS,
                            "hbm_gbs": PEAK_HBM_GBS,
                            "source": "published MI355X figures"}

    kv_tokens = int(w.ctx_lens.astype(np.int64).sum())
    out = {
        "metric": "DCP-MLA verify: KV tokens/s per GPU and % of binding roofline (HBM or MFMA)",
        "value": kv_tokens / (ms_per_step * 1e-3),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_name(w.kv_format, args.q_format, args.p_format),
        "dtype_detail": dtype_detail(w.kv_format, args.q_format, args.p_format),
        "data": "synthetic",
        "config": {"workload": w.name, "dcp_world": W, "interleave": w.interleave,
                   "batch": w.batch, "qlen": w.qlen, "heads": w.heads,
                   "block_size": w.block_size, "kv_cache": w.kv_format,
                   "kv_tokens_per_step": kv_tokens, "ranks_per_step": W, "input_sets": n_sets,
                   "row_boundary": args.row_boundary, "merge": args.merge, "q_format": args.q_format,
                   "p_format": args.p_format,
                   "streams": 1 if args.no_graph else args.streams},
        "verify_rows_per_s": w.batch * w.qlen / (ms_per_step * 1e-3),
        "step_mode": step_mode,
        "ms_per_step_eager": ms_per_step_eager,
        "per_rank": {
            "attention_us_mean": float(per_rank_ms.mean() * 1e3),
            "attention_us_max": float(per_rank_ms.max() * 1e3),
            "attention_plus_segment_merge_us_mean": float(attn_merge_ms.mean(axis=0).mean() * 1e3),
            "attention_plus_segment_merge_us_max": float(attn_merge_ms.mean(axis=0).max() * 1e3),
            "local_kv_tokens_per_s": float(np.mean([lmax_tokens[r] / (per_rank_ms[r] * 1e-3)
                                                    for r in range(W)])),
        },
        "roofline": roof,
        "device": device,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
