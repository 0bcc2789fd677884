#!/usr/bin/env python3
"""Benchmark of split-KV decode attention on one MI355X.

One step = one whole pass of the method over one batch: the per-tile partial
kernel and the merge kernel (``fd_decode_attention``), on inputs already
resident in HBM.  The default workload is the 32k-context GQA decode layer
(batch 1, 32 query heads, 8 KV heads, head_dim 128, bf16, planner splits).

Timing: W untimed eager warm-up steps; then a HIP graph of G consecutive steps
is captured (so host launch overhead is not measured) and replayed once
untimed; the timed region is exactly K steps, K / G replays of that graph,
bracketed by synchronisations and events on the stream the kernels run on,
with an event between replays as well.  Each replay gives one sample of the
time per step (its time / G); the reported time per step is the median of
those samples (the mean over the whole region is printed beside it).  The K/V
caches rotate over several identical copies (>= 1 GiB in total) so that the
256 MB last-level cache cannot hold them and every step reads HBM.

``--kv-fp8`` / ``--kv-int8`` quantise K and V to FP8 E4M3 or INT8 codes with
per-tensor scales (bf16 queries and output).  ``--page-size P`` runs the same workload on a paged cache (pages of P keys in
a shuffled pool, read in place through the block table; ``--page-layout``
picks [pages, P, Hkv, D] or [pages, Hkv, P, D]).

Printed: one JSON line with the metric (algorithmic GB/s per step: the bytes
any implementation must move -- K, V, q, out, lse -- over the step time), the
roofline of the dominant kernel (the partial pass, timed per launch over a
graph of back-to-back launches), the rate of a plain streaming read of the
same number of bytes (the library's read kernel, best of a few grid sizes:
the bandwidth this device reaches with no arithmetic at all), and the fp64
CPU oracle's rate on a bounded sample of the same workload as a reference
point.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attention HBM GB/s (% of MI355X peak) and µs/step at 32k ctx"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak of MI355X
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "decode_attention_14_amd", "csrc")
# The sources that decide each partial-pass kernel's machine code (its own
# file, the headers it includes, and the build flags).
_COMMON_SOURCES = [os.path.join(CSRC, "fd_device.h"), os.path.join(CSRC, "fd_internal.h"),
                   os.path.join(ROOT, "decode_attention_14_amd", "build.py")]
KERNEL_SOURCES = {
    "fd_partial_kernel": [os.path.join(CSRC, "fd_decode.hip")],
    "fd_mfma_partial_kernel": [os.path.join(CSRC, "fd_mfma.hip"), os.path.join(CSRC, "fd_mfma_common.h")],
    "fd_mfma_chunk_kernel": [os.path.join(CSRC, "fd_chunk.hip"), os.path.join(CSRC, "fd_mfma_common.h")],
}


def kernel_source_hash(kernel: str) -> str:
    """Hash of one kernel's sources and the build flags; counter data taken
    for that kernel is tied to it."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kernel] + _COMMON_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--graph-steps", type=int, default=10,
                    help="steps per captured graph; each replay is one timing sample")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gqa_32k")
    ap.add_argument("--num-splits", type=int, default=0, help="force a split count (0: planner)")
    ap.add_argument("--tile-len", type=int, default=0, help="override the planner's tile length")
    ap.add_argument("--spans", type=int, default=-1,
                    help="force N balanced spans (0: tiles; -1: the planner's choice)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle time")
    ap.add_argument("--page-size", type=int, default=0,
                    help="read K/V from a paged cache with pages of this many keys (0: contiguous)")
    ap.add_argument("--page-layout", default="nhd", choices=["nhd", "hnd"])
    ap.add_argument("--kv-int8", action="store_true",
                    help="INT8 K/V caches (symmetric per-tensor scales) with bf16 queries")
    ap.add_argument("--kv-fp8", action="store_true",
                    help="FP8 E4M3 K/V caches (per-tensor scales) with bf16 queries")
    ap.add_argument("--calibrate-copy", type=int, default=0,
                    help="also run N plain 512 MiB device copies (counter calibration)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read ceiling")
    return ap.parse_args()


def algorithmic_bytes(w, lens, kv_codes=False):
    """Bytes any implementation must move: visible K and V rows, q, out, lse."""
    el = 2 if w.dtype == "bf16" else 4
    kv = 2 * sum(lens) * w.num_kv_heads * w.head_dim * (1 if kv_codes else el)
    q = w.batch * w.num_q_heads * w.q_len * w.head_dim * el
    return kv, q, q, w.batch * w.num_q_heads * w.q_len * 4


def partial_kernel_name(w) -> str:
    """The partial-pass kernel the library dispatches to for this workload:
    matrix cores for bf16 (decode rows, or chunk tiles above 32 rows), vector
    ALUs for fp32 or when FD_DECODE_KERNEL=vector forces them."""
    rows = w.num_q_heads // w.num_kv_heads * w.q_len
    if w.dtype != "bf16" or os.environ.get("FD_DECODE_KERNEL") == "vector":
        return "fd_partial_kernel"
    return "fd_mfma_partial_kernel" if rows <= 32 else "fd_mfma_chunk_kernel"


def algorithmic_flops(w, lens):
    """4 * head_dim flops (the q.k and p.v products) per visible (query row,
    key) pair; row t of a chunk sees keys 0 .. L - q_len + t."""
    pairs = 0
    for L in lens:
        for t in range(w.q_len):
            pairs += max(0, min(L, L - w.q_len + t + 1))
    return 4 * w.head_dim * w.num_q_heads * pairs


def host_description():
    """CPU count and model of the host the oracle runs on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"host_cpus": os.cpu_count(), "usable_cpus": usable, "cpu_model": model}


def cpu_baseline(w, q, k, v, cl, alg_bytes, seconds):
    import oracle
    from decode_attention_14_amd.inputs import as_oracle_array

    host = host_description()
    # at most 16 threads: the share of host cores a one-GPU job gets
    threads = max(1, min(16, host["usable_cpus"]))
    qa, ka, va, la = as_oracle_array(q), as_oracle_array(k), as_oracle_array(v), cl.numpy()
    oracle.load()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.attention(qa, ka, va, la, w.scale, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    return {
        "value": round(alg_bytes * reps / el / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{reps} full step(s) of {w.name} in fp64 ({el:.1f} s) on {threads} threads",
        **host,
    }


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU sequence split is a design, not part of this build)", file=sys.stderr)
        sys.exit(2)

    import torch

    from decode_attention_14_amd import binding as fd
    from decode_attention_14_amd.inputs import (WORKLOADS, fp8_scale_for, int8_scale_for, paginate, quantize_fp8,
                                                quantize_int8, workload_inputs)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fd.load_library()
    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    q, k, v, cl = workload_inputs(w)
    lens = cl.tolist()
    if args.kv_fp8 and args.kv_int8:
        print("--kv-fp8 and --kv-int8 exclude each other", file=sys.stderr)
        sys.exit(2)
    codes = "fp8" if args.kv_fp8 else "int8" if args.kv_int8 else None  # one-byte K/V codes
    coded = codes is not None
    if coded:
        if w.dtype != "bf16":
            print(f"--kv-{codes} needs a bf16 workload", file=sys.stderr)
            sys.exit(2)
        scale_for, quantize = (fp8_scale_for, quantize_fp8) if codes == "fp8" else (int8_scale_for, quantize_int8)
        k_scale, v_scale = scale_for(k), scale_for(v)
        k, v = quantize(k, k_scale), quantize(v, v_scale)
        attn_codes = fd.decode_attention_fp8 if codes == "fp8" else fd.decode_attention_int8
        partials_codes = fd.decode_partials_fp8 if codes == "fp8" else fd.decode_partials_int8
    kv_b, q_b, out_b, lse_b = algorithmic_bytes(w, lens, coded)
    step_bytes = kv_b + q_b + out_b + lse_b
    partial_bytes = kv_b + q_b

    plan = fd.plan_splits(fd.make_dims(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.q_len,
                                       w.max_cache_len, q.dtype), cl, num_splits=args.num_splits)
    if args.tile_len:
        plan = fd.Plan(fd.FdPlan(args.tile_len, max(1, -(-max(lens) // args.tile_len))), [])
    if args.spans >= 0:
        if args.num_splits:
            raise SystemExit("bench.py: --spans and --num-splits do not combine")
        slots = plan.max_splits
        if args.spans:
            # the slots a pair needs when the line of 16-key blocks (each pair
            # with keys preceded by 16 positions) is cut into args.spans spans
            nb = [-(-max(0, min(L, w.max_cache_len)) // 16) for L in lens]
            line = sum(w.num_kv_heads * (16 + n) for n in nb if n)
            per = max(1, -(-line // args.spans))
            slots = min(fd.FD_MAX_SPLITS, max(slots, -(-max(nb) // per) + 1))
        plan = fd.Plan(fd.FdPlan(tile_len=plan.tile_len, max_splits=slots, spans=args.spans), plan.splits_per_seq)
    num_splits = args.num_splits
    slots = num_splits if num_splits else plan.max_splits

    paged = args.page_size > 0
    table = None
    if paged:
        print(f"[bench] paging the cache: {args.page_size}-key pages, {args.page_layout}", file=sys.stderr,
              flush=True)
        pc = paginate(k, v, cl, args.page_size, args.page_layout, seed=w.seed)
        k, v, table = pc.k_pages, pc.v_pages, pc.block_table.to(dev)
    copies = int(min(8, max(2, math.ceil((1 << 30) / max(1, 2 * k.numel() * k.element_size())))))
    qd, cld = q.to(dev), cl.to(dev)
    kd0, vd0 = k.to(dev), v.to(dev)
    kvs = [(kd0, vd0)] + [(kd0.clone(), vd0.clone()) for _ in range(copies - 1)]
    del q, k, v
    out = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
    dims = fd.paged_dims(qd, kd0, table, args.page_layout)[0] if paged else fd.dims_of(qd, kd0)
    dims.dtype = fd.FD_BF16 if w.dtype == "bf16" else fd.FD_F32
    ws_bytes = fd.workspace_bytes(dims, slots) if slots > 1 else 0
    ws = fd.new_workspace(ws_bytes, dev)
    o_part = torch.empty(*qd.shape[:3], slots, w.head_dim, dtype=torch.float32, device=dev)
    m_part = torch.empty(*qd.shape[:3], slots, dtype=torch.float32, device=dev)
    l_part = torch.empty_like(m_part)
    fplan = plan.plan if not num_splits else None

    def step(i):
        kd, vd = kvs[i % copies]
        if coded:
            attn_codes(qd, kd, vd, cld, k_scale, v_scale, block_table=table, layout=args.page_layout,
                                    scale=w.scale, num_splits=num_splits, plan=fplan, out=out, lse=lse,
                                    workspace=ws if ws_bytes else None)
        elif paged:
            fd.decode_attention_paged(qd, kd, vd, table, cld, layout=args.page_layout, scale=w.scale,
                                      num_splits=num_splits, plan=fplan, out=out, lse=lse,
                                      workspace=ws if ws_bytes else None)
        else:
            fd.decode_attention(qd, kd, vd, cld, scale=w.scale, num_splits=num_splits, plan=fplan,
                                out=out, lse=lse, workspace=ws if ws_bytes else None)

    def partial(i):
        kd, vd = kvs[i % copies]
        if coded and slots > 1:
            partials_codes(qd, kd, vd, cld, k_scale, v_scale, block_table=table, layout=args.page_layout,
                                   scale=w.scale, num_splits=num_splits, plan=fplan, o_part=o_part,
                                   m_part=m_part, lse_part=l_part)
        elif coded:
            attn_codes(qd, kd, vd, cld, k_scale, v_scale, block_table=table, layout=args.page_layout,
                                    scale=w.scale, out=out, lse=lse)
        elif paged and slots > 1:
            fd.decode_partials_paged(qd, kd, vd, table, cld, layout=args.page_layout, scale=w.scale,
                                     num_splits=num_splits, plan=fplan, o_part=o_part, m_part=m_part,
                                     lse_part=l_part)
        elif paged:
            fd.decode_attention_paged(qd, kd, vd, table, cld, layout=args.page_layout, scale=w.scale,
                                      out=out, lse=lse)
        elif slots > 1:
            fd.decode_partials(qd, kd, vd, cld, scale=w.scale, num_splits=num_splits, plan=fplan,
                               o_part=o_part, m_part=m_part, lse_part=l_part)
        else:
            fd.decode_attention(qd, kd, vd, cld, scale=w.scale, out=out, lse=lse)

    def combine(i):
        fd.combine(o_part, l_part, out_dtype=out.dtype, out=out, lse=lse)

    stream = torch.cuda.current_stream(dev)

    def graph_of(fn, n):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(n):
                fn(i)
        return graph

    def timed(fn, n):
        """Average ms per call of fn(0..n-1): one untimed pass, then one timed
        pass, as a graph replay unless --no-graph."""
        graph = None if args.no_graph else graph_of(fn, n)
        run = graph.replay if graph is not None else (lambda: [fn(i) for i in range(n)])
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def timed_samples(fn, total, per):
        """Exactly `total` calls of fn, as total / per replays of a graph of
        `per` calls (eager calls with --no-graph), an event after each
        replay.  Returns (per-call ms of each replay, mean ms over all)."""
        reps = max(1, total // per)
        graph = None if args.no_graph else graph_of(fn, per)
        run = graph.replay if graph is not None else (lambda: [fn(i) for i in range(per)])
        run()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for r in range(reps):
            run()
            ev[r + 1].record(stream)
        torch.cuda.synchronize()
        samples = [ev[r].elapsed_time(ev[r + 1]) / per for r in range(reps)]
        return samples, ev[0].elapsed_time(ev[reps]) / (reps * per)

    per = max(1, min(args.graph_steps, args.steps))
    if args.steps % per:
        print(f"--steps {args.steps} is not a multiple of --graph-steps {per}", file=sys.stderr)
        sys.exit(2)
    print(f"[bench] plan {plan.plan} copies={copies} warmup={args.warmup} steps={args.steps} "
          f"graph={not args.no_graph} ({per} steps per replay)", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    samples, ms_mean = timed_samples(step, args.steps, per)
    wall = time.perf_counter() - t0
    srt = sorted(samples)
    ms_per_step = srt[len(srt) // 2] if len(srt) % 2 else 0.5 * (srt[len(srt) // 2 - 1] + srt[len(srt) // 2])
    print(f"[bench] timed {args.steps} steps in {len(samples)} samples: median {ms_per_step * 1e3:.2f} us/step, "
          f"mean {ms_mean * 1e3:.2f}, min {srt[0] * 1e3:.2f}, max {srt[-1] * 1e3:.2f} (wall incl. capture "
          f"{wall:.3f} s)", file=sys.stderr, flush=True)

    # The partial pass alone and the merge alone, back to back in a graph; the
    # average per launch includes the short gap between consecutive kernels.
    n_k = max(20, min(args.steps, 200))
    part_ms = timed(partial, n_k)
    comb_ms = timed(combine, n_k) if slots > 1 else 0.0
    achieved = partial_bytes / (part_ms * 1e-3) / 1e9

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            t = json.load(open(TRAFFIC_FILE)).get(w.name + (f"/{codes}" if coded else "") +
                                                  (f"/paged{args.page_size}{args.page_layout}" if paged else ""))
            if (t and t.get("kernel") == partial_kernel_name(w)
                    and t.get("kernel_hash") == kernel_source_hash(t["kernel"])
                    and t.get("tile_len") == plan.tile_len and t.get("spans", 0) == plan.spans):
                traffic = t.get("bytes_per_launch")
        except (OSError, ValueError):
            traffic = None

    # The streaming-read ceiling: the library's plain read kernel over the
    # same number of bytes as the partial pass's K/V, in windows rotating
    # over >= 1 GiB so the last-level cache cannot serve them; best of both
    # read patterns (strided over the grid; a contiguous range per
    # workgroup) at a few grid sizes.
    ceiling = None
    if not args.no_ceiling:
        win = (kv_b + 15) // 16 * 16
        nwin = max(2, math.ceil((1 << 30) / win))
        cbuf = torch.empty(nwin * win, dtype=torch.uint8, device=dev)
        cbuf.fill_(1)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        best = None
        for pattern, wgs in ((0, (2048, 8192, 16384, 32768)), (1, (256, 512, 1024, 2048, 4096))):
            for wg in wgs:
                ms = timed(lambda i, wg=wg, pattern=pattern: fd.stream_read(
                    cbuf, win, wg, sink, offset=(i % nwin) * win, pattern=pattern), n_k)
                gbs = win / (ms * 1e-3) / 1e9
                print(f"[bench] stream read {win} B, pattern {pattern}, {wg} workgroups: {ms * 1e3:.2f} us, "
                      f"{gbs:.0f} GB/s", file=sys.stderr, flush=True)
                if best is None or gbs > best[0]:
                    best = (gbs, wg, ms, pattern)
        del cbuf
        ceiling = {"kernel": "fd_stream_read_kernel" if best[3] == 0 else "fd_stream_read_chunk_kernel",
                   "bytes_per_launch": win, "achieved": round(best[0], 2),
                   "unit": "GB/s", "us_per_launch": round(best[2] * 1e3, 3), "workgroups": best[1],
                   "frac_of_peak": round(best[0] / HBM_PEAK_GBS, 4)}

    for i in range(args.calibrate_copy):
        a = torch.empty(1 << 29, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    result = {
        "metric": METRIC,
        "value": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "timing": {"statistic": "median", "samples": len(samples), "steps_per_sample": per,
                   "us_per_step_mean": round(ms_mean * 1e3, 3), "us_per_step_min": round(srt[0] * 1e3, 3),
                   "us_per_step_max": round(srt[-1] * 1e3, 3)},
        "pct_of_hbm_peak": round(100 * step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (w.dtype + (" q/out, fp8 e4m3 k/v" if codes == "fp8" else " q/out, int8 k/v")) if coded else w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.batch, "q_heads": w.num_q_heads,
            "kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "q_len": w.q_len,
            "cache_lens": "fixed %d" % lens[0] if len(set(lens)) == 1 else "U%s sum %d" % (
                list(w.len_range), sum(lens)),
            "tile_len": plan.tile_len, "splits": slots, "spans": plan.spans, "kv_copies": copies,
            "kv_cache": (f"paged, {args.page_size}-key pages, {args.page_layout}" if paged else "contiguous") +
                        ({"fp8": ", fp8 e4m3 (per-tensor scales)", "int8": ", int8 (symmetric per-tensor scales)",
                          None: ""}[codes]),
            "step_bytes": step_bytes, "timing": "eager" if args.no_graph else "graph",
        },
        "kernels": {"partial_us": round(part_ms * 1e3, 3), "combine_us": round(comb_ms * 1e3, 3)},
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": partial_kernel_name(w), "bytes_per_launch": partial_bytes,
        },
    }
    flops = algorithmic_flops(w, lens)
    if w.dtype == "bf16" and flops / partial_bytes > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        # Above the machine balance (about 312 flop per byte) the partial
        # pass is a dense contraction (a long chunk) and is priced against the
        # matrix cores, with the HBM figures kept beside it; decode and short
        # verification chunks stay HBM-bound.
        tflops = flops / (part_ms * 1e-3) / 1e12
        result["roofline"] = {
            "bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
            "kernel": partial_kernel_name(w), "flops_per_launch": flops,
            "hbm_achieved_GBs": round(achieved, 2),
        }
    if ceiling is not None:
        result["ceiling"] = ceiling
        if result["roofline"]["bound"] == "hbm":
            result["roofline"]["frac_of_ceiling"] = round(achieved / ceiling["achieved"], 4)
    if not args.no_cpu_baseline and (coded or paged):
        print("[bench] cpu baseline is timed on the contiguous bf16/fp32 workload only", file=sys.stderr)
    elif not args.no_cpu_baseline:
        print("[bench] timing the fp64 oracle on host cores", file=sys.stderr, flush=True)
        qh, kh, vh, clh = workload_inputs(w)
        result["cpu_baseline"] = cpu_baseline(w, qh, kh, vh, clh, step_bytes, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
