"""Workgroup timeline of the matrix-core decode and chunk kernels (diagnostic).

Runs a workload's partial pass through ``libfd_timeline.so`` (the library
built with FD_WG_TIMELINE=1; ``build.build_timeline()``) and prints where a
launch spends its time: when the workgroups start, when wave 0's first block
lands, when each wave leaves its block loop, when the workgroups end (100 MHz
``s_memrealtime`` clock, shared by all XCDs), and the end times per XCD.

    python -m decode_attention_14_amd.timeline [--workload gqa_32k] [--kv-fp8 | --kv-int8] [--step]

``--step`` times the partial pass inside whole ``fd_decode_attention`` calls
(partial kernel, then the merge kernel) instead of back-to-back partial
passes.
Needs a GPU.  The timeline build computes the same results as ``libfd.so``.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import sys

import numpy as np
import torch

from . import binding as fd
from .build import TIMELINE_LIB
from .inputs import WORKLOADS, fp8_scale_for, int8_scale_for, quantize_fp8, quantize_int8, workload_inputs

SLOTS = 16           # per workgroup: start, first block, 8 wave loop exits, end, XCD
CHUNK_ROW_TILE = 128  # packed query rows per workgroup of the chunk kernel
MAX_WGS = 4096
T_START, T_FIRST, T_LOOP, T_END, T_XCC = 0, 1, 2, 10, 11
T_CLK0, T_CLK1 = 12, 13  # chunk kernel: shader clock at the first stage and at wave 0's loop exit
TICK_US = 0.01       # s_memrealtime runs at 100 MHz


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--workload", default="gqa_32k")
    ap.add_argument("--kv-fp8", action="store_true")
    ap.add_argument("--kv-int8", action="store_true")
    ap.add_argument("--launches", type=int, default=6, help="launches whose timelines are read")
    ap.add_argument("--step", action="store_true", help="time the whole fd_decode_attention call")
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        print("the timeline needs a GPU", file=sys.stderr)
        return 1
    lib = fd.use_library(TIMELINE_LIB)
    for name in ("fd_debug_timeline", "fd_debug_chunk_timeline"):
        getattr(lib, name).argtypes = [ctypes.c_void_p, ctypes.c_uint64]
        getattr(lib, name).restype = ctypes.c_int

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    q, k, v, cl = workload_inputs(w)
    plan = fd.plan_for(q, k, cl)
    if plan.spans:
        # The rows below follow the tile-mode grid (KV head, tile, sequence);
        # a span launch's grid depends on residency, so time the tile plan.
        print(f"plan asks for {plan.spans} balanced spans; timing its tile plan instead", file=sys.stderr)
        plan.plan.spans = 0
    rows = w.num_q_heads // w.num_kv_heads * w.q_len
    codes = "fp8" if args.kv_fp8 else "int8" if args.kv_int8 else None
    chunk = rows > 32
    if w.dtype != "bf16" or (chunk and codes):
        print("the timeline covers the matrix-core decode kernel (bf16 queries, up to 32 rows per KV head) and "
              "the pipelined chunk kernel (bf16 queries and caches, more rows)", file=sys.stderr)
        return 2
    read_timeline = lib.fd_debug_chunk_timeline if chunk else lib.fd_debug_timeline
    if codes:
        scale_for, quantize = (fp8_scale_for, quantize_fp8) if codes == "fp8" else (int8_scale_for, quantize_int8)
        ks, vs = scale_for(k), scale_for(v)
        k, v = quantize(k, ks), quantize(v, vs)
        partials = fd.decode_partials_fp8 if codes == "fp8" else fd.decode_partials_int8
    # K/V copies in rotation, so the last-level cache cannot serve a launch
    copies = int(min(8, max(2, -(-(1 << 30) // max(1, 2 * k.numel() * k.element_size())))))
    qd, cld = q.to(dev), cl.to(dev)
    kd0, vd0 = k.to(dev), v.to(dev)
    kvs = [(kd0, vd0)] + [(kd0.clone(), vd0.clone()) for _ in range(copies - 1)]
    slots = plan.max_splits
    o_part = torch.empty(*qd.shape[:3], slots, w.head_dim, dtype=torch.float32, device=dev)
    m_part = torch.empty(*qd.shape[:3], slots, dtype=torch.float32, device=dev)
    l_part = torch.empty_like(m_part)

    ws = fd.new_workspace(fd.workspace_bytes(fd.dims_of(qd, kd0), slots), dev)
    out = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)

    def launch(i):
        kd, vd = kvs[i % copies]
        if args.step:
            if codes:
                attn = fd.decode_attention_fp8 if codes == "fp8" else fd.decode_attention_int8
                attn(qd, kd, vd, cld, ks, vs, scale=w.scale, plan=plan.plan, out=out, lse=lse, workspace=ws)
            else:
                fd.decode_attention(qd, kd, vd, cld, scale=w.scale, plan=plan.plan, out=out, lse=lse, workspace=ws)
        elif codes:
            partials(qd, kd, vd, cld, ks, vs, scale=w.scale, plan=plan.plan, o_part=o_part, m_part=m_part,
                     lse_part=l_part)
        else:
            fd.decode_partials(qd, kd, vd, cld, scale=w.scale, plan=plan.plan, o_part=o_part, m_part=m_part,
                               lse_part=l_part)

    row_tiles = -(-rows // CHUNK_ROW_TILE) if chunk else 1
    nwg = w.num_kv_heads * slots * row_tiles * w.batch
    if nwg > MAX_WGS:
        print(f"{nwg} workgroups; the timeline keeps the first {MAX_WGS}", file=sys.stderr)
        nwg = MAX_WGS
    waves = 8 if codes or chunk else 4
    for i in range(20):
        launch(i)
    torch.cuda.synchronize()
    print(f"{w.name}{'/' + codes if codes else ''}: plan {plan.plan}, {nwg} workgroups of {waves} waves",
          flush=True)
    buf = np.zeros(nwg * SLOTS, dtype=np.uint64)
    summary = []
    for rep in range(args.launches):
        launch(2 * rep)          # the launch before keeps the clocks up
        launch(2 * rep + 1)
        torch.cuda.synchronize()
        if read_timeline(buf.ctypes.data, buf.nbytes) != 0:
            raise RuntimeError("reading the workgroup timeline failed")
        t = buf.reshape(nwg, SLOTS).astype(np.int64)
        t0 = t[:, T_START].min()
        start = (t[:, T_START] - t0) * TICK_US
        first = (t[:, T_FIRST] - t[:, T_START]) * TICK_US
        loops = (t[:, T_LOOP:T_LOOP + waves] - t[:, [T_START]]) * TICK_US
        end = (t[:, T_END] - t0) * TICK_US
        after_last = end - start - loops.max(axis=1)
        row = {
            "span_us": round(float(end.max()), 2),
            "start_spread_us": round(float(start.max()), 2),
            "first_block_us": round(float(first.mean()), 2),
            "loop_us": round(float((loops.max(axis=1) - first).mean()), 2),
            "loop_us_max": round(float((loops.max(axis=1) - first).max()), 2),
            "wave_loop_end_us": [round(float(x), 2) for x in loops.mean(axis=0)],
            "end_after_last_wave_us": round(float(after_last.mean()), 2),
            **({"loop_clock_mhz": round(float(np.median((t[:, T_CLK1] - t[:, T_CLK0]) /
                                                          np.maximum(1, t[:, T_LOOP] - t[:, T_FIRST]) / TICK_US)), 1)}
               if chunk else {}),
            "end_spread_us": round(float(end.max() - end.min()), 2),
            "end_us_per_xcd": {int(x): round(float(end[t[:, T_XCC] == x].mean()), 2)
                               for x in np.unique(t[:, T_XCC])},
        }
        summary.append(row)
        print(json.dumps(row), flush=True)
    keys = ("span_us", "start_spread_us", "first_block_us", "loop_us", "loop_us_max", "end_after_last_wave_us",
            "end_spread_us") + (("loop_clock_mhz",) if chunk else ())
    print("median over launches:", json.dumps({k: float(np.median([r[k] for r in summary])) for k in keys}),
          flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
