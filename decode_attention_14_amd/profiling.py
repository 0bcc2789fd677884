"""Summaries of rocprofv3 runs of bench.py (diagnostic; needs no GPU).

* ``trace DIR``: the kernel table of a ``--kernel-trace --stats`` run.
* ``traffic KEY FETCH_DIR WRITE_DIR BENCH_JSON [--update]``: HBM bytes per
  partial-pass launch from a ``--pmc FETCH_SIZE`` and a ``--pmc WRITE_SIZE``
  run of ``bench.py ... --calibrate-copy N``.  Each counter is scaled by what
  it reads for the plain 512 MiB device copy in the same run (512 MiB read and
  written), and the figure is tied to the kernel's source hash and the tile
  length (from the bench line in BENCH_JSON), as bench.py's roofline.traffic
  requires.  ``--update`` writes the entry into profiles/traffic.json under
  KEY (the workload name, ``/fp8`` or ``/int8`` for one-byte caches).

    python -m decode_attention_14_amd.profiling trace prof/trace_32k
    python -m decode_attention_14_amd.profiling traffic gqa_32k DIR_F DIR_W bench.json --update
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_KIB = 524288.0  # the calibration copy: 512 MiB read, 512 MiB written
PARTIAL_KERNELS = ("fd_mfma_partial_kernel<", "fd_mfma_chunk_kernel<", "fd_mfma_chunk8_kernel<",
                   "fd_partial_kernel<")


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def short_name(name: str) -> str:
    """A kernel's name without return type, namespaces and argument list."""
    name = name.replace("void ", "").replace("fdk::(anonymous namespace)::", "")
    return name[:name.rindex("(")] if name.endswith(")") else name


def kernel_table(run_dir: str):
    """(name, calls, average ns, min ns, max ns) rows of a kernel-trace run."""
    path = _one(os.path.join(run_dir, "**", "*kernel_stats.csv"))
    return [(r["Name"], int(r["Calls"]), float(r["AverageNs"]), int(float(r["MinNs"])), int(float(r["MaxNs"])))
            for r in csv.DictReader(open(path))]


def counter_per_dispatch(run_dir: str, counter: str):
    """{dispatch id: (kernel name, counter value summed over its rows)}."""
    path = _one(os.path.join(run_dir, "**", "*counter_collection.csv"))
    val = collections.defaultdict(float)
    name = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        val[d] += float(r["Counter_Value"])
        name[d] = r["Kernel_Name"]
    return {d: (name[d], v) for d, v in val.items()}


def counter_summary(run_dir: str, counter: str, copies: int = 2):
    """Average KiB per dispatch of the partial-pass kernel and of the 512 MiB
    calibration copies in one counter run: the last `copies` device copies
    of the run (bench.py makes them after its timing; earlier copies clone
    the K/V cache)."""
    per = counter_per_dispatch(run_dir, counter)
    part = [v for n, v in per.values() if any(k in n for k in PARTIAL_KERNELS)]
    copy = [per[d][1] for d in sorted(per) if "copyBuffer" in per[d][0]][-copies:]
    if not part or len(copy) < copies:
        raise ValueError(f"{run_dir}: {len(part)} partial dispatches, {len(copy)} calibration copies")
    return sum(part) / len(part), len(part), sum(copy) / len(copy), len(copy)


def traffic_entry(key: str, fetch_dir: str, write_dir: str, bench_line: dict) -> dict:
    sys.path.insert(0, ROOT)
    from bench import kernel_source_hash  # noqa: E402  (the hash bench.py checks)

    fk, nf, fc, ncf = counter_summary(fetch_dir, "FETCH_SIZE")
    wk, nw, wc, ncw = counter_summary(write_dir, "WRITE_SIZE")
    fs, ws = COPY_KIB / fc, COPY_KIB / wc
    kernel = bench_line["roofline"]["kernel"]
    return {
        "kernel": kernel,
        "kernel_hash": kernel_source_hash(kernel),
        "tile_len": bench_line["config"]["tile_len"],
        "spans": bench_line["config"].get("spans", 0),
        "fetch_kib_raw": round(fk, 2),
        "fetch_scale": round(fs, 4),
        "write_kib_raw": round(wk, 2),
        "write_scale": round(ws, 4),
        "bytes_per_launch": int(round(fk * 1024 * fs + wk * 1024 * ws)),
        "dispatches": [nf, nw],
        "calibration_kib": {"fetch": round(fc, 1), "write": round(wc, 1), "copies": [ncf, ncw]},
    }


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("run_dir")
    f = sub.add_parser("traffic")
    f.add_argument("key")
    f.add_argument("fetch_dir")
    f.add_argument("write_dir")
    f.add_argument("bench_json", help="file whose last line is bench.py's JSON line")
    f.add_argument("--update", action="store_true")
    args = ap.parse_args(argv)
    if args.cmd == "trace":
        print("| Kernel | Calls | Average ns | Min ns | Max ns |\n|---|---|---|---|---|")
        for name, calls, avg, lo, hi in kernel_table(args.run_dir):
            print(f"| {short_name(name)} | {calls} | {avg:.1f} | {lo} | {hi} |")
        return 0
    line = json.loads(open(args.bench_json).read().strip().splitlines()[-1])
    entry = traffic_entry(args.key, args.fetch_dir, args.write_dir, line)
    print(json.dumps({args.key: entry}, indent=2))
    if args.update:
        data = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}
        entry["source"] = data.get(args.key, {}).get("source", "")
        data[args.key] = entry
        with open(TRAFFIC_FILE, "w") as fh:
            json.dump(data, fh, indent=2)
            fh.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
