"""Summaries of rocprofv3 CSV output (kernel trace statistics and HBM counters).

Usage (from the repository root, after the rocprofv3 runs):

  python -m sparse_moe_ffn_02_amd.profile_summary trace  DIR  OUT.md  "COMMAND"
  python -m sparse_moe_ffn_02_amd.profile_summary counters FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR \
         COPY_BYTES OUT.md "COMMANDS"

`trace` reads DIR/run_kernel_stats.csv (rocprofv3 --kernel-trace --stats
--output-format csv -o run).  `counters` reads run_counter_collection.csv of
four --pmc runs: FETCH_SIZE and WRITE_SIZE over the workload, and the same two
counters over a plain device-to-device copy of COPY_BYTES bytes.  The copy
gives the scale from counter units to bytes (FETCH_SIZE and WRITE_SIZE are
reported in KiB; the copy shows how many bytes one unit stands for on this
part).  The counter summary ends with one machine-readable line
`traffic-json: {...}` holding, per kernel, the scaled HBM bytes per launch and
the digest of the kernel sources the counters were taken on.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import sys
from collections import defaultdict

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


def source_digest() -> str:
    """sha256 over the HIP sources and headers, in name order."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()[:16]


def short_name(kernel: str) -> str:
    """moe::k_gateup_split(moe::FfnArgs) -> gateup_split;
    void moe::k_router_logits<4>(moe::RouteArgs) -> router_logits."""
    k = kernel.split("(")[0]
    k = k.split("<")[0]
    k = k.split("::")[-1]
    if k.startswith("k_"):
        k = k[2:]
    return k


def is_library_kernel(kernel: str) -> bool:
    return kernel.startswith("moe::") or kernel.startswith("void moe::")


def trace_summary(d: str, out: str, command: str) -> None:
    rows = list(csv.DictReader(open(os.path.join(d, "run_kernel_stats.csv"))))
    lines = ["# Kernel trace statistics", "", f"Command: `{command}`", "",
             f"Kernel sources digest: `{source_digest()}`", "",
             "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['Name'][:70]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def _counter_means(d: str):
    acc = defaultdict(list)
    for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
        acc[(r["Kernel_Name"], r["Counter_Name"])].append(float(r["Counter_Value"]))
    return acc


def _copy_scale(d: str, counter: str, copy_bytes: int) -> float:
    """Bytes per counter unit, from the largest copy dispatch (the timed copy)."""
    vals = [max(v) for (k, c), v in _counter_means(d).items() if c == counter and "copyBuffer" in k]
    if not vals:
        raise SystemExit(f"no copy kernel with {counter} in {d}")
    return copy_bytes / max(vals)


def counters_summary(fd: str, wd: str, cfd: str, cwd: str, copy_bytes: int, out: str, command: str) -> None:
    fs = _copy_scale(cfd, "FETCH_SIZE", copy_bytes)
    ws = _copy_scale(cwd, "WRITE_SIZE", copy_bytes)
    fetch = {k: v for (k, c), v in _counter_means(fd).items() if c == "FETCH_SIZE"}
    write = {k: v for (k, c), v in _counter_means(wd).items() if c == "WRITE_SIZE"}
    digest = source_digest()
    lines = ["# HBM traffic per dispatch (FETCH_SIZE, WRITE_SIZE)", "", f"Commands: `{command}`", "",
             f"Kernel sources digest: `{digest}`", "",
             f"Calibration: a plain device copy of {copy_bytes} bytes reads {copy_bytes / fs:.1f} FETCH_SIZE units "
             f"and writes {copy_bytes / ws:.1f} WRITE_SIZE units, so one FETCH unit = {fs:.1f} bytes and one WRITE "
             f"unit = {ws:.1f} bytes.", "",
             "| kernel | dispatches | FETCH_SIZE mean | WRITE_SIZE mean | read MB / launch | written MB / launch |",
             "|---|---|---|---|---|---|"]
    table = {}
    for k in sorted(set(fetch) | set(write)):
        if not is_library_kernel(k):
            continue
        f = fetch.get(k, [0.0])
        w = write.get(k, [0.0])
        fm, wm = sum(f) / len(f), sum(w) / len(w)
        table[short_name(k)] = {"read_bytes": round(fm * fs), "write_bytes": round(wm * ws)}
        lines.append(f"| `{short_name(k)}` | {len(f)} | {fm:.1f} | {wm:.1f} | {fm * fs / 1e6:.2f} | {wm * ws / 1e6:.2f} |")
    lines += ["", "traffic-json: " + json.dumps({"digest": digest, "kernels": table})]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def load_traffic(path: str):
    """The traffic-json line of a counter summary, or None if the kernel
    sources changed since the counters were taken (or the file is absent)."""
    try:
        with open(path) as f:
            for line in f:
                if line.startswith("traffic-json: "):
                    data = json.loads(line[len("traffic-json: "):])
                    return data if data.get("digest") == source_digest() else None
    except OSError:
        return None
    return None


def main(argv):
    if len(argv) >= 4 and argv[1] == "trace":
        trace_summary(argv[2], argv[3], argv[4] if len(argv) > 4 else "")
    elif len(argv) >= 8 and argv[1] == "counters":
        counters_summary(argv[2], argv[3], argv[4], argv[5], int(argv[6]), argv[7], argv[8] if len(argv) > 8 else "")
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
