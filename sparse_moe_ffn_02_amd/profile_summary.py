"""Summaries of rocprofv3 CSV output (kernel trace statistics and HBM counters).

Usage (from the repository root, after the rocprofv3 runs):

  python -m sparse_moe_ffn_02_amd.profile_summary trace  DIR  OUT.md  "COMMAND"
  python -m sparse_moe_ffn_02_amd.profile_summary counters FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR \
         COPY_BYTES OUT.md "COMMANDS"

  python -m sparse_moe_ffn_02_amd.profile_summary mfma   DIR  OUT.md  "COMMAND"

`trace` reads DIR/run_kernel_stats.csv (rocprofv3 --kernel-trace --stats
--output-format csv -o run).  `counters` reads run_counter_collection.csv of
four --pmc runs: FETCH_SIZE and WRITE_SIZE over the workload, and the same two
counters over a plain device-to-device copy of COPY_BYTES bytes.  The copy
gives the scale from counter units to bytes (FETCH_SIZE and WRITE_SIZE are
reported in KiB; the copy shows how many bytes one unit stands for on this
part).  The counter summary ends with one machine-readable line
`traffic-json: {...}` holding, per kernel, the scaled HBM bytes per launch and
the digest of the kernel sources the counters were taken on.  `mfma` reads
one --pmc run of SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE (plus any other
counters in it) and ends with an `mfma-json: {...}` line of the same kind.
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


N_SIMD = 256 * 4     # MI355X: 256 compute units of 4 SIMDs


def mfma_summary(d: str, out: str, command: str) -> None:
    """MFMA pipe utilisation per kernel from one --pmc run holding rocprofv3's
    derived MfmaUtil (percent of SIMD cycles the matrix pipe is busy), or
    SQ_VALU_MFMA_BUSY_CYCLES (busy cycles summed over the SIMDs) with
    GRBM_GUI_ACTIVE (cycles the GPU is busy with the dispatch), giving
    busy fraction = MFMA busy / (GUI active x 1024 SIMDs).  Other counters
    present in the run (e.g. SQ_INSTS_VALU_MFMA_MOPS_F8, MFMA work in units
    of 512 flops) are reported per dispatch as well."""
    acc = _counter_means(d)
    counters = sorted({c for (_, c) in acc})
    digest = source_digest()
    lines = ["# MFMA utilisation per dispatch", "", f"Command: `{command}`", "",
             f"Kernel sources digest: `{digest}`", "",
             "busy fraction = MfmaUtil / 100 (rocprofv3: SQ_VALU_MFMA_BUSY_CYCLES summed over the SIMDs / "
             f"(GRBM_GUI_ACTIVE max over XCCs x {N_SIMD} SIMDs))", "",
             "| kernel | dispatches | " + " | ".join(f"{c} mean" for c in counters) + " | MFMA busy fraction |",
             "|---|---|" + "---|" * len(counters) + "---|"]
    kernels = sorted({k for (k, _) in acc if is_library_kernel(k)})
    table = {}
    for k in kernels:
        means = {c: (sum(acc[(k, c)]) / len(acc[(k, c)])) if acc.get((k, c)) else None for c in counters}
        n = max(len(acc.get((k, c), [])) for c in counters)
        busy, gui = means.get("SQ_VALU_MFMA_BUSY_CYCLES"), means.get("GRBM_GUI_ACTIVE")
        if means.get("MfmaUtil") is not None:
            # rocprofv3's own derived metric (percent): busy cycles summed over SIMDs / (max over
            # XCCs of the GUI-active cycles x SIMD count), the reductions done by the profiler
            frac = means["MfmaUtil"] / 100.0
        else:
            frac = busy / (gui * N_SIMD) if busy is not None and gui else None
        table[short_name(k)] = {"busy_frac": None if frac is None else round(frac, 4),
                                **{c: (None if v is None else round(v)) for c, v in means.items()}}
        cells = " | ".join("-" if v is None else f"{v:.4g}" for v in means.values())
        lines.append(f"| `{short_name(k)}` | {n} | {cells} | {'-' if frac is None else f'{frac:.3f}'} |")
    lines += ["", "mfma-json: " + json.dumps({"digest": digest, "kernels": table})]
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def _load_json_line(path: str, tag: str):
    try:
        with open(path) as f:
            for line in f:
                if line.startswith(tag):
                    data = json.loads(line[len(tag):])
                    return data if data.get("digest") == source_digest() else None
    except OSError:
        return None
    return None


def load_mfma(path: str):
    """The mfma-json line of an MFMA summary, or None if the kernel sources
    changed since the counters were taken (or the file is absent)."""
    return _load_json_line(path, "mfma-json: ")


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
    elif len(argv) >= 4 and argv[1] == "mfma":
        mfma_summary(argv[2], argv[3], argv[4] if len(argv) > 4 else "")
    elif len(argv) >= 8 and argv[1] == "counters":
        counters_summary(argv[2], argv[3], argv[4], argv[5], int(argv[6]), argv[7], argv[8] if len(argv) > 8 else "")
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
