"""Summaries of rocprofv3 runs of bench.py: kernel time tables and HBM traffic.

    python -m sparse_moe_layer_correction_amd.profiling stats  STATS_CSV  OUT_MD  "COMMAND"
    python -m sparse_moe_layer_correction_amd.profiling traffic WORKLOAD FETCH_CSV WRITE_CSV OUT_JSON "COMMANDS"
    python -m sparse_moe_layer_correction_amd.profiling mfma WORKLOAD COUNTER_CSV OUT_MD "COMMAND" T,H,L,E,I,K,Is

``stats`` turns a ``rocprofv3 --kernel-trace --stats -f csv`` kernel_stats.csv
into a short markdown table of the layer's kernels. ``traffic`` turns two
``rocprofv3 --pmc FETCH_SIZE`` / ``--pmc WRITE_SIZE`` counter files of the same
bench command into HBM bytes per launch for each phase of the forward, scaled
by what the counters read for a plain device-to-device copy of known size that
the same process ran (``bench.py --calibrate-copy``), and records them with a
hash of the kernel source so that bench.py stops reporting them once the kernel
changes. ``mfma`` turns one ``rocprofv3 --pmc`` run of MFMA counters over the
tiled GEMM launches into the matrix-core busy share, the issued bf16 MFMA
FLOPs against the algorithmic ones, and the clock, per product of the forward.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_moe_layer_correction_amd", "csrc")

# kernel families and the sources that define them
FAMILIES = {"gemm": ("gemm.h", "common.h"), "skinny": ("skinny.hip", "common.h")}

# copy of known size made by bench.py --calibrate-copy (bytes read = bytes written)
CALIBRATION_BYTES = 1 << 30


def _code_only(text: str) -> str:
    """Source text without comments and blank-line or trailing-space differences."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash(family: str) -> str:
    """Hash of the code (comments left out) of the sources a kernel family is built from."""
    h = hashlib.sha256()
    for f in FAMILIES[family]:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    name = re.sub(r"\(.*$", "", name.replace("void ", ""))
    return name.replace("moe::", "")


def summarize_stats(stats_csv: str, out_md: str, command: str) -> None:
    rows = list(csv.DictReader(open(stats_csv)))
    ours = [r for r in rows if "moe::" in r["Name"]]
    total = sum(float(r["TotalDurationNs"]) for r in ours)
    lines = [f"# rocprofv3 kernel summary", "", "Command:", "", "```", command, "```", "",
             "Kernels of the library only (the seeded input generator's torch kernels are left out).", "",
             "| kernel | calls | avg (us) | min (us) | max (us) | total (ms) | share |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for r in sorted(ours, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} | {100 * float(r['TotalDurationNs']) / total:.1f}% |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _per_dispatch(counter_csv: str, counter: str):
    """[(kernel name, value in KiB)] in dispatch order."""
    acc = defaultdict(float)
    names = {}
    for r in csv.DictReader(open(counter_csv)):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        acc[d] += float(r["Counter_Value"])
        names[d] = r["Kernel_Name"]
    return [(names[d], acc[d]) for d in sorted(acc)]


# which kernel a phase of the forward launches, by the order bench.py's profiled
# step runs them (grouped launches carry their epilogue in the name)
# (the few-token kernels: <slabs per wave, epilogue, weight format 0 bf16 / 1 MXFP8 / 3 MXFP4>)
PHASE_KERNELS = {
    "expert_up": (r"gemm_bf16_kernel<256, 256, 2, 4, 1, 2, 3>",) +
                 tuple(f"skinny_kernel<{ns}, 1, {f}>" for ns in (1, 4) for f in (0, 1, 3)),
    "expert_down": (r"gemm_bf16_kernel<256, 256, 2, 2, 0, 1, 3>",) +
                   tuple(f"skinny_kernel<{ns}, 0, {f}>" for ns in (1, 4) for f in (0, 1, 3)),
}


def summarize_traffic(workload: str, fetch_csv: str, write_csv: str, out_json: str, commands: str) -> dict:
    fetch = _per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _per_dispatch(write_csv, "WRITE_SIZE")
    cal_f = [v for n, v in fetch if "copyBuffer" in n or "copy" in n.lower()]
    cal_w = [v for n, v in write if "copyBuffer" in n or "copy" in n.lower()]
    if not cal_f or not cal_w:
        raise SystemExit("no calibration copy found in the counter files")
    # the largest copy is the calibration one
    f_scale = CALIBRATION_BYTES / (max(cal_f) * 1024.0)
    w_scale = CALIBRATION_BYTES / (max(cal_w) * 1024.0)
    rec = {}
    for phase, pats in PHASE_KERNELS.items():
        for pat in pats:
            fv = [v for n, v in fetch if pat in n]
            wv = [v for n, v in write if pat in n]
            if fv and wv:
                family = "gemm" if "gemm" in pat else "skinny"
                fb = sum(fv) / len(fv) * 1024.0 * f_scale
                wb = sum(wv) / len(wv) * 1024.0 * w_scale
                rec[phase] = {"kernel": pat, "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
                              "bytes_per_launch": round(fb + wb), "launches": len(fv),
                              "kernel_hash": kernel_source_hash(family)}
    data = {}
    if os.path.exists(out_json):
        data = json.load(open(out_json))
    data[workload] = {"phases": rec, "fetch_scale": f_scale, "write_scale": w_scale,
                      "calibration": f"device-to-device copy of {CALIBRATION_BYTES} bytes",
                      "commands": commands}
    with open(out_json, "w") as f:
        json.dump(data, f, indent=1)
    return data


# the tiled GEMM launches of one large-batch forward, in launch order
GEMM_PHASES = ("router", "fc1_shared_up", "expert_up", "expert_down", "fc2_shared_down")


def gemm_phase_flops(T: int, H: int, L: int, E: int, I: int, K: int, Is: int) -> dict:
    """Algorithmic FLOPs of each tiled product of the forward (multiply-adds count 2)."""
    return {"router": 2 * T * H * E, "fc1_shared_up": 2 * T * H * (L + Is), "expert_up": 2 * T * K * L * I,
            "expert_down": 2 * T * K * I * L, "fc2_shared_down": 2 * T * (L + Is) * H}


def _per_dispatch_rows(counter_csv: str):
    """{dispatch id: {"name", "start", "end", counter: summed value}} from a counter_collection.csv."""
    out = {}
    for r in csv.DictReader(open(counter_csv)):
        d = out.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
        for k in ("Start_Timestamp", "End_Timestamp"):
            if r.get(k):
                d[k] = int(r[k])
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def summarize_mfma(workload: str, counter_csv: str, out_md: str, command: str, dims: str) -> None:
    """MFMA utilisation of the tiled products from one ``rocprofv3 --pmc MfmaUtil
    SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE`` run
    restricted to the GEMM kernel; dims = "T,H,L,E,I,K,Is"."""
    flops = gemm_phase_flops(*[int(v) for v in dims.split(",")])
    rows = _per_dispatch_rows(counter_csv)
    # the raw GRBM_GUI_ACTIVE of a dispatch is the sum over the accelerator's XCDs
    n_xcc = 1
    info = os.path.join(os.path.dirname(counter_csv), "ctr_agent_info.csv")
    if os.path.exists(info):
        n_xcc = max(int(r.get("Num_Xcc") or 0) for r in csv.DictReader(open(info))) or 1
    ids = [d for d in sorted(rows) if "gemm_bf16_kernel" in rows[d]["name"]]
    if not ids or len(ids) % len(GEMM_PHASES):
        raise SystemExit(f"{len(ids)} GEMM dispatches: not whole forwards of {len(GEMM_PHASES)} launches")
    acc = defaultdict(list)
    for i, d in enumerate(ids):
        ph = GEMM_PHASES[i % len(GEMM_PHASES)]
        name = short_name(rows[d]["name"])
        # the epilogue is the fifth template argument: 1 relu2 (expert up), 0 plain (expert down), -1 dense
        m = re.search(r"<(?:[^,>]+, ){4}(-?\d+),", name)
        want = {"expert_up": "1", "expert_down": "0"}.get(ph, "-1")
        if m is None or m.group(1) != want:
            raise SystemExit(f"dispatch {d} ({name}) is not the {ph} launch")
        acc[ph].append(rows[d])
    lines = ["# MFMA utilisation of the tiled products (rocprofv3 counters)", "", "Command:", "", "```", command,
             "```", "", f"Workload: {workload} (T, H, L, E, I, K, Is = {dims}). Averages over "
             f"{len(ids) // len(GEMM_PHASES)} forwards; times are those of the dispatches under the profiler.", "",
             "* MFMA busy: rocprofv3's `MfmaUtil`, the SIMD cycles with the matrix core busy "
             "(`SQ_VALU_MFMA_BUSY_CYCLES`) over the dispatch's GPU-active cycles (`GRBM_GUI_ACTIVE`, "
             "busiest XCD) times the 1024 SIMDs.",
             "* Issued / algorithmic: `SQ_INSTS_VALU_MFMA_MOPS_BF16` x 512 over the product's own FLOPs "
             "(the padding rows of grouped tiles and the router's three bf16 weight parts issue more).",
             f"* Clock: `GRBM_GUI_ACTIVE` / {n_xcc} XCDs over the dispatch's duration; the bf16 peak at that "
             "clock scales 2.5 PFLOP/s (quoted at 2.4 GHz) by it.", "",
             "| product | kernel | ms | TFLOP/s | MFMA busy | issued / algorithmic | clock (GHz) "
             "| bf16 peak at that clock (TFLOP/s) |",
             "|---|---|---:|---:|---:|---:|---:|---:|"]
    for ph in GEMM_PHASES:
        rs = acc[ph]
        timed = [r for r in rs if r.get("End_Timestamp", 0) > r.get("Start_Timestamp", 0)]
        util = sum(r.get("MfmaUtil", float("nan")) for r in rs) / len(rs)
        mops = sum(r.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for r in rs) / len(rs)
        if timed:
            ns = sum(r["End_Timestamp"] - r["Start_Timestamp"] for r in timed) / len(timed)
            ghz = sum(r.get("GRBM_GUI_ACTIVE", 0.0) / n_xcc / (r["End_Timestamp"] - r["Start_Timestamp"])
                      for r in timed) / len(timed)
            tail = f"{ns / 1e6:.3f} | {flops[ph] / ns / 1e3:.0f} |"
            clk = f"{ghz:.2f} | {2500 * ghz / 2.4:.0f}"
        else:
            tail, clk = "n/a | n/a |", "n/a | n/a"
        lines.append(f"| {ph} | `{short_name(rs[0]['name'])}` | {tail} {util:.1f} % | "
                     f"{mops * 512 / flops[ph]:.3f} | {clk} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        summarize_stats(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "mfma":
        summarize_mfma(*sys.argv[2:7])
    elif sys.argv[1] == "traffic":
        print(json.dumps(summarize_traffic(*sys.argv[2:7]), indent=1))
    else:
        raise SystemExit(__doc__)
