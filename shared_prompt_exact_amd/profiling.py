"""Summaries of rocprofv3 output for this library's kernels.

Two summaries, both written as short markdown under ``profiles/``:

* ``kernels``: a ``rocprofv3 --kernel-trace --stats --output-format csv`` run
  of ``bench.py`` -> per-kernel call counts and durations, next to the
  library's own event timings printed by the same run (its JSON line).
* ``traffic``: two ``rocprofv3 --pmc`` runs of the same command, one with
  FETCH_SIZE and one with WRITE_SIZE (KiB per dispatch) -> HBM bytes per
  launch of one kernel.  Each counter is scaled by the factor that makes it
  read the known size of a plain copy in the same run: the repack GATHER of
  hidden-state rows that bench.py times (it reads exactly the bytes it
  writes, (P+NR) rows of Hq*D bf16).  The record stores a hash of the
  kernel's sources; ``load_traffic`` returns it only while they are
  unchanged, so a figure never outlives the code it was measured on.

Usage (repo root):
  python3 -m shared_prompt_exact_amd.profiling kernels STATS_DIR BENCH_LOG OUT.md TITLE CMD
  python3 -m shared_prompt_exact_amd.profiling traffic FETCH_DIR WRITE_DIR KERNEL WORKLOAD OUT.md CMD_FETCH CMD_WRITE
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "shared_prompt_exact_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")

# library kernel name -> (substring of the device symbol, source files it is built from)
_HEADERS = ["common.h", "mfma_common.h", "lds_tiles.h"]
KERNELS = {
    "fwd": ("fwd_mfma_kernel", ["attn_fwd_mfma.hip"] + _HEADERS),
    "bwd_dq": ("bwd_dq_kernel", ["attn_bwd_dq.hip"] + _HEADERS),
    "bwd_dkdv": ("bwd_dkdv_kernel", ["attn_bwd_mfma.hip"] + _HEADERS),
    "bwd_reduce": ("reduce_slots_kernel", ["attn_bwd_mfma.hip"] + _HEADERS),
    "bwd_delta": ("delta_lse2_kernel", ["attn_bwd_mfma.hip"] + _HEADERS),
    "repack": ("repack_kernel", ["repack.hip", "common.h"]),
    "gemm": ("gemm_bf16_kernel", ["gemm.hip"] + _HEADERS),
    "rmsnorm_fwd": ("rmsnorm_fwd_kernel", ["layer_ops.hip", "common.h"]),
    "rmsnorm_bwd": ("rmsnorm_bwd_kernel", ["layer_ops.hip", "common.h"]),
    "norm_wgrad": ("norm_wgrad_partial_kernel", ["layer_ops.hip", "common.h"]),
    "norm_wgrad_sum": ("sum_chunks_kernel", ["layer_ops.hip", "common.h"]),
    "rope": ("rope_kernel", ["layer_ops.hip", "common.h"]),
    "swiglu_fwd": ("swiglu_fwd_kernel", ["layer_ops.hip", "common.h"]),
    "swiglu_bwd": ("swiglu_bwd_kernel", ["layer_ops.hip", "common.h"]),
}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNELS[kernel][1]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def short_name(symbol: str) -> str:
    for k, (sub, _) in KERNELS.items():
        if sub in symbol:
            return k
    return "other"


def _csv(d: str, suffix: str):
    paths = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not paths:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    with open(paths[0]) as fh:
        return list(csv.DictReader(fh))


def _bench_line(path: str) -> dict:
    with open(path) as fh:
        lines = [ln for ln in fh if ln.startswith("{")]
    if not lines:
        raise ValueError(f"no JSON line in {path}")
    return json.loads(lines[-1])


def kernels_summary(stats_dir, bench_log, out_path, title, cmd):
    rows = _csv(stats_dir, "kernel_stats.csv")
    b = _bench_line(bench_log)
    out = [f"# {title}", "", "Command (repo root, MI355X):", "", "    " + cmd, "",
           "| kernel | symbol | calls | avg ms | min ms | max ms | share |", "|---|---|---|---|---|---|---|"]
    for r in rows:
        sym = r["Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").replace("dualkv::", "")
        out.append(f"| {short_name(r['Name'])} | `{sym}` | {r['Calls']} | {float(r['AverageNs']) / 1e6:.3f} | "
                   f"{float(r['MinNs']) / 1e6:.3f} | {float(r['MaxNs']) / 1e6:.3f} | {float(r['Percentage']):.2f}% |")
    if "kernels_ms_per_step" in b:        # the decoder-layer line
        out += ["", "Same run, bench.py's own timing (HIP events): step %.3f ms." % b["ms_per_step"],
                "Per-step kernel time from the library's event profiler inside the timed steps: " +
                ", ".join(f"{k} {v:.3f} ms" for k, v in b["kernels_ms_per_step"].items()) + ".", ""]
    else:
        out += ["", "Same run, bench.py's own timing (HIP events): step %.3f ms, fwd %.3f ms, bwd %.3f ms." % (
            b["ms_per_step"], b["fwd"]["ms"], b["bwd"]["ms"]),
            "Per-kernel averages from the library's event profiler inside the timed steps: " +
            ", ".join(f"{k} {v['avg_ms']:.3f} ms" for k, v in b["kernels"].items()) + ".", "",
            "Dominant kernel roofline as bench.py reports it: `" + json.dumps(b["roofline"]) + "`", ""]
    with open(out_path, "w") as fh:
        fh.write("\n".join(out))
    return "\n".join(out)


def traffic_summary(fetch_dir, write_dir, kernel, workload, out_path, cmd_fetch, cmd_write):
    sys.path.insert(0, ROOT)
    import workloads
    w = workloads.WORKLOADS[workload]
    copy_bytes = w.packed_len * w.n_q_heads * w.head_dim * 2
    f_rows = {int(r["Dispatch_Id"]): r for r in _csv(fetch_dir, "counter_collection.csv")
              if r["Counter_Name"] == "FETCH_SIZE"}
    w_rows = {int(r["Dispatch_Id"]): r for r in _csv(write_dir, "counter_collection.csv")
              if r["Counter_Name"] == "WRITE_SIZE"}
    for i in set(f_rows) & set(w_rows):
        if f_rows[i]["Kernel_Name"] != w_rows[i]["Kernel_Name"]:
            raise ValueError(f"dispatch {i} differs between the two runs")
    kib = lambda r: float(r["Counter_Value"]) * 1024.0
    # the copy: repack dispatches that wrote the gather's known size
    copies = [i for i, r in w_rows.items() if short_name(r["Kernel_Name"]) == "repack"
              and abs(kib(r) - copy_bytes) <= 0.01 * copy_bytes and i in f_rows]
    if not copies:
        raise ValueError("no repack dispatch of the copy's size in the counter runs")
    f_fac = copy_bytes / (sum(kib(f_rows[i]) for i in copies) / len(copies))
    w_fac = copy_bytes / (sum(kib(w_rows[i]) for i in copies) / len(copies))
    mine = [i for i in f_rows if i in w_rows and short_name(f_rows[i]["Kernel_Name"]) == kernel]
    if not mine:
        raise ValueError(f"no dispatch of {kernel}")
    rd = sum(kib(f_rows[i]) for i in mine) / len(mine) * f_fac
    wr = sum(kib(w_rows[i]) for i in mine) / len(mine) * w_fac
    rec = {"kernel": kernel, "workload": workload, "bytes_per_launch": round(rd + wr),
           "read_bytes": round(rd), "write_bytes": round(wr), "dispatches": len(mine),
           "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4),
           "copy_bytes": copy_bytes, "copy_dispatches": len(copies), "source_sha256": source_hash(kernel)}
    out = [f"# HBM traffic of `{kernel}`, {workload}", "",
           "Commands (repo root, MI355X), one counter per run:", "", "    " + cmd_fetch, "    " + cmd_write, "",
           f"Calibration: the repack GATHER of hidden-state rows in the same runs copies "
           f"{copy_bytes} bytes ({w.packed_len} rows x {w.n_q_heads * w.head_dim * 2} B) each way; "
           f"FETCH_SIZE read {copy_bytes / f_fac / 1024:.1f} KiB and WRITE_SIZE "
           f"{copy_bytes / w_fac / 1024:.1f} KiB for it, so the factors are "
           f"{f_fac:.4f} (fetch) and {w_fac:.4f} (write).", "",
           f"`{kernel}` over {len(mine)} dispatches: {rd / 1e9:.4f} GB read, {wr / 1e9:.4f} GB written per launch "
           f"(calibrated).", "", "```json", json.dumps(rec, indent=1), "```", ""]
    with open(out_path, "w") as fh:
        fh.write("\n".join(out))
    return "\n".join(out)


def load_traffic(kernel: str, workload: str):
    """The calibrated HBM bytes per launch recorded for `kernel` on `workload`,
    or None when there is no record or the kernel's sources have changed."""
    path = os.path.join(PROFILES, f"hbm_traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        text = fh.read()
    try:
        body = text.split("```json", 1)[1].split("```", 1)[0]
        rec = json.loads(body)
    except (IndexError, ValueError):
        return None
    if rec.get("source_sha256") != source_hash(kernel):
        return None
    return rec


def main(argv):
    if len(argv) >= 6 and argv[0] == "kernels":
        print(kernels_summary(*argv[1:6]))
    elif len(argv) >= 8 and argv[0] == "traffic":
        print(traffic_summary(*argv[1:8]))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
