"""Summaries of rocprofv3 output for this library's kernels.

Two summaries, both written as short markdown under ``profiles/``:

* ``kernels``: a ``rocprofv3 --kernel-trace --stats --output-format csv`` run
  of ``bench.py`` -> per-kernel call counts and durations, next to the
  library's own event timings printed by the same run (its JSON line).
* ``counters``: three ``rocprofv3 --pmc`` runs of bench.py (the counter sets
  PASSES below, each within one run's hardware limits) -> per kernel the
  matrix-core and vector-ALU busy fractions, how much of the matrix-core
  busy time also issued vector instructions (co-execution), LDS activity
  and bank conflicts, occupancy, and instruction counts per MFMA.
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
  python3 -m shared_prompt_exact_amd.profiling counters OUT.md TITLE DIR_A DIR_B DIR_C CMD_A CMD_B CMD_C
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

# library kernel name -> (substrings of the device symbols, source files they are built from)
_HEADERS = ["common.h", "mfma_common.h", "lds_tiles.h"]
KERNELS = {
    "fwd": (("fwd_lean_kernel",), ["attn_fwd_mfma.hip"] + _HEADERS),
    "bwd_dq": (("bwd_dq_kernel", "bwd_dq_wide_kernel"), ["attn_bwd_dq.hip", "attn_bwd_dq_wide.hip"] + _HEADERS),
    "bwd_dkdv": (("bwd_dkdv_lean_kernel", "bwd_dkdv_wide_kernel"),
                 ["attn_bwd_mfma.hip", "attn_bwd_dkdv_wide.hip", "kv_items.h"] + _HEADERS),
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
    for k, (subs, _) in KERNELS.items():
        for sub in (subs if isinstance(subs, tuple) else (subs,)):
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


# Counter sets of the ``counters`` summary, one rocprofv3 --pmc run each.
# A: rocprofv3's derived metrics (their formulas as `rocprofv3 -L` lists
#    them on MI355X): MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE
#    x SIMDs); VALUBusy = SQ_ACTIVE_INST_VALU / (CUs x GRBM_GUI_ACTIVE);
#    LdsUtil = SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE x CUs); LDSBankConflict =
#    SQ_LDS_BANK_CONFLICT / GRBM_GUI_ACTIVE / CUs; OccupancyPercent = 400 x
#    SQ_WAVE_CYCLES / GRBM_GUI_ACTIVE / CUs / 32 (of 32 waves per CU).
# B, C: raw SQ counters, used as ratios (per MFMA instruction, or co-issue
#    cycles over matrix-core busy cycles).
PASSES = {
    "A": ["MfmaUtil", "VALUBusy", "LdsUtil", "LDSBankConflict", "OccupancyPercent"],
    "B": ["SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
          "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS", "SQ_INSTS_VALU_TRANS_F32", "SQ_ACTIVE_INST_VALU", "GRBM_GUI_ACTIVE"],
    "C": ["SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_MISC",
          "SQ_INSTS_SALU", "SQ_ACTIVE_INST_VALU2", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"],
}


def _counter_means(d: str) -> dict:
    """kernel short name -> symbol, counter -> mean over the kernel's dispatches."""
    acc: dict = {}
    for r in _csv(d, "counter_collection.csv"):
        k = short_name(r["Kernel_Name"])
        sym = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").replace(
            "dualkv::", "")
        e = acc.setdefault(k, {"symbol": sym, "vals": {}})
        e["vals"].setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: {"symbol": e["symbol"], **{c: sum(v) / len(v) for c, v in e["vals"].items()}}
            for k, e in acc.items()}


def counters_summary(out_path, title, dir_a, dir_b, dir_c, cmd_a, cmd_b, cmd_c):
    merged: dict = {}
    for d in (dir_a, dir_b, dir_c):
        for k, vals in _counter_means(d).items():
            merged.setdefault(k, {}).update(vals)
    rows = []
    for k in ("fwd", "bwd_dq", "bwd_dkdv", "bwd_delta", "bwd_reduce", "gemm"):
        if k not in merged:
            continue
        m = merged[k]
        mf = max(m.get("SQ_INSTS_MFMA", 0.0), 1.0)
        busy = max(m.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0), 1.0)
        rows.append((k, m["symbol"], m.get("MfmaUtil", float("nan")), m.get("VALUBusy", float("nan")),
                     m.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) / busy, m.get("LdsUtil", float("nan")),
                     m.get("LDSBankConflict", float("nan")), m.get("OccupancyPercent", float("nan")) * 8 / 100,
                     (m.get("SQ_INSTS_VALU", 0.0) - m.get("SQ_INSTS_MFMA", 0.0)) / mf,
                     m.get("SQ_INSTS_VALU_TRANS_F32", 0.0) / mf, m.get("SQ_INSTS_LDS", 0.0) / mf,
                     m.get("SQ_INSTS_SALU", 0.0) / mf))
    out = [f"# {title}", "", "Commands (repo root, MI355X), one counter set per run:", "",
           "    " + cmd_a, "    " + cmd_b, "    " + cmd_c, "",
           "Per kernel, means over its dispatches in the profiled steps.  MFMA and VALU busy are % of the "
           "kernel's cycles on all SIMDs; co-exec is the share of matrix-core busy cycles in which a "
           "vector instruction also issued; waves/SIMD is the mean occupancy; the last columns are "
           "instructions per MFMA instruction (VALU excluding MFMA, of them transcendental, LDS, scalar).",
           "",
           "| kernel | symbol | MFMA busy % | VALU busy % | co-exec | LDS busy % | LDS bank conflict % | "
           "waves/SIMD | VALU/MFMA | trans/MFMA | LDS/MFMA | SALU/MFMA |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {r[0]} | `{r[1]}` | {r[2]:.1f} | {r[3]:.1f} | {r[4]:.3f} | {r[5]:.1f} | {r[6]:.2f} | "
                   f"{r[7]:.2f} | {r[8]:.2f} | {r[9]:.2f} | {r[10]:.2f} | {r[11]:.2f} |")
    out += ["", "```json", json.dumps({k: {c: v for c, v in merged[k].items()} for k in merged if k != "other"},
                                      indent=1, sort_keys=True), "```", ""]
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
    elif len(argv) >= 9 and argv[0] == "counters":
        print(counters_summary(*argv[1:9]))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
