"""Host-side checks of the rocprofv3 summaries that feed bench.py's roofline."""
import csv
import json
import os

from shared_prompt_exact_amd import profiling

COLS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=COLS)
        wr.writeheader()
        for i, (name, kib) in enumerate(rows, 1):
            wr.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib})


def test_traffic_calibration(tmp_path):
    import workloads
    w = workloads.WORKLOADS["qwen3_8b"]
    copy = w.packed_len * w.n_q_heads * w.head_dim * 2
    rep = "void dualkv::(anonymous namespace)::repack_kernel<uint4>(...)"
    dkdv = "void dualkv::(anonymous namespace)::bwd_dkdv_lean_kernel<128, 8, 3>(...)"
    # the fetch counter reads half of the copy's bytes, the write counter all of them
    _write(tmp_path / "f", "FETCH_SIZE", [(rep, copy / 2048), (dkdv, 1000.0), (dkdv, 1002.0)])
    _write(tmp_path / "w", "WRITE_SIZE", [(rep, copy / 1024), (dkdv, 10.0), (dkdv, 10.0)])
    out = tmp_path / "t.md"
    profiling.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), "bwd_dkdv", "qwen3_8b", str(out), "a", "b")
    rec = json.loads(out.read_text().split("```json", 1)[1].split("```", 1)[0])
    assert abs(rec["fetch_factor"] - 2.0) < 1e-9 and abs(rec["write_factor"] - 1.0) < 1e-9
    assert rec["read_bytes"] == round(1001.0 * 1024 * 2) and rec["write_bytes"] == 10 * 1024
    assert rec["dispatches"] == 2 and rec["source_sha256"] == profiling.source_hash("bwd_dkdv")


def test_load_traffic_tracks_sources(monkeypatch, tmp_path):
    rec = {"kernel": "fwd", "bytes_per_launch": 123, "source_sha256": profiling.source_hash("fwd")}
    (tmp_path / "hbm_traffic_fwd_x.md").write_text("# t\n\n```json\n" + json.dumps(rec) + "\n```\n")
    monkeypatch.setattr(profiling, "PROFILES", str(tmp_path))
    assert profiling.load_traffic("fwd", "x")["bytes_per_launch"] == 123
    assert profiling.load_traffic("fwd", "missing") is None
    monkeypatch.setattr(profiling, "source_hash", lambda k: "changed")
    assert profiling.load_traffic("fwd", "x") is None


def test_committed_records_parse():
    for f in os.listdir(profiling.PROFILES):
        if f.startswith("hbm_traffic_") and f.endswith(".md"):
            text = open(os.path.join(profiling.PROFILES, f)).read()
            rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
            assert rec["bytes_per_launch"] > 0 and rec["kernel"] in profiling.KERNELS


def test_counters_summary(tmp_path):
    fwd = "void dualkv::(anonymous namespace)::fwd_lean_kernel<128, 64, 12, 3>(...)"
    dkdv = "void dualkv::(anonymous namespace)::bwd_dkdv_lean_kernel<128, 8, 3>(...)"
    def put(d, rows):
        os.makedirs(d, exist_ok=True)
        with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
            wr = csv.DictWriter(fh, fieldnames=COLS)
            wr.writeheader()
            for i, (name, c, v) in enumerate(rows, 1):
                wr.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": c, "Counter_Value": v})
    put(tmp_path / "a", [(fwd, "MfmaUtil", 50.0), (fwd, "OccupancyPercent", 37.5), (dkdv, "MfmaUtil", 40.0)])
    put(tmp_path / "b", [(fwd, "SQ_INSTS_MFMA", 100.0), (fwd, "SQ_INSTS_VALU", 600.0),
                         (fwd, "SQ_VALU_MFMA_BUSY_CYCLES", 3200.0), (fwd, "SQ_VALU_MFMA_COEXEC_CYCLES", 800.0)])
    put(tmp_path / "c", [(fwd, "SQ_INSTS_SALU", 200.0)])
    out = tmp_path / "c.md"
    text = profiling.counters_summary(str(out), "t", str(tmp_path / "a"), str(tmp_path / "b"),
                                      str(tmp_path / "c"), "x", "y", "z")
    row = [ln for ln in text.splitlines() if ln.startswith("| fwd |")][0].split("|")
    # MFMA busy 50, co-exec 800/3200, 3 waves per SIMD, (600-100)/100 VALU per MFMA, 2 SALU per MFMA
    assert float(row[3]) == 50.0 and float(row[5]) == 0.25 and float(row[8]) == 3.0
    assert float(row[9]) == 5.0 and float(row[12]) == 2.0
    assert any(ln.startswith("| bwd_dkdv |") for ln in text.splitlines())
