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
    dkdv = "void dualkv::(anonymous namespace)::bwd_dkdv_kernel<128>(...)"
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
