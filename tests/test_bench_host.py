"""bench.py's host-side contract, on the CPU: more than one GPU is refused with a message
(one process, one GPU here), the traffic figure is only reported for the sources the
counters were taken on, and the counter-file reader turns rocprofv3 CSVs into bytes per
launch with the copy calibration."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_tracks_the_kernel_sources(tmp_path, monkeypatch):
    h = bench._source_hash()                            # of the real kernel sources
    d = tmp_path / "profiles"
    d.mkdir()
    (d / "hbm_traffic.json").write_text(json.dumps({"decode_c2": {"source_hash": h, "bytes_per_launch": 123.0}}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "_source_hash", lambda: h)
    assert bench._traffic("decode_c2") == 123.0
    monkeypatch.setattr(bench, "_source_hash", lambda: "0000000000000000")
    assert bench._traffic("decode_c2") is None          # sources changed since the counters
    assert bench._traffic("missing") is None


def _counter_csv(path, rows):
    import csv
    path.mkdir(parents=True)
    with open(path / "c2_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_counter_files_to_bytes_per_launch(tmp_path, monkeypatch):
    """Two passes (FETCH_SIZE, WRITE_SIZE), each with attention launches and a 1 GiB copy
    for calibration: bytes per launch = median counter KiB x 1024 x (copy bytes / copy
    counter bytes)."""
    def rows(counter, attn_kib, copy_kib):
        out = []
        for i, v in enumerate(attn_kib):
            out.append({"Dispatch_Id": i, "Kernel_Name": "void mlafa::(anonymous namespace)::attn_kernel<1, 8, 2, 0, false>(mlafa::AttnArgs)",
                        "Counter_Name": counter, "Counter_Value": v})
        out.append({"Dispatch_Id": 99, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": counter,
                    "Counter_Value": copy_kib})
        return out
    _counter_csv(tmp_path / "f", rows("FETCH_SIZE", [100.0, 110.0, 90.0], 524288.0))
    _counter_csv(tmp_path / "w", rows("WRITE_SIZE", [50.0, 50.0, 60.0], 1048576.0))
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "_source_hash", lambda: "feedfacefeedface")
    bench.write_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "decode_c2")
    d = json.loads((tmp_path / "profiles" / "hbm_traffic.json").read_text())["decode_c2"]
    assert d["source_hash"] == "feedfacefeedface"
    assert d["counters"]["FETCH_SIZE"]["kib_per_launch"] == 100.0
    assert abs(d["counters"]["FETCH_SIZE"]["factor"] - 2.0) < 1e-12
    assert d["counters"]["WRITE_SIZE"]["kib_per_launch"] == 50.0
    assert abs(d["bytes_per_launch"] - (100.0 * 1024 * 2.0 + 50.0 * 1024 * 1.0)) < 1e-6
