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


def test_source_hash_ignores_comments_not_code():
    """The traffic key covers the kernels' code: a comment or layout edit keeps it, any
    change to code (a constant, an operator) changes it."""
    names = ("attn.hip", "compact.hip", "api.hip", "mla_fa_internal.h", "device_common.h")
    src = {f: open(os.path.join(ROOT, "mla_flash_attention_amd", "csrc", f)).read() for f in names}
    h = bench._source_hash(src)
    assert h == bench._source_hash()
    edited = dict(src)
    edited["attn.hip"] = "// a new note\n/* and a\n   block */\n" + src["attn.hip"].replace("\n", "\n\n", 5)
    assert bench._source_hash(edited) == h
    for old, new in (("kRescaleThresh = 8.0f", "kRescaleThresh = 9.0f"), ("x += __builtin_amdgcn", "x -= __builtin_amdgcn")):
        assert old in src["attn.hip"]
        changed = dict(src)
        changed["attn.hip"] = src["attn.hip"].replace(old, new, 1)
        assert bench._source_hash(changed) != h


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


def test_counter_files_per_kernel(tmp_path, monkeypatch):
    """A run with several kernels (the sparse step: compaction, two attention kernels for
    two cache types, merge) is stored per kernel name; no single attention figure is
    made up from two different kernels."""
    names = {"count": "mlafa::(anonymous namespace)::chunk_count_kernel(unsigned short const*)",
             "write": "mlafa::(anonymous namespace)::chunk_write_kernel(unsigned short const*)",
             "bf16": "void mlafa::(anonymous namespace)::attn_kernel<1, 8, 2, 0, true>(mlafa::AttnArgs)",
             "q8": "void mlafa::(anonymous namespace)::attn_kernel<1, 8, 2, 2, true>(mlafa::AttnArgs)",
             "merge": "mlafa::(anonymous namespace)::merge_kernel(int, int, int, float const*)"}

    def rows(counter, kib, copy_kib):
        out = [{"Dispatch_Id": i, "Kernel_Name": names[k], "Counter_Name": counter, "Counter_Value": v}
               for i, (k, v) in enumerate(kib)]
        out.append({"Dispatch_Id": 99, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": counter,
                    "Counter_Value": copy_kib})
        return out
    fetch = [("count", 10.0), ("count", 12.0), ("write", 20.0), ("bf16", 300.0), ("q8", 160.0), ("merge", 400.0)]
    write = [("count", 1.0), ("write", 5.0), ("bf16", 100.0), ("q8", 100.0), ("merge", 8.0), ("merge", 8.0)]
    _counter_csv(tmp_path / "f", rows("FETCH_SIZE", fetch, 524288.0))
    _counter_csv(tmp_path / "w", rows("WRITE_SIZE", write, 1048576.0))
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "_source_hash", lambda: "feedfacefeedface")
    bench.write_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "sparse_c5")
    e = json.loads((tmp_path / "profiles" / "hbm_traffic.json").read_text())["sparse_c5"]
    assert "bytes_per_launch" not in e
    k = e["kernels"]
    assert k[names["count"]] == {"read_bytes": 11.0 * 1024 * 2.0, "write_bytes": 1.0 * 1024}
    assert k[names["q8"]] == {"read_bytes": 160.0 * 1024 * 2.0, "write_bytes": 100.0 * 1024}
    # the sparse bench line takes its own cache type's attention kernel
    t = bench._traffic_by_kernel("sparse_c5")
    assert t == k
    monkeypatch.setattr(bench, "_source_hash", lambda: "0000000000000000")
    assert bench._traffic_by_kernel("sparse_c5") is None


def test_sparse_line_reports_measured_traffic(monkeypatch):
    from mla_flash_attention_amd import synth
    p = synth.make_problem(kind="sparse", n_seq=1, n_head=128, n_kv=4096, kv_type=synth.TYPE_Q8_0, seed=5)
    t = {"x::chunk_count_kernel(a)": {"read_bytes": 10.0, "write_bytes": 1.0},
         "x::chunk_write_kernel(a)": {"read_bytes": 20.0, "write_bytes": 2.0},
         "void x::attn_kernel<1, 8, 2, 0, true>(a)": {"read_bytes": 300.0, "write_bytes": 30.0},
         "void x::attn_kernel<1, 8, 2, 2, true>(a)": {"read_bytes": 400.0, "write_bytes": 40.0},
         "x::merge_kernel(a)": {"read_bytes": 50.0, "write_bytes": 5.0}}
    monkeypatch.setattr(bench, "_traffic_by_kernel", lambda key: t if key == "sparse_c5" else None)
    r = dict(kept=400, n_split=16, step_ms=0.03, compact_ms=0.007, part_ms=0.02, merge_ms=0.005)
    line = bench._sparse_line(p, r)
    assert line["traffic"] == {"compaction": 33.0, "attention": 440.0, "merge": 55.0}
    assert line["partial_bytes"] == 16 * 128 * 1040
    monkeypatch.setattr(bench, "_traffic_by_kernel", lambda key: None)
    assert bench._sparse_line(p, r)["traffic"] is None
