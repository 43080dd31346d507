"""Benchmark: MLA flash-attention decode over the latent cache on one MI355X.

Headline workload: 4 sequences x 1 query token x 128 heads, each with its own latent
cache of 32768 rows x 576 bf16 (DeepSeek-V3 head count), split-KV with a partial
(m, l, O) merge.  A step is one mla_fa_decode call (split attention + merge) with
every input already resident in HBM.  Timed steps rotate over 4 copies of the inputs
(4 x 151 MB, more than the 256 MB last-level cache) so every step reads the cache from
HBM.  Prints one JSON line (see the repository's bench contract).

Secondary lines (same JSON object, key "secondary"): the other workloads - 16-head
f16 decode (warm, and cold: caches flushed before each call), 2048-token causal prefill, Q8_0 decode, sparse decode at 131072 cells (bf16 warm and cold, Q8_0 warm),
ragged 2-token decode, per-head (DK=192 / DV=128) prefill, and decode with the absorbed
W_UK / W_UV projections either side.

Every timed loop follows W warm-up calls and at least 0.1 s of warm-up load in total
("warmup_min_seconds"): the GPU reaches its steady clock only after tens of
milliseconds of load.

Key "measured_peaks": what this GPU measurably delivers (HBM stream read, dense bf16
MFMA issue, LDS reads; include/mla_peaks.h), so each roofline fraction is also stated
against a measured peak ("frac_measured", "mfma_frac_measured") beside the published one.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16/f16 MFMA, published
ROW_BYTES = {1: 1152, 2: 1152, 3: 612}
METRIC = "MLA FA latent KV cells/s per GPU + % of HBM / MFMA roofline"


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=4, help="rotating input copies (cold cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak micro-benchmarks")
    ap.add_argument("--only", default="",
                    help="run only these workloads, e.g. 'c2' or 'c3,c4' ('peaks' alone: only the measured peaks)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this script with "
                         "--copy-calibration into profiles/hbm_traffic.json and exit")
    ap.add_argument("--traffic-key", default="decode_c2",
                    help="workload the --traffic-from runs timed (decode_c2, decode_c4_q8_0, sparse_c5)")
    return ap.parse_args()


def _counter_rows(d):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def write_traffic(fetch_dir, write_dir, key):
    """HBM bytes per launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by
    what the same counter reads for a 1 GiB device copy (copy reads 1 GiB and writes
    1 GiB); stored under `key` (the workload the two counter runs timed) in
    profiles/hbm_traffic.json: per kernel name (medians over its dispatches), and at the
    top level for the attention kernel when the runs launched exactly one."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    out = {}
    if os.path.exists(path):
        with open(path) as f:
            out = json.load(f)
    per, kernels = {}, {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(d) if r["Counter_Name"] == name]
        is_copy = lambda n: "copy" in n.lower() or "elementwise" in n.lower()
        copy = [float(r["Counter_Value"]) for r in rows if is_copy(r["Kernel_Name"])]
        copy = [c for c in copy if c > 1e5]          # the 1 GiB copy, not small fills
        if not copy:
            raise SystemExit(f"{name}: no calibration copy in {d}")
        factor = (1 << 30) / (max(copy) * 1024.0)    # bytes per counted KiB
        by_kernel = {}
        for r in rows:
            if not is_copy(r["Kernel_Name"]):
                by_kernel.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        field = "read_bytes" if name == "FETCH_SIZE" else "write_bytes"
        for kn, v in by_kernel.items():
            kernels.setdefault(kn, {})[field] = float(np.median(v)) * 1024.0 * factor
        attn = [kn for kn in by_kernel if "attn_kernel" in kn]
        if len(attn) == 1:
            kib = float(np.median(by_kernel[attn[0]]))
            per[name] = dict(kib_per_launch=kib, copy_kib=max(copy), factor=factor, bytes_per_launch=kib * 1024.0 * factor)
    entry = dict(source_hash=_source_hash(), kernels=kernels)
    if len(per) == 2:
        entry.update(bytes_per_launch=per["FETCH_SIZE"]["bytes_per_launch"] + per["WRITE_SIZE"]["bytes_per_launch"],
                     read_bytes=per["FETCH_SIZE"]["bytes_per_launch"],
                     write_bytes=per["WRITE_SIZE"]["bytes_per_launch"], counters=per)
    out[key] = entry
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out[key], indent=1))


def _dev(a):
    import torch
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def _code_only(text):
    """C++ source without its comments and with runs of whitespace collapsed, so that an
    edit to comments alone leaves the hash (and the measurements keyed by it) valid.
    (These sources hold no string literal with a comment marker in it.)"""
    return " ".join(_COMMENT.sub(" ", text).split())


def _source_hash(files=None):
    """Hash of the code (comments and layout aside) of the sources that decide the
    split-attention kernels and their launches."""
    h = hashlib.sha256()
    for f in ("attn.hip", "compact.hip", "api.hip", "mla_fa_internal.h", "device_common.h"):
        if files is None:
            with open(os.path.join(ROOT, "mla_flash_attention_amd", "csrc", f)) as fh:
                text = fh.read()
        else:
            text = files[f]
        h.update(_code_only(text).encode())
    return h.hexdigest()[:16]


def _traffic(kernel_key):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/), or None when the
    counters are missing or were taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    e = d.get(kernel_key)
    if not e or e.get("source_hash") != _source_hash():
        return None
    return e.get("bytes_per_launch")


def _traffic_by_kernel(key):
    """{kernel name: {read_bytes, write_bytes}} measured for workload `key`, or None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        e = json.load(f).get(key)
    if not e or e.get("source_hash") != _source_hash():
        return None
    return e.get("kernels")


WARM_FLOOR_S = 0.1   # minimum warm-up time before every timed loop


def _warm(fn, warmup):
    """`warmup` untimed calls fn(0 .. warmup-1), then more until at least WARM_FLOOR_S
    has passed: the GPU needs tens of milliseconds of load to reach its steady clock (the
    C2 step measured ~70 us in its first ~10 ms of load and ~60 us from ~50 ms on)."""
    import torch
    t = time.perf_counter()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    n = warmup
    while time.perf_counter() - t < WARM_FLOOR_S:
        for _ in range(8):
            fn(n)
            n += 1
        torch.cuda.synchronize()


def _time_decode(B, p, copies, steps, warmup, n_split=0):
    """Per-call times on the launch stream.  step: the one-call API (compaction first on the
    sparse path, then attention and merge) repeated back to back between two events;
    kernel, merge and compaction: that launch alone repeated back to back (what a
    kernel-trace profiler averages).  Inputs rotate over `copies` distinct copies.  The
    p10/p90 spread of the attention kernel comes from events around single launches."""
    import torch
    from mla_flash_attention_amd import synth
    stream = torch.cuda.current_stream()
    qs, kvs = [], []
    for c in range(copies):
        qs.append(_dev(p.q.reshape(p.n_seq, p.n_head, synth.DK)))
        kvs.append(_dev(p.kv))
    mask = None if p.mask is None else _dev(p.mask.reshape(p.n_seq, p.n_kv))
    out = torch.empty((p.n_seq, p.n_head, synth.DV), dtype=torch.float32, device="cuda")
    ns = n_split or B.mla_fa_auto_splits(p.n_seq, p.n_head, p.n_kv, p.kv_type)
    ws = B.workspace_for(p.n_seq, p.n_head, p.n_kv, p.kv_type, ns)
    sparse = p.kind == "sparse"
    idx = cnt = None
    if sparse:
        idx = torch.empty((p.n_seq, p.n_kv), dtype=torch.int32, device="cuda")
        cnt = torch.empty((p.n_seq,), dtype=torch.int32, device="cuda")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)

    def timed(fn):
        _warm(fn, warmup)
        t0.record(stream)
        for i in range(steps):
            fn(i)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    cws = None
    if sparse:      # the multi-workgroup compaction's chunk counts
        cws = torch.empty(max(B.fa_mask_compact_workspace_size(p.n_seq, p.n_kv), 1), dtype=torch.uint8,
                          device="cuda")

    def compact(i):
        B.fa_mask_compact_ws(mask, idx, cnt, cws, stream=stream)

    def part(i):
        c = i % copies
        B.mla_fa_decode_partials(qs[c], p.q_type, kvs[c], p.kv_type, p.scale, out, mask=mask, kv_idx=idx,
                                 kv_idx_count=cnt, n_split=ns, workspace=ws, stream=stream)

    def merge(i):
        B.mla_fa_merge_partials(p.n_seq, p.n_head, ns, out, ws, stream=stream)

    def call(i):
        if sparse:
            compact(i)
        c = i % copies
        B.mla_fa_decode(qs[c], p.q_type, kvs[c], p.kv_type, p.scale, out, mask=mask, kv_idx=idx,
                        kv_idx_count=cnt, n_split=ns, workspace=ws, stream=stream)

    compact_ms = timed(compact) if sparse else None
    part_ms = timed(part)
    merge_ms = timed(merge) if ns > 1 else 0.0
    step_ms = timed(call)
    single = []
    for i in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        part(i)
        e1.record(stream)
        single.append((e0, e1))
    torch.cuda.synchronize()
    single_ms = [a.elapsed_time(b) for a, b in single]
    kept = int(cnt.cpu()[0]) if sparse else None
    return dict(total_ms=step_ms * steps, step_ms=step_ms, part_ms=part_ms,
                part_ms_p10=float(np.percentile(single_ms, 10)), part_ms_p90=float(np.percentile(single_ms, 90)),
                merge_ms=merge_ms, compact_ms=compact_ms, n_split=ns, kept=kept)


def _time_decode_cold(B, p, calls=30):
    """One-call decode (compaction first on the sparse path) with the caches cold: before
    every call an untimed 512 MB write evicts the 256 MB last-level cache; each call is
    timed alone between events on the launch stream.  Returns the median, p10 and p90."""
    import torch
    from mla_flash_attention_amd import synth
    stream = torch.cuda.current_stream()
    q = _dev(p.q.reshape(p.n_seq, p.n_head, synth.DK))
    kv = _dev(p.kv)
    mask = None if p.mask is None else _dev(p.mask.reshape(p.n_seq, p.n_kv))
    out = torch.empty((p.n_seq, p.n_head, synth.DV), dtype=torch.float32, device="cuda")
    ns = B.mla_fa_auto_splits(p.n_seq, p.n_head, p.n_kv, p.kv_type)
    ws = B.workspace_for(p.n_seq, p.n_head, p.n_kv, p.kv_type, ns)
    sparse = p.kind == "sparse"
    idx = torch.empty((p.n_seq, p.n_kv), dtype=torch.int32, device="cuda") if sparse else None
    cnt = torch.empty((p.n_seq,), dtype=torch.int32, device="cuda") if sparse else None
    cws = None
    if sparse:
        cws = torch.empty(max(B.fa_mask_compact_workspace_size(p.n_seq, p.n_kv), 1), dtype=torch.uint8,
                          device="cuda")
    flush = torch.empty(128 << 20, dtype=torch.float32, device="cuda")     # 512 MB

    def call():
        if sparse:
            B.fa_mask_compact_ws(mask, idx, cnt, cws, stream=stream)
        B.mla_fa_decode(q, p.q_type, kv, p.kv_type, p.scale, out, mask=mask, kv_idx=idx, kv_idx_count=cnt,
                        n_split=ns, workspace=ws, stream=stream)

    _warm(lambda i: call(), 3)
    evs = []
    for i in range(calls):
        flush.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    return dict(ms=float(np.median(ms)), p10=float(np.percentile(ms, 10)), p90=float(np.percentile(ms, 90)))


def _time_attend(B, p, steps, warmup, n_split=0):
    """Back-to-back mla_fa_attend calls (attention + merge) between two events."""
    import torch
    stream = torch.cuda.current_stream()
    q = _dev(p.q)
    kv = _dev(p.kv)
    out = torch.empty((p.n_seq, p.n_tok, p.n_head, 512), dtype=torch.float32, device="cuda")
    mask = None if p.mask is None else _dev(p.mask)
    f = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kv_len, alibi, sinks = f(p.kv_len), f(p.alibi), f(p.sinks)
    ns = n_split or B.mla_fa_auto_splits(p.n_seq * p.n_tok, p.n_head, p.n_kv, p.kv_type)
    ws = B.workspace_for(p.n_seq * p.n_tok, p.n_head, p.n_kv, p.kv_type, ns)

    def call():
        B.mla_fa_attend(q, p.q_type, kv, p.kv_type, p.scale, out, kv_len=kv_len, causal=p.causal, mask=mask,
                        alibi=alibi, sinks=sinks, softcap=p.softcap, n_split=ns, workspace=ws, stream=stream)

    _warm(lambda i: call(), warmup)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        call()
    t1.record(stream)
    torch.cuda.synchronize()
    return dict(step_ms=t0.elapsed_time(t1) / steps, n_split=ns)


def _time_prefill(B, p, steps, warmup):
    import torch
    from mla_flash_attention_amd import synth
    stream = torch.cuda.current_stream()
    q = _dev(p.q.reshape(p.n_tok, p.n_head, synth.DK))
    kv = _dev(p.kv.reshape(p.n_kv, -1))
    out = torch.empty((p.n_tok, p.n_head, synth.DV), dtype=torch.float32, device="cuda")
    _warm(lambda i: B.mla_fa_prefill(q, p.q_type, kv, p.kv_type, p.scale, out, causal=True, n_split=1,
                                     stream=stream), warmup)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        B.mla_fa_prefill(q, p.q_type, kv, p.kv_type, p.scale, out, causal=True, n_split=1, stream=stream)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[1]) for e in evs]
    return dict(step_ms=float(np.mean(ms)), p10=float(np.percentile(ms, 10)), p90=float(np.percentile(ms, 90)))


def _time_mha(B, p, steps, warmup):
    """Back-to-back mla_fa_prefill_mha calls between two events, and single-launch p10/p90."""
    import torch
    stream = torch.cuda.current_stream()
    q, k, v = _dev(p.q), _dev(p.k), _dev(p.v)
    out = torch.empty((p.n_tok, p.n_head, 128), dtype=torch.float32, device="cuda")

    def call():
        B.mla_fa_prefill_mha(q, p.q_type, k, v, p.kv_type, p.scale, out, causal=p.causal, stream=stream)

    _warm(lambda i: call(), warmup)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        call()
        evs[i][1].record(stream)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        call()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[1]) for e in evs]
    return dict(step_ms=t0.elapsed_time(t1) / steps, p10=float(np.percentile(ms, 10)),
                p90=float(np.percentile(ms, 90)))


def _time_absorbed(B, p, steps, warmup):
    """Back-to-back mla_fa_absorbed calls (query projection, attention, merge, output
    projection) between two events."""
    import torch
    stream = torch.cuda.current_stream()
    qn, qp, wk, wv, kv = _dev(p.q_nope), _dev(p.q_pe), _dev(p.w_uk), _dev(p.w_uv), _dev(p.kv)
    out = torch.empty((p.n_seq, p.n_tok, p.n_head, 128), dtype=torch.float32, device="cuda")
    ns = B.mla_fa_auto_splits(p.n_seq * p.n_tok, p.n_head, p.n_kv, p.kv_type)
    ws = B.absorbed_workspace_for(p.n_seq * p.n_tok, p.n_head, p.n_kv, p.kv_type, ns)
    kv_len = None if p.kv_len is None else _dev(p.kv_len)

    def call():
        B.mla_fa_absorbed(qn, qp, p.q_type, wk, wv, kv, p.kv_type, p.scale, out, kv_len=kv_len, causal=p.causal,
                          n_split=ns, workspace=ws, stream=stream)

    _warm(lambda i: call(), warmup)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        call()
    t1.record(stream)
    torch.cuda.synchronize()
    return dict(step_ms=t0.elapsed_time(t1) / steps, n_split=ns)


def _algo_decode(p, kept=None):
    """Algorithmic bytes and flops of one decode call: cache rows attended, Q, O (and the
    mask/index traffic of the sparse path); flops 2*H*(576+512) per attended cell."""
    cells = p.n_seq * (kept if kept is not None else p.n_kv)
    row = ROW_BYTES[p.kv_type]
    qb = p.n_seq * p.n_head * 576 * 2
    ob = p.n_seq * p.n_head * 512 * 4
    kernel_bytes = cells * row + qb                      # what the attention kernel must read
    call_bytes = kernel_bytes + ob
    if kept is not None:
        call_bytes += 2 * p.n_kv * p.n_seq + (4 + 4 + 2) * cells
    flops = cells * 2 * p.n_head * (576 + 512)
    return cells, kernel_bytes, call_bytes, flops


def _sparse_line(p, r):
    """The sparse decode step and its three launches, each with its HBM fraction:
    compaction (2 B of mask read per scanned cell, 4 B of index written per kept cell),
    attention (kept rows + Q), merge (the split partials read, the output written)."""
    kept, ns = r["kept"], r["n_split"]
    cells, kb, cb, fl = _algo_decode(p, kept=kept)
    partial_bytes = ns * p.n_seq * p.n_head * (16 + 512 * 2)
    compact_bytes = 2 * p.n_kv * p.n_seq + 4 * cells + 4 * p.n_seq
    merge_bytes = partial_bytes + p.n_seq * p.n_head * 512 * 4
    frac = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
    # HBM bytes per launch measured with rocprofv3 counters (profiles/hbm_traffic.json,
    # the same seeded workload), when taken on the current kernel sources
    traffic = None
    t = _traffic_by_kernel("sparse_c5")
    if t:
        from mla_flash_attention_amd import synth
        kind = {synth.TYPE_BF16: 0, synth.TYPE_F16: 1, synth.TYPE_Q8_0: 2}[p.kv_type]   # template argument

        def measured(match):
            m = [v for k, v in t.items() if match(k)]
            return m[0].get("read_bytes", 0.0) + m[0].get("write_bytes", 0.0) if len(m) == 1 else None
        cnt, wr = measured(lambda k: "chunk_count_kernel" in k), measured(lambda k: "chunk_write_kernel" in k)
        traffic = {"compaction": cnt + wr if cnt is not None and wr is not None else None,
                   "attention": measured(lambda k: "attn_kernel" in k and f", {kind}, true>" in k),
                   "merge": measured(lambda k: "merge_kernel" in k)}
    return dict(ms=r["step_ms"], compact_ms=r["compact_ms"], compaction="fa_mask_compact_ws (4096-cell chunks)",
                attn_ms=r["part_ms"], merge_ms=r["merge_ms"], kept=kept, n_split=ns,
                kept_row_bytes=cells * ROW_BYTES[p.kv_type], partial_bytes=partial_bytes,
                scanned_cells_per_s=p.n_kv / (r["step_ms"] * 1e-3),
                kept_cells_per_s=kept / (r["step_ms"] * 1e-3),
                hbm_frac={"compaction": frac(compact_bytes, r["compact_ms"]), "attention": frac(kb, r["part_ms"]),
                          "merge": frac(merge_bytes, r["merge_ms"]) if r["merge_ms"] else None,
                          "step": frac(cb, r["step_ms"])},
                algorithmic_bytes={"compaction": compact_bytes, "attention": kb, "merge": merge_bytes},
                traffic=traffic)


def _measured_peaks(torch, reps=5):
    """What this GPU measurably delivers (libmlapeaks, include/mla_peaks.h): HBM stream
    read of 4 GiB (past the 256 MB last-level cache), dense bf16 MFMA issue, and LDS
    reads (ds_read_b128 and the ds_read_b64_tr_b16 transpose read).  Best of `reps`
    launches at each of a few grid sizes, timed with events on the launch stream."""
    from mla_flash_attention_amd import peaks as P
    P.lib()

    def best_ms(fn):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        fn()
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return min(a.elapsed_time(b) for a, b in ev)

    out = {}
    nbytes = 4 << 30
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    out["hbm_read_gbs"] = max(nbytes / (best_ms(lambda: P.hbm_read(buf, sink, n)) * 1e-3) / 1e9
                              for n in (2048, 4096, 8192))
    del buf
    fsink = torch.zeros(2048 * P.THREADS, dtype=torch.float32, device="cuda")
    iters = 4096
    out["mfma_bf16_tflops"] = max(
        n * 4 * iters * 8 * P.MFMA_FLOPS / (best_ms(lambda: P.mfma_bf16(iters, 2.0 ** -10, fsink, n)) * 1e-3) / 1e12
        for n in (512, 1024, 2048))
    lds_iters = 8192
    for tag, tr in (("lds_b128_gbs", False), ("lds_tr16_gbs", True)):
        out[tag] = max(n * 4 * lds_iters * P.LDS_STEP_BYTES /
                       (best_ms(lambda: P.lds_read(lds_iters, tr, sink, n)) * 1e-3) / 1e9 for n in (512, 1024))
    out["lds_b128_bytes_per_cu_clk_at_2p4ghz"] = out["lds_b128_gbs"] * 1e9 / (256 * 2.4e9)
    out["lds_tr16_bytes_per_cu_clk_at_2p4ghz"] = out["lds_tr16_gbs"] * 1e9 / (256 * 2.4e9)
    return out


def _cpu_baseline(p, limit_s=40.0):
    """The fp64 oracle on the host cores over the full workload (it finishes in seconds
    there); cells/s."""
    import oracle
    t0 = time.perf_counter()
    oracle.attention_problem(p)
    dt = time.perf_counter() - t0
    return dict(value=p.n_seq * p.n_kv / dt, unit="cells/s", cores=oracle.num_threads(), kind="oracle",
                sample=f"the whole workload ({p.n_seq} seq x {p.n_kv} cells x {p.n_head} heads, fp64), "
                       f"{dt:.2f} s wall", seconds=round(dt, 3))


def main():
    args = _args()
    if args.traffic_from:
        write_traffic(*args.traffic_from, args.traffic_key)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(sharding across GPUs is a design only; this benchmark runs on one GPU)", file=sys.stderr)
        sys.exit(2)
    import torch
    from mla_flash_attention_amd import binding as B
    from mla_flash_attention_amd import synth
    B.lib()
    only = set(x.strip().lower() for x in args.only.split(",") if x.strip())
    want = lambda k: not only or k in only

    peaks = None if args.no_peaks else _measured_peaks(torch)
    mfma_meas = peaks["mfma_bf16_tflops"] if peaks else None
    result = {}
    if want("c2"):
        p2 = synth.make_config(2)
        r = _time_decode(B, p2, args.copies, args.steps, args.warmup)
        cells, kbytes, cbytes, flops = _algo_decode(p2)
        value = cells / (r["step_ms"] * 1e-3)
        achieved = kbytes / (r["part_ms"] * 1e-3) / 1e9
        result = {
            "metric": METRIC, "value": value, "unit": "cells/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "warmup_min_seconds": WARM_FLOOR_S,
            "ms_per_step": r["step_ms"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic: seeded N(0,1) rounded to bf16, DeepSeek-V3 MLA shapes",
            "config": {"workload": "MLA decode, 4 seq x 1 token x 128 heads, latent cache n_kv=32768 x 576 bf16 "
                                   "per sequence, split-KV + merge", "n_seq": 4, "n_head": 128,
                       "n_kv": 32768, "n_split": r["n_split"], "input_copies": args.copies},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": _traffic("decode_c2"),
                         "kernel": "attn_kernel (split attention)", "kernel_ms": r["part_ms"],
                         "kernel_ms_p10": r["part_ms_p10"], "kernel_ms_p90": r["part_ms_p90"],
                         "algorithmic_bytes": kbytes, "merge_ms": r["merge_ms"],
                         "mfma_tflops": flops / (r["part_ms"] * 1e-3) / 1e12,
                         "mfma_frac": flops / (r["part_ms"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                         "call_frac_hbm": cbytes / (r["step_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS},
        }
        if peaks:
            rf = result["roofline"]
            rf["peak_measured"] = peaks["hbm_read_gbs"]
            rf["frac_measured"] = achieved / peaks["hbm_read_gbs"]
            rf["mfma_frac_measured"] = rf["mfma_tflops"] / mfma_meas
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = _cpu_baseline(p2)
    sec = {}
    if not args.no_secondary:
        if want("c1"):
            p = synth.make_config(1)
            r = _time_decode(B, p, 1, args.steps, args.warmup)
            cells, kb, cb, fl = _algo_decode(p)
            sec["c1_decode_16h_f16_warm"] = dict(ms=r["step_ms"], cells_per_s=cells / (r["step_ms"] * 1e-3),
                                                 kernel_ms=r["part_ms"], n_split=r["n_split"])
            rc = _time_decode_cold(B, p)
            sec["c1_decode_16h_f16_cold"] = dict(ms=rc["ms"], p10=rc["p10"], p90=rc["p90"],
                                                 cells_per_s=cells / (rc["ms"] * 1e-3))
        if want("c3"):
            p = synth.make_config(3)
            r = _time_prefill(B, p, max(5, args.steps // 5), max(2, args.warmup // 5))
            pairs = sum(p.n_kv - p.n_tok + t + 1 for t in range(p.n_tok))
            fl = pairs * 2 * p.n_head * (576 + 512)
            tf = fl / (r["step_ms"] * 1e-3) / 1e12
            sec["c3_prefill_2048x128h_causal"] = dict(ms=r["step_ms"], p10=r["p10"], p90=r["p90"],
                                                      cells_per_s=pairs / (r["step_ms"] * 1e-3), tflops=tf,
                                                      mfma_frac=tf / MFMA_BF16_PEAK_TFLOPS, bound="mfma",
                                                      mfma_frac_measured=tf / mfma_meas if peaks else None)
        if want("n2"):
            # non-absorbed MLA prefill: per-head 192-wide keys, 128-wide values, the C3 chunk shape
            p = synth.make_mha_problem(2048, 128, 4096, synth.TYPE_BF16, synth.TYPE_BF16, seed=3, causal=True)
            r = _time_mha(B, p, max(5, args.steps // 5), max(2, args.warmup // 5))
            pairs = sum(p.n_kv - p.n_tok + t + 1 for t in range(p.n_tok))
            fl = pairs * 2 * p.n_head * (192 + 128)
            tf = fl / (r["step_ms"] * 1e-3) / 1e12
            sec["n2_prefill_mha_2048x128h_causal"] = dict(ms=r["step_ms"], p10=r["p10"], p90=r["p90"],
                                                          cells_per_s=pairs / (r["step_ms"] * 1e-3), tflops=tf,
                                                          mfma_frac=tf / MFMA_BF16_PEAK_TFLOPS, bound="mfma",
                                                          mfma_frac_measured=tf / mfma_meas if peaks else None)
        if want("n4"):
            # absorbed projections either side of the decode workload's attention: 4 sequences x
            # 128 heads over 32768-cell bf16 caches, plus W_UK / W_UV (16 MiB each)
            p = synth.make_absorbed_problem(4, 1, 128, 32768, synth.TYPE_BF16, synth.TYPE_BF16, seed=2)
            r = _time_absorbed(B, p, args.steps, args.warmup)
            cells = p.n_seq * p.n_kv
            nbytes = cells * 1152 + 2 * p.n_head * 512 * 128 * 2
            sec["n4_absorbed_decode_4x128h_32768"] = dict(
                ms=r["step_ms"], cells_per_s=cells / (r["step_ms"] * 1e-3), n_split=r["n_split"],
                algorithmic_bytes=nbytes, hbm_frac=nbytes / (r["step_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS)
            # the same projections over the ragged 2-token batch of the n3 lines (8 sequences
            # of U{2..32768} valid cells, causal): the serving shape of absorbed decode
            p = synth.make_absorbed_problem(8, 2, 128, 32768, synth.TYPE_BF16, synth.TYPE_BF16, seed=6, causal=True,
                                            ragged=True)
            r = _time_absorbed(B, p, args.steps, args.warmup)
            lens = p.kv_len.astype(np.int64)
            cells = int(sum(L - p.n_tok + t + 1 for L in lens for t in range(p.n_tok)))
            nbytes = int(lens.sum()) * 1152 + 2 * p.n_head * 512 * 128 * 2
            sec["n4_absorbed_ragged_2tok_8x128h"] = dict(
                ms=r["step_ms"], cells_per_s=cells / (r["step_ms"] * 1e-3), n_split=r["n_split"],
                algorithmic_bytes=nbytes, hbm_frac=nbytes / (r["step_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS)
        if want("c4"):
            p = synth.make_config(4)
            r = _time_decode(B, p, args.copies, args.steps, args.warmup)
            cells, kb, cb, fl = _algo_decode(p)
            tf = fl / (r["part_ms"] * 1e-3) / 1e12
            # the Q8_0 kernel computes with f16 MFMA operands: its bound is the f16 peak
            # (the same 2.5 PFLOP/s dense as bf16); HBM is the secondary fraction
            sec["c4_decode_q8_0"] = dict(ms=r["step_ms"], cells_per_s=cells / (r["step_ms"] * 1e-3),
                                         kernel_ms=r["part_ms"], merge_ms=r["merge_ms"], n_split=r["n_split"],
                                         hbm_frac=kb / (r["part_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                                         roofline={"bound": "mfma", "achieved": tf, "peak": MFMA_BF16_PEAK_TFLOPS,
                                                   "unit": "TFLOP/s", "frac": tf / MFMA_BF16_PEAK_TFLOPS,
                                                   "traffic": _traffic("decode_c4_q8_0"),
                                                   "kernel": "attn_kernel (Q8_0, split attention)",
                                                   "algorithmic_flops": fl, "algorithmic_bytes": kb})
        for tag, kvt in (("c5_sparse_131072_cells", synth.TYPE_BF16), ("c5_q8_0_sparse_131072_cells", synth.TYPE_Q8_0)):
            if not want("c5"):
                break
            p = synth.make_config(5, kv_type=kvt)
            r = _time_decode(B, p, 1, args.steps, args.warmup)
            sec[tag] = _sparse_line(p, r)
            if kvt != synth.TYPE_BF16:
                continue
            rc = _time_decode_cold(B, p)
            sec["c5_sparse_131072_cells_cold"] = dict(ms=rc["ms"], p10=rc["p10"], p90=rc["p90"],
                                                      scanned_cells_per_s=p.n_kv / (rc["ms"] * 1e-3))
        if want("n3"):
            # ragged multi-token decode: 8 sequences of U{2..32768} valid cells, 2 query tokens
            # each (causal), 128 heads; plain, then with softcap 50, sinks and ALiBi over a
            # distance mask
            for tag, kw in (("plain", {}), ("softcap_sinks_alibi", dict(softcap=50.0, sinks=True, alibi=True,
                                                                         mask_kind="distance"))):
                p = synth.make_problem(kind="decode", n_seq=8, n_tok=2, n_head=128, n_kv=32768, seed=6,
                                       ragged=True, causal=True, **kw)
                r = _time_attend(B, p, args.steps, args.warmup)
                lens = p.kv_len.astype(np.int64)
                cells = int(sum(L - p.n_tok + t + 1 for L in lens for t in range(p.n_tok)))
                cache_bytes = int(lens.sum()) * 1152
                sec[f"n3_ragged_2tok_decode_{tag}"] = dict(
                    ms=r["step_ms"], cells_per_s=cells / (r["step_ms"] * 1e-3), n_split=r["n_split"],
                    cache_bytes_once=cache_bytes,
                    hbm_frac_cache_once=cache_bytes / (r["step_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS)
    if sec:
        result["secondary"] = sec
    if peaks:
        result["measured_peaks"] = peaks
    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        result.setdefault("calibration", {})["copy_bytes"] = n
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
