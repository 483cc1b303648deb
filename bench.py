"""Benchmark of the attention hot path on one MI355X; prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one pass over every kernel of the path on its workload, inputs already resident in HBM:
  * fa_fwd, bf16, causal, B=1 H=32 N=8192 d=128, scale 1/sqrt(128)   (prefill; the headline value)
  * fa_decode, bf16, B=64 H=32 N_kv=8192 d=128, 16 splits + combine   (split-KV decode)
  * fa_fwd, fp32, non-causal, B=1 H=1 N=256 d=64, scale 1/8            (fp32 path)
Untimed steps for 0.25 s (the clock ramps up from idle under load), then W untimed warm-up steps, then
K timed steps between device synchronisations (the extra workloads in "next" and the two probes each get
the same 0.25 s of untimed calls before their warm-up).  Every launch is
bracketed by HIP events on the stream it runs on, which gives each kernel's average duration over
the timed region.  value = prefill TFLOP/s (algorithmic flops 4*d per allowed pair / kernel time);
the decode figures (GB/s of algorithmic bytes) sit in "decode".  "context" holds the read bandwidth of a
plain streaming kernel and the shader clock under dense MFMA load, measured in the same run.  The CPU
oracle is timed on the host cores in the same run ("cpu_baseline": one worker process per core, whole
heads of the prefill workload, bounded samples of the other four).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(paths) -> str:
    """Short hash of the kernel source files (concatenated), to tell whether stored counters still apply."""
    h = hashlib.sha256()
    for path in ([paths] if isinstance(paths, str) else paths):
        h.update(open(os.path.join(ROOT, path), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str):
    """HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by the counters' ratio on a plain
    copy of known size) from profiles/traffic.json, or None if the kernel source changed since."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(kernel)
        if not rec or rec.get("source_sha") != source_sha(rec["source"]):
            return None
        return float(rec["bytes_per_launch"])
    except Exception:
        return None


TRAFFIC_KERNELS = {
    # name in traffic.json: (run directory prefix, kernel-name substring, kernel sources)
    "prefill_bf16_c3": ("prefill", "prefill_bf16_kernel",
                        ["exact_tiled_attention_09_amd/csrc/prefill_bf16.hip", "exact_tiled_attention_09_amd/csrc/common.h",
                         "exact_tiled_attention_09_amd/csrc/lds_tiles.h"]),
    "decode_split_c5": ("decode", "decode_split_kernel",
                        ["exact_tiled_attention_09_amd/csrc/decode.hip", "exact_tiled_attention_09_amd/csrc/common.h"]),
    "prefill_bf16_c4": ("prefill_c4", "prefill_bf16_kernel",
                        ["exact_tiled_attention_09_amd/csrc/prefill_bf16.hip", "exact_tiled_attention_09_amd/csrc/common.h",
                         "exact_tiled_attention_09_amd/csrc/lds_tiles.h"]),
}


def write_traffic(run_dir: str, copy_bytes: int = 1 << 30):
    """Build profiles/traffic.json from rocprofv3 --pmc runs of this script: <run_dir>/<prefix>.<COUNTER>/
    holding p_counter_collection.csv for prefix copy (--copy-bytes), prefill (--only prefill), decode
    (--only decode) and prefill_c4 (--only prefill_c4), COUNTER in FETCH_SIZE, WRITE_SIZE.  The copy of known size gives the factor that turns
    each counter's KiB into bytes."""
    import csv
    import glob
    import synthetic as syn

    def per_dispatch(prefix, counter, kernel):
        vals = {}
        for f in glob.glob(os.path.join(run_dir, f"{prefix}.{counter}", "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if kernel in r["Kernel_Name"] and r["Counter_Name"] == counter:
                    vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        if not vals:
            raise SystemExit(f"no {counter} samples for {kernel} under {run_dir}/{prefix}.{counter}")
        return sum(vals.values()) / len(vals), len(vals)

    # the runtime's device-to-device copy kernel (not the fill that initialises the source): per dispatch it
    # reads and writes copy_bytes
    fetch_copy, _ = per_dispatch("copy", "FETCH_SIZE", "copyBuffer")
    write_copy, _ = per_dispatch("copy", "WRITE_SIZE", "copyBuffer")
    rf, wf = copy_bytes / (fetch_copy * 1024), copy_bytes / (write_copy * 1024)
    out = {"_calibration": {"copy_bytes": copy_bytes, "fetch_kib": fetch_copy, "write_kib": write_copy,
                            "read_factor": rf, "write_factor": wf,
                            "note": "device-to-device copy of copy_bytes: bytes = counter KiB * 1024 * factor"}}
    wp, wd = syn.WORKLOADS["c3"], syn.WORKLOADS["c5"]
    alg = {"prefill_bf16_c3": wp.io_bytes,
           "decode_split_c5": 2 * wd.B * wd.H * wd.Nkv * wd.d * 2 + wd.B * wd.H * wd.d * 2,
           "prefill_bf16_c4": syn.WORKLOADS["c4"].io_bytes}
    for name, (prefix, kernel, sources) in TRAFFIC_KERNELS.items():
        fk, n = per_dispatch(prefix, "FETCH_SIZE", kernel)
        wk, _ = per_dispatch(prefix, "WRITE_SIZE", kernel)
        rb, wb = fk * 1024 * rf, wk * 1024 * wf
        out[name] = {"source": sources, "source_sha": source_sha(sources), "fetch_kib": fk, "write_kib": wk,
                     "read_bytes": rb, "write_bytes": wb, "bytes_per_launch": rb + wb,
                     "algorithmic_bytes": alg[name], "dispatches": n}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    json.dump(out, open(path, "w"), indent=1)
    print(json.dumps(out, indent=1))


# Seconds of untimed calls before each measurement of time_events (set by main from --settle): the GPU idles
# while the host generates the next workload's inputs, and the shader clock ramps up again from there.
SETTLE_S = {"value": 0.0}


def time_events(fn, stream, steps: int, warmup: int):
    """Average duration (ms) of fn() over `steps` calls, each bracketed by HIP events on `stream`, after
    SETTLE_S seconds of untimed calls in synchronised batches of five and `warmup` more calls."""
    import torch
    t_end = time.perf_counter() + SETTLE_S["value"]
    while time.perf_counter() < t_end:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))


def to_pages_dev(x, table, page_size: int):
    """Device-side layout change (input plumbing, untimed): contiguous cache x [B, H_kv, N, d] -> page pool
    [B * N / page_size, H_kv, page_size, d] with logical block j of sequence b at page table[b, j]."""
    import torch
    B, Hkv, N, d = x.shape
    nb = N // page_size
    blocks = x.view(B, Hkv, nb, page_size, d).permute(0, 2, 1, 3, 4).reshape(B * nb, Hkv, page_size, d)
    pool = torch.empty_like(blocks)
    pool[table.reshape(-1).long()] = blocks
    return pool


def time_paged(fa, syn, dev, stream, q, k, v, H: int, scale: float, S: int, steps: int, warmup: int, label: str):
    """fa_decode_paged over k, v [B, H_kv, N, d] moved into 16-token pages under a shuffled block table."""
    import torch
    B, Hkv, N, d = k.shape
    P = 16
    nb = N // P
    table = torch.from_numpy(syn.page_table(B, nb, B * nb, 8)).to(dev)
    kp, vp = to_pages_dev(k, table, P), to_pages_dev(v, table, P)
    sl = torch.full((B,), N, dtype=torch.int32, device=dev)
    o = torch.empty((B, H, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.fa_decode_paged_workspace_bytes(B, H, Hkv, N, d, S), dtype=torch.uint8, device=dev)
    t = time_events(lambda: fa.fa_decode_paged(q, kp, vp, table, sl, o, lse, scale, S, ws, stream), stream, steps,
                    warmup)
    by = 2 * B * Hkv * N * d * 2 + 2 * B * H * d * 2 + table.numel() * 4 + B * 4  # K, V, q, o, table, lengths
    return {"workload": f"fa_decode_paged bf16 B{B} H{H} H_kv{Hkv} N_kv{N} d{d}, {P}-token pages under a "
                        f"shuffled block table, {S} splits + combine ({label})",
            "value": round(by / (t * 1e-3) / 1e9, 1), "unit": "GB/s",
            "frac_of_peak": round(by / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "avg_ms": round(t, 4)}


def time_backward(fa, syn, upload, dev, stream, w, steps: int, warmup: int):
    """fa_bwd on a causal bf16 workload, the forward's O and LSE as input; TFLOP/s at 2.5x the forward's flops."""
    import torch
    log(f"[bench] next: backward of {w.name}")
    q, k, v = (upload(syn.make_tensor(w, t), "bf16") for t in "qkv")
    do = upload(syn.make_tensor(w, "do"), "bf16")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    fa.fa_fwd(q, k, v, o, lse, w.scale, True, stream)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.Nq), dtype=torch.uint8, device=dev)
    reps = max(3, steps // 4) if w.Nq >= 8192 else steps
    t = time_events(lambda: fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, w.scale, True, ws, stream), stream,
                    reps, warmup)
    fl = 2.5 * w.flops  # five products of 2*d flops per allowed pair (S, dP, dV, dQ, dK)
    tf = fl / (t * 1e-3) / 1e12
    return {"workload": f"fa_bwd causal bf16 B{w.B} H{w.H} N{w.Nq} d{w.d} (dQ, dK, dV)",
            "value": round(tf, 2), "unit": "TFLOP/s", "flops_per_call": fl,
            "flops_convention": "2.5x the forward's 4*d per allowed pair",
            "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "avg_ms": round(t, 4)}


def time_next(fa, syn, upload, dev, stream, steps: int, warmup: int, decode_inputs=None):
    """Workloads beyond the timed step (timed after it, not part of ms_per_step).  decode_inputs: the
    decode workload's (q, k, v, scale, splits) already on the device, reused for paged decode."""
    import torch
    out = {}
    # the two other causal bf16 prefill workloads (fa_fwd), for reference next to the timed one
    for cfg in ("c2", "c4"):
        w = syn.WORKLOADS[cfg]
        log(f"[bench] next: {w.name}")
        q, k, v = (upload(syn.make_tensor(w, t), "bf16") for t in "qkv")
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
        ts = []
        for _ in range(3):  # medians of three event-timed batches
            ts.append(time_events(lambda: fa.fa_fwd(q, k, v, o, lse, w.scale, True, stream), stream, steps, warmup))
        t = float(np.median(ts))
        out[f"prefill_{cfg}"] = {"workload": f"fa_fwd {w.name}", "value": round(w.flops / (t * 1e-3) / 1e12, 2),
                                 "unit": "TFLOP/s",
                                 "frac_of_peak": round(w.flops / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                 "avg_ms": round(t, 4)}
        del q, k, v, o, lse
    w = syn.NEXT_WORKLOADS["chunk"]
    log(f"[bench] next: {w.name}")
    q, k, v = (upload(syn.make_tensor(w, t), "bf16") for t in "qkv")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    t = time_events(lambda: fa.fa_fwd(q, k, v, o, lse, w.scale, True, stream), stream, steps, warmup)
    S = fa.fa_fwd_split_num_splits(w.B, w.H, w.Nq, w.Nkv, w.d)
    ws = torch.empty(fa.fa_fwd_split_workspace_bytes(w.B, w.H, w.Nq, w.d, S), dtype=torch.uint8, device=dev)
    ts = time_events(lambda: fa.fa_fwd_split(q, k, v, o, lse, w.scale, True, S, ws, stream), stream, steps, warmup)
    out["chunked_prefill"] = {"workload": "causal (bottom-right) bf16 B1 H32 N_q1000 N_kv8192 d128",
                              "value": round(w.flops / (ts * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                              "frac_of_peak": round(w.flops / (ts * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                              "entry_point": f"fa_fwd_split, {S} splits (fa_fwd_split_num_splits) + combine", "avg_ms": round(ts, 4),
                              "fa_fwd_single_pass_tflops": round(w.flops / (t * 1e-3) / 1e12, 2)}
    del q, k, v, o, lse, ws
    # grouped key/value decode: 32 query heads over 8 key/value heads, 8192 cached keys
    B, H, Hkv, N, d = 64, 32, 8, 8192, 128
    S = fa.fa_decode_gqa_num_splits(B, H, Hkv, N, d, 0)  # the library's own choice (4 here)
    wq = syn.custom(B, H, 1, 1, d, "bf16", False, None, seed=6)
    wkv = syn.custom(B, Hkv, 1, N, d, "bf16", False, None, seed=7)
    log(f"[bench] next: GQA decode B{B} H{H} H_kv{Hkv} N_kv{N} d{d}")
    q = upload(syn.make_tensor(wq, "q")[:, :, 0].copy(), "bf16")
    k, v = upload(syn.make_tensor(wkv, "k"), "bf16"), upload(syn.make_tensor(wkv, "v"), "bf16")
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.fa_decode_gqa_workspace_bytes(B, H, Hkv, N, d, S), dtype=torch.uint8, device=dev)
    t = time_events(lambda: fa.fa_decode_gqa(q, k, v, o, lse, wq.scale, S, ws, stream), stream, steps, warmup)
    by = 2 * B * Hkv * N * d * 2 + 2 * B * H * d * 2  # K, V read once; q read, o written
    out["gqa_decode"] = {"workload": f"fa_decode_gqa bf16 B{B} H{H} H_kv{Hkv} N_kv{N} d{d}, {S} splits + combine",
                         "value": round(by / (t * 1e-3) / 1e9, 1), "unit": "GB/s",
                         "frac_of_peak": round(by / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "avg_ms": round(t, 4)}
    log("[bench] next: paged GQA decode")
    out["paged_gqa_decode"] = time_paged(fa, syn, dev, stream, q, k, v, H, wq.scale, S, steps, warmup,
                                         "same data as gqa_decode")
    del q, k, v, o, lse, ws
    if decode_inputs is None:  # --only next: the decode workload's inputs are not on the device yet
        wd = syn.WORKLOADS["c5"]
        decode_inputs = (upload(syn.make_tensor(wd, "q")[:, :, 0].copy(), "bf16"),
                         upload(syn.make_tensor(wd, "k"), "bf16"), upload(syn.make_tensor(wd, "v"), "bf16"),
                         wd.scale, wd.num_splits)
    if decode_inputs is not None:
        log("[bench] next: paged decode")
        dq, dk, dv, dscale, dS = decode_inputs
        out["paged_decode"] = time_paged(fa, syn, dev, stream, dq, dk, dv, dq.shape[1], dscale, dS, steps, warmup,
                                         "same data as the decode step")
        del dq, dk, dv, decode_inputs
        torch.cuda.empty_cache()
    # backward of the causal prefill workloads (B1 H32 N8192 d128; B4 H16 N2048 d64): dQ, dK, dV from O, LSE
    # and dO
    out["backward"] = time_backward(fa, syn, upload, dev, stream, syn.WORKLOADS["c3"], steps, warmup)
    out["backward_d64"] = time_backward(fa, syn, upload, dev, stream, syn.WORKLOADS["c2"], steps, warmup)
    return out


def _warm(_):
    """Worker start-up: imports only (not timed)."""
    import synthetic  # noqa: F401
    import oracle  # noqa: F401
    return os.getpid()


def _oracle_head(args):
    """Worker: the oracle on one whole (b, h) slice of a workload (inputs generated in the worker, not
    timed).  Returns (seconds, flops)."""
    cfg, b, h, rows = args
    from threadpoolctl import threadpool_limits

    import synthetic as syn
    from oracle import attention_ref
    w = syn.WORKLOADS[cfg]
    with threadpool_limits(1):
        q, k, v = (syn.as_f64(syn.make_tensor(w, t, bh=[(b, h)], workers=1), w.dtype)[None] for t in "qkv")
        t0 = time.perf_counter()
        if rows is None:
            attention_ref(q, k, v, w.scale, w.causal)
            n = w.flops // (w.B * w.H)
        else:
            r = np.asarray(rows)
            attention_ref(q, k, v, w.scale, w.causal, rows=r)
            n = int(4 * w.d * (r + 1 + (w.Nkv - w.Nq)).sum()) if w.causal else 4 * w.d * w.Nkv * len(r)
        return time.perf_counter() - t0, n, os.getpid()


def _oracle_decode_rows(args):
    """Worker: the oracle on whole decode rows (b, h) of the decode workload.  Returns (seconds, bytes)."""
    pairs, = args
    from threadpoolctl import threadpool_limits

    import synthetic as syn
    from oracle import decode_ref
    w = syn.WORKLOADS["c5"]
    with threadpool_limits(1):
        q, k, v = (syn.as_f64(syn.make_tensor(w, t, bh=pairs, workers=1), "bf16")[None] for t in "qkv")
        t0 = time.perf_counter()
        decode_ref(q[:, :, 0], k, v, w.scale)
        return time.perf_counter() - t0, len(pairs) * (2 * w.Nkv * w.d * 2 + w.d * 2), os.getpid()


def cpu_baseline():
    """The fp64 oracle as it stands, on the host cores: one worker process per core (started fresh, not
    forked from this GPU process), BLAS held to one thread per worker, each worker taking whole heads.  The
    headline sample is every head of the causal prefill workload; bounded samples of the other four
    workloads follow.  Rate = work done / wall time of the pool."""
    import multiprocessing as mp

    import synthetic as syn
    cores = len(os.sched_getaffinity(0))
    ctx = mp.get_context("spawn")

    def run(fn, tasks):
        """(oracle seconds, results): the largest per-worker sum of timed oracle work, i.e. the wall time of
        the pool with the input generation (done in the workers, untimed) left out."""
        with ctx.Pool(cores) as pool:
            pool.map(_warm, range(cores))  # start-up imports, not timed
            res = pool.map(fn, tasks, chunksize=1)
        per_worker = {}
        for r in res:
            per_worker[r[2]] = per_worker.get(r[2], 0.0) + r[0]
        return max(per_worker.values()), res

    w = syn.WORKLOADS["c3"]
    wall, res = run(_oracle_head, [("c3", 0, h, None) for h in range(w.H)])
    flops = sum(r[1] for r in res)
    out = {"value": flops / wall / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
           "workers": f"{cores} processes (spawned), BLAS threads 1 each, one whole head per task",
           "sample": f"causal bf16 prefill B1 H32 N8192 d128: all {w.H} heads, every row, {flops / 1e9:.1f} GFLOP "
                     f"in fp64 in {wall:.2f} s on {cores} host cores (busiest worker's oracle time; "
                     f"{sum(r[0] for r in res):.1f} s of oracle time over all workers)"}
    per = {}
    for cfg in ("c1", "c2"):
        wc = syn.WORKLOADS[cfg]
        tasks = [(cfg, b, h, None) for b in range(wc.B) for h in range(wc.H)]
        wall, res = run(_oracle_head, tasks)
        per[cfg] = {"value": round(sum(r[1] for r in res) / wall / 1e12, 4), "unit": "TFLOP/s",
                    "wall_s": round(wall, 3), "sample": f"{wc.name}: all {len(tasks)} heads"}
    wc = syn.WORKLOADS["c4"]
    rows = np.linspace(0, wc.Nq - 1, 512).astype(np.int64)
    tasks = [("c4", 0, h, rows[i::2].tolist()) for h in range(wc.H) for i in range(2)]
    wall, res = run(_oracle_head, tasks)
    per["c4"] = {"value": round(sum(r[1] for r in res) / wall / 1e12, 4), "unit": "TFLOP/s", "wall_s": round(wall, 3),
                 "sample": f"{wc.name}: 512 evenly spaced causal rows of each of the {wc.H} heads"}
    wc = syn.WORKLOADS["c5"]
    pairs = [(b, h) for b in range(0, wc.B, 2) for h in range(0, wc.H, 4)]
    tasks = [(pairs[i::cores],) for i in range(cores) if pairs[i::cores]]
    wall, res = run(_oracle_decode_rows, tasks)
    per["c5"] = {"value": round(sum(r[1] for r in res) / wall / 1e9, 3), "unit": "GB/s (bf16 q, K, V bytes)",
                 "wall_s": round(wall, 3), "sample": f"{wc.name}: {len(pairs)} of {wc.B * wc.H} (b, h) rows"}
    out["per_config"] = per
    return out


def machine_context(fa, dev, stream, read_buf, steps: int = 5):
    """Measured machine figures beside the kernels' own: the read bandwidth of a plain non-temporal
    streaming kernel over read_buf (a byte view of a device tensor far larger than the caches) and the
    shader clock under dense MFMA load (s_memtime against the 100 MHz s_memrealtime)."""
    import torch
    n_cu = fa.device_num_cu() or 256
    groups = 2 * n_cu  # two streaming groups per CU read fastest (6.6-7.1 TB/s for 2-16 per CU on MI355X)
    sink = torch.empty(groups * 512, dtype=torch.int32, device=dev)
    t = time_events(lambda: fa.probe_read_bandwidth(read_buf, sink, groups, stream), stream, steps, 2)
    gbs = read_buf.numel() / (t * 1e-3) / 1e9
    cgroups, iters = 2 * n_cu, 10000
    out = torch.zeros(5 * cgroups, dtype=torch.int64, device=dev)
    tc = time_events(lambda: fa.probe_clock(out, cgroups, iters, stream), stream, 3, 1)
    o = out.view(cgroups, 5).cpu().numpy().astype(np.float64)
    mhz = 100.0 * (o[:, 2] - o[:, 0]) / np.maximum(o[:, 3] - o[:, 1], 1)
    assert not o[:, 4].any(), "clock probe accumulators went NaN"
    mfma_tflops = cgroups * 4 * (-(-iters // 8) * 64) * 32768 / (tc * 1e-3) / 1e12
    return {"read_stream": {"value": round(gbs, 1), "unit": "GB/s", "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
                            "bytes": read_buf.numel(), "avg_ms": round(t, 4),
                            "kernel": "fa_probe_read_bandwidth: 16-byte non-temporal loads, 4 in flight per "
                                      f"thread, {groups} groups of 512 each streaming one contiguous span"},
            "sclk_under_mfma": {"median_mhz": round(float(np.median(mhz)), 1), "min_mhz": round(float(mhz.min()), 1),
                                "max_mhz": round(float(mhz.max()), 1), "mfma_tflops": round(mfma_tflops, 1),
                                "kernel": f"fa_probe_clock: {cgroups} groups x 4 waves x {iters * 8} bf16 "
                                          "32x32x16 MFMAs on changing pseudo-random operands"},
            "num_cu": n_cu}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle", type=float, default=None,
                    help="seconds of untimed steps before the warm-up, so the timed steps see the clock the GPU "
                         "holds under this load rather than its ramp from idle (default 0.25 for the full run, "
                         "0 with --only, whose profiler runs count dispatches)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "step", "prefill", "decode", "f32", "next", "prefill_c2", "prefill_c4",
                                       "backward", "chunked"], default="all",
                    help="launch only this part (for profiler runs): 'step' is the timed step without the extra "
                         "workloads, 'next' only the extra workloads; 'prefill_c2' / 'prefill_c4' the other two causal "
                         "bf16 prefill workloads, 'backward' fa_bwd on the headline prefill workload and 'chunked' "
                         "fa_fwd_split on the chunked-prefill workload, each "
                         "--warmup + --steps times (a JSON line with their mean times is printed)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead of the step, run 5 device-to-device copies of this many bytes (calibrates "
                         "the profiler's HBM byte counters against a copy of known size) and exit")
    ap.add_argument("--write-traffic", metavar="RUN_DIR",
                    help="no GPU work: turn rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this script under RUN_DIR into "
                         "profiles/traffic.json and exit")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(args.write_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (the library drives one "
              f"MI355X per process; sharding across GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_tiled_attention_09_amd as fa
    import synthetic as syn

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.copy_bytes:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "copies": 5}))
        return

    def upload(x, dtype):
        if dtype == "f32":
            return torch.from_numpy(x).to(dev)
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)

    if args.only in ("prefill_c2", "prefill_c4", "backward", "chunked"):  # one workload alone, for profiler runs
        w = (syn.NEXT_WORKLOADS["chunk"] if args.only == "chunked"
             else syn.WORKLOADS["c3" if args.only == "backward" else args.only[-2:]])
        q, k, v = (upload(syn.make_tensor(w, t), "bf16") for t in "qkv")
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
        fa.fa_fwd(q, k, v, o, lse, w.scale, True, stream)
        if args.only == "backward":
            do = upload(syn.make_tensor(w, "do"), "bf16")
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.Nq), dtype=torch.uint8, device=dev)
            fn = lambda: fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, w.scale, True, ws, stream)  # noqa: E731
            fl = 2.5 * w.flops
        elif args.only == "chunked":
            S = fa.fa_fwd_split_num_splits(w.B, w.H, w.Nq, w.Nkv, w.d)
            ws = torch.empty(fa.fa_fwd_split_workspace_bytes(w.B, w.H, w.Nq, w.d, S), dtype=torch.uint8, device=dev)
            fn = lambda: fa.fa_fwd_split(q, k, v, o, lse, w.scale, True, S, ws, stream)  # noqa: E731
            fl = w.flops
        else:
            fn = lambda: fa.fa_fwd(q, k, v, o, lse, w.scale, True, stream)  # noqa: E731
            fl = w.flops
        t = time_events(fn, stream, args.steps, args.warmup)
        print(json.dumps({"workload": f"{args.only} {w.name}", "avg_ms": round(t, 4),
                          "tflops": round(fl / (t * 1e-3) / 1e12, 2)}))
        return

    wp, wd, w1 = syn.WORKLOADS["c3"], syn.WORKLOADS["c5"], syn.WORKLOADS["c1"]
    run_p = args.only in ("all", "step", "prefill")
    run_d = args.only in ("all", "step", "decode")
    run_f = args.only in ("all", "step", "f32")
    S = wd.num_splits
    log(f"[bench] generating inputs: {wp.name}, {wd.name}, {w1.name} (only={args.only})")
    if run_p:
        pq, pk, pv = (upload(syn.make_tensor(wp, t), "bf16") for t in "qkv")
        po = torch.empty_like(pq)
        plse = torch.empty(pq.shape[:-1], dtype=torch.float32, device=dev)
    if run_d:
        dq = upload(syn.make_tensor(wd, "q")[:, :, 0].copy(), "bf16")
        dk = upload(syn.make_tensor(wd, "k"), "bf16")
        dv = upload(syn.make_tensor(wd, "v"), "bf16")
        do = torch.empty_like(dq)
        dlse = torch.empty(dq.shape[:-1], dtype=torch.float32, device=dev)
        ws = fa.decode_workspace(wd.B, wd.H, wd.Nkv, wd.d, S, dev)
    if run_f:
        fq, fk, fv = (upload(syn.make_tensor(w1, t), "f32") for t in "qkv")
        fo = torch.empty_like(fq)
        flse = torch.empty(fq.shape[:-1], dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if run_p:
            fa.fa_fwd(pq, pk, pv, po, plse, wp.scale, True, stream)
        if ev is not None:
            ev[1].record(stream)
        if run_d:
            fa.fa_decode_split(dq, dk, dv, wd.scale, S, ws, stream)
        if ev is not None:
            ev[2].record(stream)
        if run_d:
            fa.fa_decode_combine(ws, do, dlse, S, stream)
        if ev is not None:
            ev[3].record(stream)
        if run_f:
            fa.fa_fwd(fq, fk, fv, fo, flse, w1.scale, False, stream)
        if ev is not None:
            ev[4].record(stream)

    # The shader clock ramps up from idle over the first tens of milliseconds of load (a 5-step warm-up
    # leaves the first timed steps ~6% slower than the rest).  The step therefore runs untimed, in
    # synchronised batches, until --settle seconds have passed, then the W warm-up steps, then the K
    # timed steps; the record states how long and how many steps the settling took.
    settle = args.settle if args.settle is not None else (0.25 if args.only == "all" else 0.0)
    SETTLE_S["value"] = settle  # the same settling before each of the extra workloads and probes
    log(f"[bench] settle {settle} s")
    t_settle0, n_settle = time.perf_counter(), 0
    while time.perf_counter() - t_settle0 < settle:
        for _ in range(5):
            step()
        n_settle += 5
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_settle0
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = lambda a, b: np.array([evs[i][a].elapsed_time(evs[i][b]) for i in range(args.steps)])  # noqa: E731
    t_prefill, t_split, t_comb, t_f32 = ms(0, 1), ms(1, 2), ms(2, 3), ms(3, 4)
    t_step = ms(0, 4)

    # parts left out by --only report null rather than a rate over an empty interval
    def rate(work, ms_, ran, unit):
        return round(work / (ms_ * 1e-3) / unit, 3) if ran and ms_ > 0 else None

    def frac(x, peak):
        return None if x is None else round(x / peak, 4)

    def kms(t, ran, f=np.mean):
        return round(float(f(t)), 4) if ran else None

    pf_tflops = rate(wp.flops, t_prefill.mean(), run_p, 1e12)
    split_bytes = 2 * wd.B * wd.H * wd.Nkv * wd.d * 2 + wd.B * wd.H * wd.d * 2   # K, V, q read once
    split_gbs = rate(split_bytes, t_split.mean(), run_d, 1e9)
    dec_gbs = rate(wd.io_bytes, t_split.mean() + t_comb.mean(), run_d, 1e9)
    f32_tflops = rate(w1.flops, t_f32.mean(), run_f, 1e12)

    rec = {
        "metric": "prefill TFLOP/s & % bf16 MFMA peak; decode KV-read GB/s & % HBM peak",
        "value": pf_tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"seconds": round(settle_s, 3), "steps": n_settle},
        "ms_per_step": kms(t_step, args.only in ("all", "step")),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "fa_fwd causal bf16 prefill B1 H32 N8192 d128 (value) + fa_decode split-KV bf16 "
                        "B64 H32 N_kv8192 d128 S16 + combine + fa_fwd fp32 B1 H1 N256 d64",
            "prefill": {"B": wp.B, "H": wp.H, "N_q": wp.Nq, "N_kv": wp.Nkv, "d": wp.d, "causal": True,
                        "flops_per_launch": wp.flops},
            "decode": {"B": wd.B, "H": wd.H, "N_kv": wd.Nkv, "d": wd.d, "num_splits": S,
                       "alg_bytes_per_call": wd.io_bytes},
        },
        "roofline": {
            "kernel": "prefill_bf16_kernel<128,...,causal>",
            "bound": "mfma",
            "achieved": pf_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": frac(pf_tflops, PEAK_BF16_TFLOPS),
            "traffic": traffic_from_profiles("prefill_bf16_c3"),
            "avg_kernel_ms": kms(t_prefill, run_p),
            "median_kernel_ms": kms(t_prefill, run_p, np.median),
            "min_kernel_ms": kms(t_prefill, run_p, np.min),
        },
        "decode": {
            "value": dec_gbs,
            "unit": "GB/s",
            "frac_of_peak": frac(dec_gbs, PEAK_HBM_GBS),
            "ms": kms(t_split + t_comb, run_d),
            "roofline": {
                "kernel": "decode_split_kernel<128>",
                "bound": "hbm",
                "achieved": split_gbs,
                "peak": PEAK_HBM_GBS,
                "unit": "GB/s",
                "frac": frac(split_gbs, PEAK_HBM_GBS),
                "traffic": traffic_from_profiles("decode_split_c5"),
                "avg_kernel_ms": kms(t_split, run_d),
                "median_kernel_ms": kms(t_split, run_d, np.median),
                "min_kernel_ms": kms(t_split, run_d, np.min),
                "combine_avg_kernel_ms": kms(t_comb, run_d),
            },
        },
        "fp32_prefill": {"value": f32_tflops, "unit": "TFLOP/s", "avg_kernel_ms": kms(t_f32, run_f)},
        "wall_s_timed": round(wall, 4),
        "gpu": torch.cuda.get_device_name(0),
    }
    if args.only in ("all", "step", "decode") and run_d:
        log("[bench] machine context: read-stream bandwidth and shader clock")
        rec["context"] = machine_context(fa, dev, stream, dk.view(torch.uint8).view(-1))
    if args.only in ("all", "next"):
        rec["next"] = time_next(fa, syn, upload, dev, stream, args.steps, args.warmup,
                                (dq, dk, dv, wd.scale, S) if run_d else None)
    if not args.no_cpu_baseline and args.only == "all":
        log("[bench] timing the CPU oracle on a bounded sample")
        rec["cpu_baseline"] = cpu_baseline()
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
