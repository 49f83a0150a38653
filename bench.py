"""Benchmark of paged MLA decode on one MI355X.

A step is one pass of the whole path over one synthetic decode batch:
split-KV metadata, the decode kernel and the combine kernel, enqueued through
the C ABI on one stream.  Inputs are resident in HBM before timing starts.
Successive steps read different copies of the latent cache (as successive
layers do), so the 256 MB last-level cache cannot serve a repeated batch.

Prints one JSON line: whole-job TFLOPS (value) and HBM GB/s over the timed
steps, the decode kernel's roofline fraction from HIP events on its stream
(taken in a second pass of the same steps: events between the kernels of a
step would add to the step time), and the CPU oracle timed on a bounded
sample of the same workload.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBPS * 1e9)

DEFAULT_CONFIG = 3  # dense bf16, h_q=128, s_q=2 causal: the workload the target is stated on


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU raises its clock over the first tens to hundreds of
    # milliseconds of sustained work: a time-based settle phase runs first,
    # whatever the warm-up count.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--settle-ms", type=float, default=600.0,
                    help="untimed settle phase before the warm-up: at least this many ms of "
                         "steps, then until the per-step time is stable")
    ap.add_argument("--settle-max-ms", type=float, default=3000.0)
    ap.add_argument("--config", type=int, default=DEFAULT_CONFIG, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--num-parts", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-units", type=int, default=None)
    ap.add_argument("--kernel", choices=["decode", "small", "small_fp8", "writer", "prefill", "indexer"],
                    default="decode",
                    help="decode: the decode step (default); writer: the FP8 KV writer filling "
                         "128 sequences x 4096 new tokens; prefill: sparse prefill, 4096 query "
                         "tokens x 128 heads over a 32768-row cache, topk 2048; small: decode with "
                         "16 query heads (an 8-way head split of the 128), batch 128, lengths "
                         "U[1024, 8192]; small_fp8: the same heads over the 656-byte FP8 cache, "
                         "lengths U[8192, 32768]; indexer: the FP8 top-k indexer over 128 x 65536 "
                         "cached FP8 rows, 2 query tokens x 128 heads, topk 2048")
    ap.add_argument("--no-measured-peaks", action="store_true",
                    help="skip the reference measurements of HBM copy bandwidth and bf16 GEMM "
                         "throughput on this GPU")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run three 1 GiB device-to-device copies (reference for the HBM byte "
                         "counters under rocprofv3), print nothing else")
    return ap.parse_args()


def copy_calibration():
    """Three copies of a 1 GiB device buffer: a kernel of known traffic
    (1 GiB read and 1 GiB written per dispatch) that calibrates rocprofv3's
    FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()


def measured_peaks():
    """What this GPU reaches on plain reference work, after the timed region:
    HBM bandwidth of a 1 GiB device-to-device copy (bytes read + written per
    second) and bf16 matrix-core throughput of an 8192^3 library GEMM.  The
    roofline fractions are also reported against these."""
    import torch

    out = {}
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    out["hbm_copy_gbps"] = 2 * n * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    m = 8192
    x = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    y = torch.randn(m, m, device="cuda").to(torch.bfloat16)
    for _ in range(5):
        torch.matmul(x, y)
    e0.record()
    for _ in range(20):
        torch.matmul(x, y)
    e1.record()
    torch.cuda.synchronize()
    out["bf16_gemm_tflops"] = 2 * m ** 3 * 20 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    return out


def with_measured(roof, peaks):
    """Adds the fraction of the measured reference peak to a roofline record."""
    if peaks is None:
        return None
    ref = peaks["hbm_copy_gbps"] if roof["unit"] == "GB/s" else peaks["bf16_gemm_tflops"]
    return dict(peaks, frac_of_measured=roof["achieved"] / ref)


def traffic_record(config_name: str, prefix: str = "decode"):
    """HBM traffic of a kernel from the committed rocprofv3 counter summary,
    if it was taken on the current source of the kernel it names; else None."""
    path = os.path.join(ROOT, "profiles", f"{prefix}_{config_name}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    source = rec.get("source", "decode.hip")
    src_path = os.path.join(ROOT, "paged_kv_head_amd", "csrc", source)
    if not os.path.exists(src_path):
        return None
    src = open(src_path, "rb").read()
    if rec.get("source_sha256", rec.get("decode_source_sha256")) != hashlib.sha256(src).hexdigest():
        return None
    return rec


def settle(step, min_ms: float, max_ms: float, window: int = 20):
    """Untimed steps before the warm-up: the GPU raises its clock over the
    first tens to hundreds of milliseconds of sustained work.  Steps run in
    windows until at least min_ms of wall time has passed and the mean step
    time of the last window is within 2 % of the one before (or max_ms has
    passed).  Returns (elapsed ms, steps)."""
    import torch

    t0 = time.perf_counter()
    n = 0
    last = None
    while True:
        ts = time.perf_counter()
        for _ in range(window):
            step(n)
            n += 1
        torch.cuda.synchronize()
        dt = (time.perf_counter() - ts) / window
        elapsed = (time.perf_counter() - t0) * 1e3
        if elapsed >= max_ms:
            break
        if elapsed >= min_ms and last is not None and abs(dt - last) <= 0.02 * last:
            break
        last = dt
    return elapsed, n


def clock_record():
    """Shader clock right after the timed region, from the library's probe
    (the matrix cores kept busy by every workgroup)."""
    import paged_kv_head_amd as mla

    return {"shader_clock_mhz": round(mla.shader_clock_mhz(), 1),
            "method": "s_memtime / s_memrealtime (100 MHz) over ~2 ms of bf16 MFMA chains on "
                      "256 workgroups, measured right after the timed region"}


def cpu_baseline(w, sample_units, min_seconds=10.0, max_reps=6):
    """The oracle on the host cores over a bounded sample of the workload's
    query tokens (all of them by default), repeated until about min_seconds
    of CPU work have been timed."""
    import oracle

    threads = oracle.num_threads()
    U = w.batch * w.s_q
    n = U if sample_units is None else min(sample_units, U)
    rng = np.random.default_rng(0)
    pick = np.sort(rng.choice(U, size=n, replace=False))
    mask = np.zeros(U, dtype=np.uint8)
    mask[pick] = 1
    # FLOPs of the sampled query tokens (each attends over its own key count)
    if w.topk > 0:
        sk = np.full(U, w.topk, dtype=np.int64)
    else:
        sk = np.repeat(w.cache_seqlens.astype(np.int64), w.s_q)
    flops = float(2 * w.h_q * sk[pick].sum() * (576 + 512))
    secs, reps = 0.0, 0
    while reps < max_reps and (reps == 0 or secs < min_seconds):
        _, _, t = oracle.timed_mla_decode(w, unit_mask=mask)
        secs += t
        reps += 1
    return {"value": flops * reps / secs / 1e12, "unit": "TFLOPS", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {U} query tokens (all {w.h_q} heads each) of {w.name}, "
                      f"{reps} pass(es), {secs:.1f} s on the host"}


WRITER_WORKLOAD = dict(name="fp8_writer_fill_b128_n4096", batch=128, n_new=4096, seed=2024)


def writer_cpu_baseline(w, n_tokens=20000, min_seconds=10.0, max_reps=6):
    """The oracle's append (one thread) over a bounded sample of the fill's
    tokens: the first n_tokens of sequence order."""
    import oracle

    B, n_new, _ = w.kv_new.shape
    nb = max(1, min(B, n_tokens // n_new)) if n_tokens >= n_new else 1
    nn = min(n_new, n_tokens)
    sub_new = np.ascontiguousarray(w.kv_new[:nb, :nn])
    secs, reps = 0.0, 0
    while reps < max_reps and (reps == 0 or secs < min_seconds):
        t = time.perf_counter()
        oracle.kv_append_fp8(sub_new, w.start_pos[:nb], w.block_table[:nb], w.pool)
        secs += time.perf_counter() - t
        reps += 1
    tok = nb * nn
    return {"value": tok * 1808 * reps / secs / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{tok} of {B * n_new} tokens ({nb} sequences x {nn}) of {w.name}, "
                      f"{reps} pass(es), {secs:.1f} s on one host thread (pool copy included)"}


def bench_writer(args):
    """FP8 KV writer: quantise 128 x 4096 new bf16 latent rows into the
    656-byte paged layout.  Algorithmic bytes per token: 1152 read + 656
    written, plus the block table (4 bytes per page) and start positions."""
    import torch

    import paged_kv_head_amd as mla
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    c = WRITER_WORKLOAD
    t0 = time.time()
    w = synth.make_append(c["name"], batch=c["batch"], n_new=c["n_new"],
                          start_pos=[0] * c["batch"], seed=c["seed"])
    print(f"[bench] workload {w.name}: generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    kv_new = torch.from_numpy(w.kv_new.view(np.int16)).to(dev).view(torch.bfloat16)
    sp = torch.from_numpy(w.start_pos).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    pool = torch.from_numpy(w.pool).to(dev)
    stream = torch.cuda.current_stream()
    mla.mla_kv_quantize_fp8(kv_new, sp, bt, pool)  # checked call once
    lib = mla._load()
    P = ctypes.c_void_p
    B, n_new = int(kv_new.shape[0]), int(kv_new.shape[1])
    call = (B, n_new, 64, int(pool.shape[0]), int(bt.shape[1]), P(kv_new.data_ptr()),
            P(sp.data_ptr()), P(bt.data_ptr()), P(pool.data_ptr()), P(stream.cuda_stream))
    settle_ms, settle_steps = settle(lambda i: lib.mla_kv_quantize_fp8(*call), args.settle_ms,
                                     args.settle_max_ms)
    for _ in range(args.warmup):
        lib.mla_kv_quantize_fp8(*call)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        if lib.mla_kv_quantize_fp8(*call):
            raise RuntimeError(mla.mla_last_error())
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    # the kernel's duration: a second pass with events around every launch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record(stream)
        rc = lib.mla_kv_quantize_fp8(*call)
        evs[i][1].record(stream)
        if rc:
            raise RuntimeError(mla.mla_last_error())
    torch.cuda.synchronize()
    k_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    ms_per_step = wall * 1e3 / args.steps
    clock = clock_record()
    tokens = w.tokens
    pages = int((w.block_table >= 0).sum())
    alg_bytes = tokens * (1152 + 656) + 4 * pages + 4 * B
    achieved = alg_bytes / (k_ms * 1e-3) / 1e9
    tr = traffic_record(w.name, "kv_writer")
    peaks = None if args.no_measured_peaks else measured_peaks()
    cpu = None if args.no_cpu_baseline else writer_cpu_baseline(w)
    line = {
        "metric": "FP8 KV writer GB/s (bf16 576-value rows -> 656-byte paged FP8 rows), % of HBM roofline",
        "value": alg_bytes / (ms_per_step * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic", "settle_ms": round(settle_ms, 1), "settle_steps": settle_steps,
        "clock": clock,
        "config": {"workload": w.name, "batch": B, "n_new": n_new, "tokens": tokens,
                   "num_pages": int(pool.shape[0]), "algorithmic_bytes_per_step": alg_bytes},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS,
                     "traffic": None if tr is None else tr["hbm_bytes_per_launch"],
                     "kernel": "kv_quantize_fp8_kernel", "kernel_ms": k_ms},
        "measured_peaks": with_measured({"unit": "GB/s", "achieved": achieved}, peaks),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


SMALL_WORKLOAD = dict(name="b128_h16_sq1_dense_bf16")

PREFILL_WORKLOAD = dict(name="prefill_s4096_kv32768_topk2048", s_q=4096, h_q=128, s_kv=32768,
                        topk=2048, seed=77)


def prefill_cpu_baseline(w, n_tokens=640, min_seconds=10.0, max_reps=8):
    """The prefill oracle (numpy fp64) on the first n_tokens query tokens."""
    from oracle.sparse_prefill import sparse_prefill

    n = min(n_tokens, w.s_q)
    secs, reps = 0.0, 0
    while reps < max_reps and (reps == 0 or secs < min_seconds):
        t = time.perf_counter()
        sparse_prefill(w.q[:n], w.kv, w.indices[:n], w.softmax_scale, w.kv_format)
        secs += time.perf_counter() - t
        reps += 1
    flops = 2 * w.h_q * n * w.topk * (576 + 512) * reps
    return {"value": flops / secs / 1e12, "unit": "TFLOPS", "cores": int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count(),
            "kind": "oracle",
            "sample": f"{n} of {w.s_q} query tokens (all {w.h_q} heads) of {w.name}, {reps} pass(es), "
                      f"{secs:.1f} s on the host (numpy fp64; BLAS threads as the host allows)"}


def bench_prefill(args):
    """Sparse prefill: gather-attend of 4096 query tokens (128 heads each)
    over their own 2048 rows of a flat 32768-row bf16 latent cache."""
    import torch

    import paged_kv_head_amd as mla
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    c = PREFILL_WORKLOAD
    t0 = time.time()
    w = synth.make_sparse_prefill(c["name"], s_q=c["s_q"], h_q=c["h_q"], s_kv=c["s_kv"],
                                  topk=c["topk"], seed=c["seed"])
    print(f"[bench] workload {w.name}: generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    q = torch.from_numpy(w.q.view(np.int16)).to(dev).view(torch.bfloat16)
    kv = torch.from_numpy(w.kv).to(dev).view(torch.bfloat16)
    idx = torch.from_numpy(w.indices).to(dev)
    parts = mla.mla_sparse_prefill_num_parts(w.h_q, w.topk, 0, 0)
    need = mla.mla_sparse_prefill_workspace_bytes(w.s_q, w.h_q, w.s_kv, w.topk, 0, parts)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    out = torch.empty((w.s_q, w.h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.s_q, w.h_q), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    mla.mla_sparse_prefill(q, kv, idx, w.softmax_scale, num_parts=parts, workspace=ws, out=out,
                           lse=lse)  # checked call once
    lib = mla._load()
    P = ctypes.c_void_p
    call = (w.s_q, w.h_q, w.s_kv, w.topk, 0, 0, ctypes.c_float(w.softmax_scale), P(q.data_ptr()),
            P(kv.data_ptr()), P(idx.data_ptr()), parts, P(ws.data_ptr()), ctypes.c_size_t(need),
            P(out.data_ptr()), P(lse.data_ptr()), P(stream.cuda_stream))
    warm = max(3, args.warmup // 20)
    steps = max(5, args.steps // 10)
    settle_ms, settle_steps = settle(lambda i: lib.mla_sparse_prefill(*call), args.settle_ms,
                                     args.settle_max_ms, window=2)
    for _ in range(warm):
        lib.mla_sparse_prefill(*call)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(steps):
        if lib.mla_sparse_prefill(*call):
            raise RuntimeError(mla.mla_last_error())
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    # the call's duration: a second pass with events around every call
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record(stream)
        rc = lib.mla_sparse_prefill(*call)
        evs[i][1].record(stream)
        if rc:
            raise RuntimeError(mla.mla_last_error())
    torch.cuda.synchronize()
    call_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    ms_per_step = wall * 1e3 / steps
    clock = clock_record()
    flops = w.flops()
    alg_bytes = w.algorithmic_bytes()
    achieved = flops / (call_ms * 1e-3) / 1e12
    traffic = traffic_record(w.name, "prefill")
    peaks = None if args.no_measured_peaks else measured_peaks()
    cpu = None if args.no_cpu_baseline else prefill_cpu_baseline(w)
    line = {
        "metric": "sparse MLA prefill TFLOPS (h_q=128, d_qk=576, d_v=512, topk=2048), % of roofline",
        "value": flops / (ms_per_step * 1e-3) / 1e12, "unit": "TFLOPS", "n_gpus": 1, "steps": steps,
        "warmup": warm, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "arithmetic_intensity": flops / alg_bytes, "settle_ms": round(settle_ms, 1),
        "settle_steps": settle_steps, "clock": clock,
        "config": {"workload": w.name, "s_q": w.s_q, "h_q": w.h_q, "s_kv": w.s_kv, "topk": w.topk,
                   "kv_format": "bf16", "num_parts": parts, "flops_per_step": flops,
                   "algorithmic_bytes_per_step": alg_bytes},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     # HBM bytes of the whole call (every kernel it launches)
                     "traffic": None if traffic is None else traffic["hbm_bytes_per_launch"],
                     "kernel": "mla_sparse_prefill call (identity table; per 2048-token chunk: "
                               "metadata, decode_kernel, combine_kernel)",
                     "kernel_ms": call_ms},
        "measured_peaks": with_measured({"unit": "TFLOP/s", "achieved": achieved}, peaks),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


INDEX_WORKLOAD = dict(name="index_b128_sq2_h128_l65536_topk2048", batch=128, s_q=2, h=128, seqlen=65536,
                      topk=2048, seed=88)


def index_cpu_baseline(w, n_tokens=16, min_seconds=10.0, max_reps=8):
    """The indexer oracle (numpy fp64) on a bounded sample of query tokens;
    value in GB/s of the sample's algorithmic bytes (its share of the cache
    rows, query and indices)."""
    from oracle import indexer as ix

    U = w.batch * w.s_q
    rng = np.random.default_rng(0)
    pick = [(int(u) // w.s_q, int(u) % w.s_q) for u in np.sort(rng.choice(U, size=min(n_tokens, U), replace=False))]
    secs, reps = 0.0, 0
    while reps < max_reps and (reps == 0 or secs < min_seconds):
        t = time.perf_counter()
        ix.top_k(w, tokens=pick)
        secs += time.perf_counter() - t
        reps += 1
    per_token = w.algorithmic_bytes() / U
    return {"value": per_token * len(pick) * reps / secs / 1e9, "unit": "GB/s",
            "cores": int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count(), "kind": "oracle",
            "sample": f"{len(pick)} of {U} query tokens (all {w.h} heads, all {int(w.rows()[0])} rows) of "
                      f"{w.name}, {reps} pass(es), {secs:.1f} s on the host (numpy fp64; BLAS threads "
                      f"as the host allows)"}


def bench_indexer(args):
    """FP8 top-k indexer over the sparse decode benchmark's cache: 128
    sequences of 65536 tokens in the 656-byte FP8 layout, two query tokens of
    128 heads each, topk 2048.  A step is one mla_fp8_index_top_k call (the
    score kernel, then the selection kernel), timed as its two phases."""
    import torch

    import paged_kv_head_amd as mla
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    c = INDEX_WORKLOAD
    t0 = time.time()
    w = synth.make_index_workload(c["name"], batch=c["batch"], s_q=c["s_q"], h=c["h"],
                                  seqlens=[c["seqlen"]] * c["batch"], seed=c["seed"], topk=c["topk"])
    print(f"[bench] workload {w.name}: generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    p = mla.index_problem_for(w)
    qc, qs, kv, bt, sl = mla.index_tensors(w)
    need = mla.mla_fp8_index_workspace_bytes(p)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    idx = torch.empty((w.batch, w.s_q, w.topk), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    mla.mla_fp8_index_top_k(p, qc, qs, kv, bt, sl, ws, idx)  # checked call once
    lib = mla._load()
    P = ctypes.c_void_p
    pp = ctypes.byref(p)
    st = P(stream.cuda_stream)
    score_args = (pp, P(qc.data_ptr()), P(qs.data_ptr()), P(kv.data_ptr()), P(bt.data_ptr()),
                  P(sl.data_ptr()), P(ws.data_ptr()), ctypes.c_size_t(need), st)
    select_args = (pp, P(sl.data_ptr()), P(ws.data_ptr()), ctypes.c_size_t(need), P(idx.data_ptr()), None, st)

    def step(i, ev=None):
        if ev:
            ev[0].record(stream)
        a = lib.mla_fp8_index_scores(*score_args)
        if ev:
            ev[1].record(stream)
        b = lib.mla_fp8_index_select(*select_args)
        if ev:
            ev[2].record(stream)
        if a or b:
            raise RuntimeError(mla.mla_last_error())

    settle_ms, settle_steps = settle(step, args.settle_ms, args.settle_max_ms, window=5)
    warm = max(3, args.warmup // 5)
    steps = max(10, args.steps // 4)
    for i in range(warm):
        step(i)
    torch.cuda.synchronize()
    # timed region: plain steps; the phase durations come from a second pass
    # with events between the phases (events cost a few us per step)
    t_start = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    score_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    select_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ms_per_step = wall * 1e3 / steps
    clock = clock_record()
    rows = int(w.rows().sum())
    alg_bytes = w.algorithmic_bytes()
    # the score kernel alone: quantised part of every row (528 B), the FP8
    # query, block-table entries and lengths
    pages = int(((w.rows() + 63) // 64).sum())
    score_bytes = rows * 528 + w.batch * w.s_q * w.h * 528 + 4 * pages + 4 * w.batch
    # multiply-adds of the definition (every head); the kernels sum the
    # heads first and do 512 per (token, row), far below any compute roof,
    # so the score phase is bound by the cache stream
    flops = w.flops()
    roof = {"bound": "hbm", "achieved": score_bytes / (score_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBPS,
            "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    tr = traffic_record(w.name, "indexer")
    roof["traffic"] = None if tr is None else tr["hbm_bytes_per_launch"]
    roof["kernel"] = "index_score_kernel (with index_query_kernel: the mla_fp8_index_scores phase)"
    roof["kernel_ms"] = score_ms
    roof["kernel_ms_method"] = "HIP events around each phase, in a second pass of the same steps after the timed region"
    peaks = None if args.no_measured_peaks else measured_peaks()
    cpu = None if args.no_cpu_baseline else index_cpu_baseline(w)
    line = {
        "metric": "FP8 top-k indexer GB/s (656-byte FP8 cache rows scored against an FP8 query of 128 heads, "
                  "top-2048 per query token), % of roofline",
        "value": alg_bytes / (ms_per_step * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": warm, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8", "data": "synthetic",
        "settle_ms": round(settle_ms, 1),
        "settle_steps": settle_steps, "clock": clock,
        "config": {"workload": w.name, "batch": w.batch, "s_q": w.s_q, "h": w.h, "seqlen": c["seqlen"],
                   "topk": w.topk, "rows": rows, "definition_flops_per_step": flops,
                   "algorithmic_bytes_per_step": alg_bytes, "score_kernel_algorithmic_bytes": score_bytes,
                   "select_kernel_ms": select_ms},
        "roofline": roof,
        "measured_peaks": with_measured({"unit": "GB/s", "achieved": score_bytes / (score_ms * 1e-3) / 1e9},
                                        peaks),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py: this benchmark measures one GPU only (got --gpus {args.gpus}); "
              "the path shards by batch or by query head with no exchange, so N GPUs "
              "would run N independent copies of the one-GPU step.", file=sys.stderr)
        sys.exit(2)
    if args.kernel == "writer":
        bench_writer(args)
        return
    if args.kernel == "indexer":
        bench_indexer(args)
        return
    if args.kernel == "prefill":
        bench_prefill(args)
        return

    import torch

    import paged_kv_head_amd as mla
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    t0 = time.time()
    if args.kernel == "small":
        w = synth.make_workload(SMALL_WORKLOAD["name"], batch=128, h_q=16, s_q=1,
                                seqlens=synth.Uniform(1024, 8192), seed=1006, max_pages_per_seq=128)
    elif args.kernel == "small_fp8":
        w = synth.make_workload("b128_h16_sq1_fp8_l8k_32k", batch=128, h_q=16, s_q=1,
                                seqlens=synth.Uniform(8192, 32768), seed=1008,
                                max_pages_per_seq=512, kv_format=synth.KV_FP8_656)
    else:
        w = synth.config_workload(args.config)
    print(f"[bench] workload {w.name}: generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    p = mla.problem_for(w)
    q, kv, bt, sl, idx = mla.workload_tensors(w, dev)
    pool_bytes = kv.numel()
    copies = max(2, math.ceil(1.0e9 / pool_bytes))
    kvs = [kv] + [kv.clone() for _ in range(copies - 1)]
    plan = mla.DecodePlan(p, dev, args.num_parts)
    out = torch.empty((w.batch, w.s_q, w.h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.s_q, w.h_q), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    # Checked calls once (argument and buffer checks), then a lean loop that
    # calls the C ABI with pre-built ctypes arguments so that host overhead
    # stays far below the GPU time of a step and the queue never drains.
    mla.mla_decode_get_metadata(p, sl, plan.num_parts, plan.sched, plan.num_splits)
    for i in range(copies):
        mla.mla_decode_paged(p, q, kvs[i], bt, sl, idx, plan.sched, plan.num_parts,
                             plan.num_splits, plan.workspace, out, lse)
    mla.mla_decode_combine(p, plan.num_parts, plan.num_splits, plan.workspace, out, lse)
    lib = mla._load()
    P = ctypes.c_void_p
    ref = ctypes.byref(p)
    st = P(stream.cuda_stream)
    ws_bytes = plan.workspace.numel()
    meta_args = (ref, P(sl.data_ptr()), plan.num_parts, P(plan.sched.data_ptr()),
                 P(plan.num_splits.data_ptr()), st)
    dec_args = [(ref, P(q.data_ptr()), P(kvs[i].data_ptr()), P(bt.data_ptr()), P(sl.data_ptr()),
                 None if idx is None else P(idx.data_ptr()), P(plan.sched.data_ptr()),
                 plan.num_parts, P(plan.num_splits.data_ptr()), P(plan.workspace.data_ptr()),
                 ws_bytes, P(out.data_ptr()), P(lse.data_ptr()), st) for i in range(copies)]
    comb_args = (ref, plan.num_parts, P(plan.num_splits.data_ptr()), P(plan.workspace.data_ptr()),
                 ws_bytes, P(out.data_ptr()), P(lse.data_ptr()), st)

    def step(i, ev=None):
        rc = lib.mla_decode_get_metadata(*meta_args)
        if ev is not None:
            ev[0].record(stream)
        rc |= lib.mla_decode_paged(*dec_args[i % copies])
        if ev is not None:
            ev[1].record(stream)
        rc |= lib.mla_decode_combine(*comb_args)
        if rc:
            raise RuntimeError(mla.mla_last_error())

    settle_ms, settle_steps = settle(step, args.settle_ms, args.settle_max_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # The timed region: K plain steps.  Timing events between the kernels
    # of a step cost about 5 us per step on this GPU (each record waits for
    # the kernel before it to drain), so the decode kernel's own duration is
    # taken in a second pass of K steps right after it, with events around
    # every decode launch.
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t_ev = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    ms_per_step_with_events = (time.perf_counter() - t_ev) * 1e3 / args.steps
    dec_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    ms_per_step = wall * 1e3 / args.steps
    clock = clock_record()

    flops = w.flops()
    alg_bytes = w.algorithmic_bytes()
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    gbps = alg_bytes / (ms_per_step * 1e-3) / 1e9
    intensity = flops / alg_bytes
    if intensity >= RIDGE:
        roof = {"bound": "mfma", "achieved": flops / (dec_ms * 1e-3) / 1e12,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": alg_bytes / (dec_ms * 1e-3) / 1e9,
                "peak": PEAK_HBM_GBPS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    tr = traffic_record(w.name)
    roof["traffic"] = None if tr is None else tr["hbm_bytes_per_launch"]
    roof["kernel"] = mla.mla_decode_kernel_name(p)
    roof["kernel_ms"] = dec_ms
    roof["kernel_ms_method"] = ("HIP events around every decode launch, in a second pass of the same "
                                "steps right after the timed region (that pass: "
                                f"{ms_per_step_with_events:.4f} ms per step)")

    peaks = None if args.no_measured_peaks else measured_peaks()
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, args.cpu_sample_units)

    line = {
        "metric": ("paged MLA decode TFLOPS + HBM GB/s (h_q=128, d_qk=576, d_v=512), % of roofline"
                   if args.kernel == "decode" else
                   f"paged MLA decode TFLOPS + HBM GB/s (h_q={w.h_q}, d_qk=576, d_v=512), % of roofline"),
        "value": tflops, "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "hbm_gbps": gbps, "arithmetic_intensity": intensity,
        "settle_ms": round(settle_ms, 1), "settle_steps": settle_steps, "clock": clock,
        "config": {"workload": w.name, "batch": w.batch, "s_q": w.s_q, "h_q": w.h_q,
                   "kv_format": "bf16" if w.kv_format == 0 else "fp8_656", "topk": w.topk,
                   "is_causal": w.is_causal, "sum_seqlen": int(w.cache_seqlens.astype(np.int64).sum()),
                   "num_parts": plan.num_parts, "kv_copies": copies,
                   "flops_per_step": flops, "algorithmic_bytes_per_step": alg_bytes},
        "roofline": roof,
        "measured_peaks": with_measured(roof, peaks),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
