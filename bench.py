#!/usr/bin/env python3
"""Benchmark of libattn's causal GQA attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME | --all] [--no-cpu-baseline]

A step is one forward pass (one kernel launch) over the whole workload: the
LLaMA3-70B-shaped B=64 S=8192 Hq=64 Hkv=8 D=128 causal configuration by
default, inputs seeded N(0,1) fp16 and resident in HBM before timing.  W
untimed steps, then exactly K steps between two device synchronisations
(defaults: W = 3, K = 20 for the bench workload; see below for short ones).
Rank 0 prints one JSON line per workload:

  value      whole-job TFLOP/s = metric FLOPs (2*B*Hq*S^2*D) * K / wall time
  roofline   the kernel against the MFMA roofline: metric FLOPs per launch over
             the average launch duration from HIP events on the launch stream,
             against MI355X's published dense fp16 MFMA peak (2.5 PFLOP/s);
             traffic = HBM bytes per launch from the committed rocprofv3
             counter summary (null if that summary is for another kernel build)
  peak_derived  the same peak from the runtime's compute-unit count and peak
             clock (CUs x clock x 4096 FLOP/clk), with the derivation;
             pct_of_mfma_peak is taken against it
  mfma_ceiling  context: the rate this box's matrix cores sustain on random
             operands with nothing else to do (attn_mfma_ceiling, measured after
             the timed region; not with --no-per-config), and the kernel's
             rate as a fraction of it
  variant    the kernel variant that ran (schedule, ring, xcd, lpt)
  per_config (default workload only) the other four attention configurations,
             each timed in the same run under the --all warmup rule below:
             TFLOP/s, % of peak, kernel ms per launch and variant
  cpu_baseline  the fp64 CPU oracle timed on the host on a bounded sample of
             rows of the same workload (a baseline, not a target), with the
             host CPU model

`--pmc-copy BYTES` also launches a plain elementwise copy (negation) kernel that
reads and writes BYTES bytes after the timed region (counter calibration for the HBM traffic figure), and
`--summarize-traffic FETCH_DIR WRITE_DIR` turns two rocprofv3 --pmc runs
(FETCH_SIZE, then WRITE_SIZE) into the traffic summary under profiles/, and
`--summarize-kernel-trace TRACE_DIR COMMAND` writes the kernel-trace summary,
and `--summarize-counters DIR [DIR ...]` the summary of rocprofv3 --pmc runs of
SQ/GRBM counters (MFMA busy fraction, VALU/MFMA co-execution, LDS activity).

`--workload gemm_8k_nn` / `gemm_8k_nt` time the fp16 GEMM instead (the 8k
MatMul: M = N = K = 8192, B stored [K,N] or [N,K]); its line has the same
fields, with metric FLOPs 2*M*N*K and the fp64 GEMM oracle as cpu_baseline.
`--workload llama3-70b_decode_b64_s8192` times the split-KV decode path
(attn_fwd_decode: split kernel + combine kernel per step) and reports HBM
GB/s (K, V, Q, O and LSE once) against the 8 TB/s HBM roofline.
`--variants` prints one line per attention variant shape (inputs.VARIANT_SHAPES: non-causal, sequence
lengths off the tiles, chunked prefill, head dimensions 64 and 256), FLOPs counted exactly as 4*D per
computed (query, key) pair.
`--all` prints one line per attention, GEMM and decode workload.  Without --steps / --warmup, and
under --all, each workload gets at least about 0.25 s of warmup and 0.25 s of timed launches (20
and 3 for the long ones, more launches for the short ones, reported in the line), so that its
launches are timed at the clock a sustained run settles to rather than while the clock is still
rising after input generation; --steps / --warmup given alone are used exactly.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "causal attention fwd TFLOP/s (fp16) + % of MFMA peak, LLaMA3 shapes"
VARIANT_METRIC = "attention fwd TFLOP/s (fp16), 4*D FLOPs per computed (query, key) pair"
PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published
DEFAULT_WORKLOAD = "llama3-70b_b64_s8192"
KERNEL_NAME = "attn_fwd_kernel"
WIDE_KERNEL_NAME = "attn_wide_kernel"
MFMA_FP16_FLOP_PER_CU_CLK = 4 * 1024  # gfx950: 4 SIMDs, each 1024 dense fp16 MFMA FLOP per clock
GEMM_METRIC = "fp16 GEMM TFLOP/s (8k MatMul, fp32 accumulation) + % of MFMA peak"
GEMM_KERNEL_NAME = "gemm_kernel"
DECODE_METRIC = "split-KV decode attention, HBM GB/s (K/V/Q/O/LSE once) + % of HBM peak"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def is_gemm(workload: str) -> bool:
    from dnn_compiler_pipelining_amd import inputs

    return workload in inputs.GEMM_BY_NAME


def is_decode(workload: str) -> bool:
    from dnn_compiler_pipelining_amd import inputs

    return workload in inputs.DECODE_BY_NAME


def tuned_variant(workload: str, schedule: str | None = None) -> dict | None:
    """The attention variant that runs `workload` (the library's tuned choice, or `schedule` forced)."""
    from dnn_compiler_pipelining_amd import binding, inputs

    if is_gemm(workload) or is_decode(workload):
        return None
    w = inputs.BY_NAME[workload]
    v = binding.attn_tuned_variant(w.B, w.S, w.S, w.Hq, w.Hkv, w.D)
    if schedule:
        v["schedule"] = schedule
    return v


def kernel_name(workload: str, schedule: str | None = None) -> str:
    """Symbol (substring) of the kernel that runs `workload`."""
    if is_gemm(workload):
        return GEMM_KERNEL_NAME
    if is_decode(workload):
        return KERNEL_NAME
    return WIDE_KERNEL_NAME if tuned_variant(workload, schedule)["schedule"] == "wide" else KERNEL_NAME


PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_fingerprint(workload: str = DEFAULT_WORKLOAD) -> str:
    """sha256 over the sources and build flags of the kernel that runs `workload`: identifies the measured
    kernel build."""
    from dnn_compiler_pipelining_amd import build as hipbuild

    if is_gemm(workload):
        files = hipbuild.GEMM_SOURCES + [os.path.join(hipbuild.CSRC, n) for n in ("gemm_kernel.h", "gfx950.h")]
    else:
        files = hipbuild.ATTN_SOURCES + [os.path.join(hipbuild.CSRC, n) for n in
                                         ("attn_kernel.h", "attn_tile.h", "attn_wide.h", "variant.h", "tuned_table.h",
                                          "gfx950.h")]
    h = hashlib.sha256()
    for path in files:
        with open(path, "rb") as f:
            h.update(f.read())
    h.update(" ".join(hipbuild.HIP_FLAGS[:9]).encode())
    return h.hexdigest()[:16]


def traffic_path(workload: str) -> str:
    return os.path.join(PROFILES, "hbm_traffic_%s.json" % workload)


def load_traffic(workload: str):
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_fingerprint") != kernel_fingerprint(workload):
        return None
    return t


# ------------------------------------------------------------------ GPU timing

def device_info() -> dict:
    """The GPU the line was measured on (torch's view of the HIP device properties)."""
    import torch

    pr = torch.cuda.get_device_properties(0)
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", None), "compute_units": pr.multi_processor_count,
            "memory_gib": round(pr.total_memory / 2**30, 1)}


def mfma_peak() -> dict:
    """Dense fp16 MFMA peak of device 0 from the runtime's compute-unit count and peak clock, with the
    derivation, beside the published figure."""
    from dnn_compiler_pipelining_amd import binding

    cu, khz = binding.attn_device_clock(0)
    tf = cu * khz * 1e3 * MFMA_FP16_FLOP_PER_CU_CLK / 1e12
    return {"tflops": round(tf, 1), "derivation": "%d CUs x %.3f GHz x %d FLOP/clk/CU (dense fp16 MFMA)" %
            (cu, khz / 1e6, MFMA_FP16_FLOP_PER_CU_CLK), "published_tflops": PEAK_TFLOPS}


def mfma_ceiling(achieved: float, shape: int = 32) -> dict:
    """The box's sustained MFMA-only rate on random operands for the instruction the kernel runs (`shape` 32:
    v_mfma_f32_32x32x16_f16, the attention kernels; 16: v_mfma_f32_16x16x32_f16, the GEMM), measured after
    the timed region (context for `achieved`: under the power limit it varies from box to box and sits well
    below the published peak)."""
    from dnn_compiler_pipelining_amd import binding

    tf = binding.attn_mfma_ceiling_shape(shape, 200000)
    name = "v_mfma_f32_32x32x16_f16" if shape == 32 else "v_mfma_f32_16x16x32_f16"
    return {"tflops": round(tf, 1), "frac": round(achieved / tf, 4),
            "method": "attn_mfma_ceiling_shape(%d): back-to-back %s (the kernel's MFMA) on random fp16 operands, one "
                      "wave per SIMD on every CU, timed with HIP events in this run after the timed region"
                      % (shape, name)}


def cpu_model() -> str | None:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def calibration_copy(nbytes: int):
    """One elementwise kernel that reads and writes `nbytes` bytes each: the reference reading for the
    FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    n = nbytes // 2
    src = torch.ones(n, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log("[bench] calibration copy of %d bytes done" % (2 * n))
    del src, dst


def time_workload(w, steps: int, warmup: int, pmc_copy: int = 0, variant=None):
    import torch

    from dnn_compiler_pipelining_amd import binding, inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("[bench] %s: generating seeded inputs" % w.name)
    q, k, v = inputs.make_inputs(w, dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()

    def step():
        binding.forward(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream, variant=variant)

    log("[bench] %s: %d warmup steps" % (w.name, warmup))
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    log("[bench] %s: %d timed steps" % (w.name, steps))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / steps
    kernel_ms = e0.elapsed_time(e1) / steps
    ok = bool(torch.isfinite(o[-1, -1]).all().item()) and bool(torch.isfinite(lse[-1, -1]).all().item())
    if pmc_copy:
        calibration_copy(pmc_copy)
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return wall_ms, kernel_ms, ok


def time_variant(w, steps: int, warmup: int):
    """Time one attention variant shape (inputs.VariantShape): HIP events on the launch stream around
    `steps` launches after `warmup`.  Returns (wall ms, kernel ms per launch, finite output)."""
    import torch

    from dnn_compiler_pipelining_amd import binding, inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("[bench] %s: generating seeded inputs" % w.name)
    q, k, v = inputs.make_variant_inputs(w, dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()

    def step():
        binding.forward(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    kernel_ms = e0.elapsed_time(e1) / steps
    ok = bool(torch.isfinite(o).all().item()) and bool(torch.isfinite(lse).all().item())
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return wall_ms, kernel_ms, ok


def time_gemm(w, steps: int, warmup: int, pmc_copy: int = 0):
    import torch

    from dnn_compiler_pipelining_amd import binding, inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("[bench] %s: generating seeded inputs" % w.name)
    a, b = inputs.make_gemm_inputs(w, dev)
    c = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()

    def step():
        binding.matmul(a, b, w.b_layout, out=c, stream=stream)

    log("[bench] %s: %d warmup steps" % (w.name, warmup))
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    log("[bench] %s: %d timed steps" % (w.name, steps))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / steps
    kernel_ms = e0.elapsed_time(e1) / steps
    ok = bool(torch.isfinite(c[-1]).all().item())
    if pmc_copy:
        calibration_copy(pmc_copy)
    del a, b, c
    torch.cuda.empty_cache()
    return wall_ms, kernel_ms, ok


def time_decode(w, steps: int, warmup: int, pmc_copy: int = 0):
    import torch

    from dnn_compiler_pipelining_amd import binding, inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("[bench] %s: generating seeded inputs" % w.name)
    q, k, v = inputs.make_decode_inputs(w, dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    need = binding.attn_decode_workspace_size(w.B, w.Sq, w.Sk, w.Hq, w.Hkv, w.D)
    ws = torch.empty(((need + 3) // 4,), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()

    def step():
        binding.decode(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, workspace=ws, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    log("[bench] %s: %d timed steps" % (w.name, steps))
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ok = bool(torch.isfinite(o).all().item())
    if pmc_copy:
        calibration_copy(pmc_copy)
    del q, k, v, o, lse, ws
    torch.cuda.empty_cache()
    return (t1 - t0) * 1e3 / steps, e0.elapsed_time(e1) / steps, ok


def cpu_baseline_decode(w, target_s: float = 15.0):
    """Times the fp64 oracle on (head, query row) outputs of batch entries in turn, in the decode metric's
    unit: each output row accounts for its share of the algorithmic bytes."""
    import numpy as np

    from dnn_compiler_pipelining_amd import inputs
    from oracle import oracle as oracle_mod

    threads = oracle_mod.default_threads()
    per_row = w.bytes / (w.B * w.Hq * w.Sq)
    rows = secs = 0.0
    b = 0
    while secs < target_s and b < w.B:
        q = inputs.make_slice(w.Sq, w.Hq, w.D, w.seed, inputs.Q, b).numpy()
        k = inputs.make_slice(w.Sk, w.Hkv, w.D, w.seed, inputs.K, b).numpy()
        v = inputs.make_slice(w.Sk, w.Hkv, w.D, w.seed, inputs.V, b).numpy()
        hs = np.repeat(np.arange(w.Hq, dtype=np.int32), w.Sq)
        rs = np.tile(np.arange(w.Sq, dtype=np.int32), w.Hq)
        t = time.perf_counter()
        oracle_mod.attn_rows(q, k, v, hs, rs, w.causal, w.scale, nthreads=threads)
        secs += time.perf_counter() - t
        rows += len(hs)
        b += 1
    log("[bench] cpu oracle: %d threads, %d batch entries in %.1f s" % (threads, b, secs))
    return {"value": round(rows * per_row / secs / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "all %d (head, row) outputs of %d batch entries of %s, fp64, %.1f s wall; bytes = the "
                      "workload's algorithmic bytes per output row" % (w.Hq * w.Sq, b, w.name, secs)}


def per_config(skip: str, schedule: str | None, peak: dict) -> dict:
    """{workload: rates} for every attention workload but `skip`: at least about 0.25 s of warmup and 0.25 s
    of timed launches each (as --all), so each is timed at the clock a sustained run settles to."""
    from dnn_compiler_pipelining_amd import inputs

    out = {}
    for w in inputs.WORKLOADS:
        if w.name == skip:
            continue
        n = min(5000, max(1, int(250.0 / max(w.flops / 8e11, 1e-3)) + 1))
        wall_ms, kernel_ms, ok = time_workload(w, n, n, 0, schedule)
        if not ok:
            raise RuntimeError("non-finite output in %s" % w.name)
        value = w.flops / (wall_ms * 1e-3) / 1e12
        achieved = w.flops / (kernel_ms * 1e-3) / 1e12
        out[w.name] = {"tflops": round(value, 2), "pct_of_mfma_peak": round(100.0 * value / peak["tflops"], 2),
                       "kernel_tflops": round(achieved, 2), "kernel_ms": round(kernel_ms, 4),
                       "ms_per_step": round(wall_ms, 4), "steps": n, "warmup": n,
                       "variant": tuned_variant(w.name, schedule), "config": w.describe()}
        log("[bench] %s: %.1f TFLOP/s (%.4f ms per launch)" % (w.name, value, kernel_ms))
    return out


# ------------------------------------------------------------------ CPU oracle baseline

def cpu_baseline(w, target_s: float = 15.0):
    """Times the fp64 oracle on rows of batch entry 0 (uniformly random rows, all heads)."""
    import numpy as np

    from dnn_compiler_pipelining_amd import inputs
    from oracle import oracle as oracle_mod

    threads = oracle_mod.default_threads()
    qb, kb, vb = inputs.make_batch_cpu(w, 0)
    qn, kn, vn = qb.numpy(), kb.numpy(), vb.numpy()
    rng = np.random.default_rng(12345)

    def run(nrows):
        heads = rng.integers(0, w.Hq, nrows).astype(np.int32)
        rows = rng.integers(0, w.S, nrows).astype(np.int32)
        keys = (rows.astype(np.float64) + 1.0) if w.causal else np.full(nrows, float(w.S))
        flops = float(4.0 * w.D * keys.sum())  # QK^T and PV over the allowed keys of each row
        t = time.perf_counter()
        oracle_mod.attn_rows(qn, kn, vn, heads, rows, w.causal, w.scale, nthreads=threads)
        return flops, time.perf_counter() - t

    f0, t0 = run(256 * threads)  # calibration (includes widening K/V of the batch entry once)
    rate = f0 / max(t0, 1e-6)
    avg_row = 4.0 * w.D * ((w.S + 1) / 2.0 if w.causal else w.S)
    n = int(min(max(rate * max(target_s - t0, 1.0) / avg_row, 64), 4_000_000))
    log("[bench] cpu oracle: %d threads, %.2f GFLOP/s calibration, timing %d rows" % (threads, rate / 1e9, n))
    f1, t1 = run(n)
    flops, secs = f0 + f1, t0 + t1
    return {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d (head,row) outputs of batch entry 0 of %s (rows uniform in [0,S), heads uniform), "
                      "fp64, %.1f s wall; FLOPs = 4*D*(allowed keys) per row" % (256 * threads + n, w.name, secs)}


def cpu_baseline_gemm(w, target_s: float = 15.0):
    """Times the fp64 GEMM oracle (numpy's float64 matmul) on blocks of rows of C."""
    import numpy as np

    from dnn_compiler_pipelining_amd import inputs
    from oracle import gemm_oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    a, b = inputs.make_gemm_inputs(w)
    an, bn = a.numpy(), b.numpy()
    order = np.random.default_rng(54321).permutation(w.M)
    flops = secs = 0.0
    done = 0
    while secs < target_s and done < w.M:  # blocks of 512 rows of C until the target time is reached
        rows = np.sort(order[done:done + 512])
        t = time.perf_counter()
        gemm_oracle.gemm_rows(an, bn, w.b_layout, rows)
        secs += time.perf_counter() - t
        flops += 2.0 * len(rows) * w.N * w.K
        done += len(rows)
    log("[bench] cpu oracle: %d BLAS threads, %d rows in %.1f s" % (threads, done, secs))
    return {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d rows of C (uniform without replacement, blocks of 512) of %s, binary64, %.1f s wall; "
                      "FLOPs = 2*N*K per row" % (done, w.name, secs)}


# ------------------------------------------------------------------ traffic summary from rocprofv3 --pmc runs

def _db_files(d: str):
    files = glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True)
    if not files:
        raise FileNotFoundError("no rocprofv3 *_results.db under %s" % d)
    return files


def _per_dispatch(d: str, counter: str):
    """{(kernel_name, dispatch_id): value} for one counter of a rocprofv3 --pmc run (rocpd SQLite output)."""
    import sqlite3

    out = {}
    for f in _db_files(d):
        con = sqlite3.connect(f)
        for name, disp, val in con.execute(
                "select kernel_name, dispatch_id, value from counters_collection where counter_name = ?", (counter,)):
            out[(name, disp)] = out.get((name, disp), 0.0) + float(val)
        con.close()
    return out


def summarize_kernel_trace(d: str, workload: str, command: str, schedule: str | None = None):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run, written under profiles/."""
    import sqlite3

    lines = ["# rocprofv3 kernel trace: %s" % workload, "", "Command (from the repository root):", "",
             "    " + command, "", "| kernel | calls | average us | total us | share % |", "|---|---|---|---|---|"]
    info = None
    kn = kernel_name(workload, schedule)
    for f in _db_files(d):
        con = sqlite3.connect(f)
        for name, calls, total, avg, pct in con.execute(
                "select name, total_calls, total_duration, average, percentage from top_kernels"):
            short = name if len(name) < 70 else name[:67] + "..."
            lines.append("| `%s` | %d | %.1f | %.1f | %.3f |" % (short, calls, avg, total, pct))
        row = con.execute("select grid_x, workgroup_x, lds_size, scratch_size, vgpr_count, accum_vgpr_count, "
                          "sgpr_count from kernels where name like ? limit 1", ("%" + kn + "%",)).fetchone()
        if row:
            info = row
        con.close()
    if info:
        lines += ["", "%s dispatch: grid %d work-items, workgroup %d, LDS %d B, scratch %d B, vgpr_count %d, "
                      "accum_vgpr_count %d, sgpr_count %d (as the trace reports them)" % ((kn,) + tuple(info))]
    lines += ["", "Kernel source fingerprint: %s" % kernel_fingerprint(workload), ""]
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, "%s_%s_kernel_trace.md" % (kn, workload))
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def summarize_traffic(fetch_dir: str, write_dir: str, workload: str, copy_bytes: int, schedule: str | None = None):
    res = {}
    # a step of the decode workload is two kernels (the split kernel and the combine kernel): its bytes are the
    # sum of their per-dispatch means
    knames = ("attn_fwd_kernel", "attn_combine_kernel") if is_decode(workload) else (kernel_name(workload, schedule),)
    knm = " + ".join(knames)
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = _per_dispatch(d, counter)
        per_kernel = {n: [v for (kn, _), v in vals.items() if n in kn] for n in knames}
        other = [(kn, v) for (kn, _), v in vals.items() if not any(n in kn for n in knames)]
        if not all(per_kernel.values()):
            raise RuntimeError("no %s dispatches in %s" % (knm, d))
        # the calibration copy is the largest dispatch of another kernel
        copy_kib = max(v for _, v in other) if other else 0.0
        factor = copy_bytes / (copy_kib * 1024.0) if copy_kib else None
        raw = sum(sum(v) / len(v) for v in per_kernel.values()) * 1024.0
        launches = min(len(v) for v in per_kernel.values())
        res[counter] = {"kib_per_launch": raw / 1024.0, "launches": launches, "copy_kib": copy_kib,
                        "copy_bytes": copy_bytes, "factor": factor,
                        "bytes_per_launch": raw * factor if factor else None}
    total = None
    if res["FETCH_SIZE"]["bytes_per_launch"] and res["WRITE_SIZE"]["bytes_per_launch"]:
        total = res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"]
    from dnn_compiler_pipelining_amd import inputs

    if is_gemm(workload):
        g = inputs.GEMM_BY_NAME[workload]
        algo = 2 * (g.M * g.K + g.K * g.N + g.M * g.N)
    elif is_decode(workload):
        algo = inputs.DECODE_BY_NAME[workload].bytes
    else:
        w = inputs.BY_NAME[workload]
        algo = 2 * (2 * w.B * w.S * w.Hq * w.D + 2 * w.B * w.S * w.Hkv * w.D) + 4 * w.B * w.Hq * w.S
    cmd = ("rocprofv3 --pmc %s -d <dir> -o <name> -- python3 bench.py --workload %s --steps 2 --warmup 1 "
           "--no-cpu-baseline --no-per-config --pmc-copy %d")
    out = {"workload": workload, "kernel": knm, "kernel_fingerprint": kernel_fingerprint(workload),
           "hbm_bytes_per_launch": total, "algorithmic_bytes_per_launch": algo,
           "commands": [cmd % ("FETCH_SIZE", workload, copy_bytes), cmd % ("WRITE_SIZE", workload, copy_bytes),
                        "python3 bench.py --workload %s --pmc-copy %d --summarize-traffic <fetch dir> <write dir>"
                        % (workload, copy_bytes)],
           "calibration": "each counter is scaled by copy_bytes / (its reading for an elementwise kernel that "
                          "reads and writes copy_bytes bytes, launched in the same run)",
           "counters": res}
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_path(workload), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def summarize_counters(dirs, workload: str, schedule: str | None = None):
    """Markdown summary of rocprofv3 --pmc runs of SQ/GRBM counters for the attention kernel.

    Per-dispatch averages of each counter (summed over the device), plus derived figures:
    per-SIMD MFMA busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs * GRBM_GUI_ACTIVE / XCDs),
    co-execution share = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES.
    """
    import sqlite3

    n_xcd, n_simd = 8, 256 * 4
    vals, cmds = {}, []
    for d in dirs:
        names = set()
        for f in _db_files(d):
            con = sqlite3.connect(f)
            for name, counter, val, n in con.execute(
                    "select kernel_name, counter_name, sum(value), count(distinct dispatch_id) from counters_collection "
                    "where kernel_name like ? group by kernel_name, counter_name", ("%" + kernel_name(workload, schedule) + "%",)):
                vals[counter] = val / max(n, 1)
                names.add(counter)
            con.close()
        cmds.append("rocprofv3 --pmc %s -d <dir> -o <name> -- python3 bench.py --workload %s --steps 2 --warmup 1 "
                    "--no-cpu-baseline --no-per-config" % (" ".join(sorted(names)), workload))
    lines = ["# rocprofv3 counters: %s, %s" % (kernel_name(workload, schedule), workload), "", "Commands (from the repository root; one "
             "--pmc pass per line, counters grouped within the per-block limits):", ""]
    lines += ["    " + c for c in cmds]
    lines += ["", "Values are per dispatch of %s, summed over the device." % kernel_name(workload, schedule), "",
              "| counter | per dispatch |", "|---|---|"]
    for k in sorted(vals):
        lines.append("| %s | %.4g |" % (k, vals[k]))
    gui = vals.get("GRBM_GUI_ACTIVE")
    if gui:
        cyc = gui / n_xcd
        lines += ["", "Derived:", "", "- active cycles per XCD: %.4g" % cyc]
        if "SQ_VALU_MFMA_BUSY_CYCLES" in vals:
            lines.append("- MFMA busy per SIMD: %.1f %% of active cycles" %
                         (100.0 * vals["SQ_VALU_MFMA_BUSY_CYCLES"] / (n_simd * cyc)))
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in vals and vals.get("SQ_VALU_MFMA_BUSY_CYCLES"):
            lines.append("- VALU issued during MFMA busy cycles: %.1f %% of MFMA busy cycles" %
                         (100.0 * vals["SQ_VALU_MFMA_COEXEC_CYCLES"] / vals["SQ_VALU_MFMA_BUSY_CYCLES"]))
        if "SQ_LDS_IDX_ACTIVE" in vals:
            lines.append("- LDS indexed-access active: %.1f %% of active cycles per CU" %
                         (100.0 * vals["SQ_LDS_IDX_ACTIVE"] / (256 * cyc)))
    lines += ["", "Kernel source fingerprint: %s" % kernel_fingerprint(workload), ""]
    os.makedirs(PROFILES, exist_ok=True)
    out = os.path.join(PROFILES, "%s_%s_counters.md" % (kernel_name(workload, schedule), workload))
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def launch_counts(est_ms: float, steps: int | None, warmup: int | None, all_workloads: bool) -> tuple[int, int]:
    """(timed launches, warmup launches) for a workload whose launch takes about `est_ms`.  A count given on
    the command line is used as given (under --all: at least that many).  Otherwise, and under --all, each
    workload gets at least ~0.25 s of warmup and of timed launches (20 and 3 at least), so that short launches
    are timed at the clock a sustained run settles to, not while it is still rising."""
    n = min(5000, max(1, int(250.0 / max(est_ms, 1e-3)) + 1))  # launch-bound shapes: at most 5000
    k = steps if steps is not None and not all_workloads else max(steps or 20, n)
    w = warmup if warmup is not None and not all_workloads else max(warmup or 3, n)
    return k, w


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed launches (default: 20, or more for short workloads, about 0.25 s in all)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed launches before them (default: 3, or more for short workloads, about 0.25 s)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--all", action="store_true", help="one line per workload (parity-test configurations too)")
    ap.add_argument("--variants", action="store_true",
                    help="one line per attention variant shape (non-causal, ragged S, chunked prefill, D 64 / 256)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="time only the named workload (profiling runs: no other configuration's launches)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--pmc-copy", type=int, default=0)
    ap.add_argument("--schedule", default=None, help="attention tile schedule to time instead of the tuned one "
                    "(serial, overlap, pingpong, serial4, wide), for same-box comparisons")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-kernel-trace", nargs=2, metavar=("TRACE_DIR", "COMMAND"))
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR")
    args = ap.parse_args()

    from dnn_compiler_pipelining_amd import inputs

    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.workload, args.schedule)
        return
    if args.summarize_kernel_trace:
        summarize_kernel_trace(args.summarize_kernel_trace[0], args.workload, args.summarize_kernel_trace[1], args.schedule)
        return 0
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic[0], args.summarize_traffic[1], args.workload, args.pmc_copy, args.schedule)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build measures one MI355X's share of the workload; "
              "--gpus %d (WORLD_SIZE %d) is not supported" % (args.gpus, world), file=sys.stderr)
        return 2

    names = ([w.name for w in inputs.WORKLOADS] + [w.name for w in inputs.GEMM_WORKLOADS] +
             [w.name for w in inputs.DECODE_WORKLOADS]) if args.all else [args.workload]

    def counts(est_ms: float):
        return launch_counts(est_ms, args.steps, args.warmup, args.all or args.variants)

    peak = mfma_peak()
    log("[bench] dense fp16 MFMA peak: %.1f TFLOP/s = %s (published %.0f)" %
        (peak["tflops"], peak["derivation"], PEAK_TFLOPS))
    if args.variants:
        from dnn_compiler_pipelining_amd import binding

        for w in inputs.VARIANT_SHAPES:
            steps, warmup = counts(w.flops / 8e11)
            wall_ms, kernel_ms, ok = time_variant(w, steps, warmup)
            if not ok:
                log("[bench] non-finite output in %s" % w.name)
                return 1
            value = w.flops / (wall_ms * 1e-3) / 1e12
            achieved = w.flops / (kernel_ms * 1e-3) / 1e12
            line = {"metric": VARIANT_METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
                    "steps": steps, "warmup": warmup, "ms_per_step": round(wall_ms, 4), "higher_is_better": True,
                    "scaling": "weak", "vs_baseline": None, "dtype": "f16",
                    "data": "synthetic: seeded i.i.d. N(0,1) fp16 Q/K/V",
                    "pct_of_mfma_peak": round(100.0 * value / peak["tflops"], 2), "config": w.describe(),
                    "kernel_ms": round(kernel_ms, 4), "kernel_tflops": round(achieved, 2),
                    "flops_per_launch": w.flops,
                    "variant": binding.attn_tuned_variant(w.B, w.Sq, w.Sk, w.Hq, w.Hkv, w.D),
                    "device": device_info()}
            print(json.dumps(line), flush=True)
        return 0
    for name in names:
        if is_decode(name):
            w = inputs.DECODE_BY_NAME[name]
            steps, warmup = counts(w.bytes / 5e9)
            wall_ms, kernel_ms, ok = time_decode(w, steps, warmup, args.pmc_copy)
            traffic = load_traffic(w.name)
            if not ok:
                log("[bench] non-finite output")
                return 1
            value = w.bytes / (wall_ms * 1e-3) / 1e9
            achieved = w.bytes / (kernel_ms * 1e-3) / 1e9
            line = {"metric": DECODE_METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
                    "steps": steps, "warmup": warmup, "ms_per_step": round(wall_ms, 4),
                    "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
                    "data": "synthetic: seeded i.i.d. N(0,1) fp16 Q/K/V", "config": w.describe(),
                    "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round(achieved / HBM_PEAK_GBS, 4),
                                 "traffic": (round(traffic["hbm_bytes_per_launch"])
                                             if traffic and traffic.get("hbm_bytes_per_launch") else None),
                                 "kernel": "attn_fwd_kernel (split-KV) + attn_combine_kernel",
                                 "kernel_ms": round(kernel_ms, 4), "bytes_per_step": w.bytes},
                    "device": device_info()}
            if not args.no_cpu_baseline and not args.all:
                line["cpu_baseline"] = cpu_baseline_decode(w, args.cpu_seconds)
            print(json.dumps(line), flush=True)
            continue
        gemm = is_gemm(name)
        if gemm:
            w = inputs.GEMM_BY_NAME[name]
            steps, warmup = counts(w.flops / 8e11)
            wall_ms, kernel_ms, ok = time_gemm(w, steps, warmup, args.pmc_copy)
        else:
            w = inputs.BY_NAME[name]
            steps, warmup = counts(w.flops / 8e11)
            wall_ms, kernel_ms, ok = time_workload(w, steps, warmup, args.pmc_copy, args.schedule)
        if not ok:
            log("[bench] non-finite output")
            return 1
        value = w.flops / (wall_ms * 1e-3) / 1e12
        achieved = w.flops / (kernel_ms * 1e-3) / 1e12
        traffic = load_traffic(w.name)
        line = {
            "metric": GEMM_METRIC if gemm else METRIC,
            "value": round(value, 2),
            "unit": "TFLOP/s",
            "n_gpus": 1,
            "steps": steps,
            "warmup": warmup,
            "ms_per_step": round(wall_ms, 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "f16",
            "data": "synthetic: seeded i.i.d. N(0,1) fp16 %s" % ("A/B" if gemm else "Q/K/V"),
            "pct_of_mfma_peak": round(100.0 * value / peak["tflops"], 2),
            "config": w.describe(),
            "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(achieved / PEAK_TFLOPS, 4),
                         "traffic": (round(traffic["hbm_bytes_per_launch"])
                                     if traffic and traffic.get("hbm_bytes_per_launch") else None),
                         "kernel": kernel_name(name, args.schedule), "kernel_ms": round(kernel_ms, 4),
                         "flops_per_launch": w.flops},
            "peak_derived": dict(peak, frac=round(achieved / peak["tflops"], 4)),
            "device": device_info(),
        }
        if not gemm:
            line["variant"] = tuned_variant(name, args.schedule)
        if not args.all and not args.no_per_config and not gemm and name == DEFAULT_WORKLOAD:
            # the other attention configurations, each timed under the --all warmup rule, in the same run
            line["per_config"] = per_config(w.name, args.schedule, peak)
        if not args.all and not args.no_per_config:
            line["mfma_ceiling"] = mfma_ceiling(achieved, 16 if gemm else 32)
        if not args.no_cpu_baseline and not args.all:
            line["cpu_baseline"] = (cpu_baseline_gemm if gemm else cpu_baseline)(w, args.cpu_seconds)
            line["cpu_baseline"]["cpu_model"] = cpu_model()
        print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
