#!/usr/bin/env python3
"""Decode-step benchmark for paged-KV decode attention on one MI355X.

A step is one pass of the whole hot path over one decode batch: the slot
write of each sequence's new K/V (paged_kv_write) followed by the fused paged
decode attention (paged_decode_attention, plus its log-sum-exp merge when the
context is split).  Inputs are seeded synthetic batches (see
paged_kv_decode_13_amd/workloads.py) uploaded to HBM before the timed region.

Prints ONE JSON line on stdout.  The headline is the GQA batch-256 bf16
workload: ``value`` is the effective KV-read bandwidth of the whole step,
sum(ctx) * num_kv_heads * head_dim * 2 * bytes / step time; ``roofline``
rates the decode call alone (HIP events on the launch stream) against the
8 TB/s HBM peak; ``parity`` is max |gpu - oracle| over every output of the
timed run; ``graph`` times the step replayed from a captured HIP graph;
``cold`` repeats it with L2 and the MALL flushed before each step;
``stream_read`` is a plain contiguous read (libpkvstream.so) as the
achievable-read yardstick; ``cpu_baseline`` is the fp64 oracle timed on the
same batch on the host cores.

``configs`` holds one record per workload measured in the same run: the
single-sequence fp32 step (latency), the MHA, long-context and 8-bit (E4M3)
decode batches, the shared-prefix batch at block sizes 8/16/32/64 through
both decode entry points, the bulk prompt write and the causal prefill.
Each record carries its algorithmic bytes (or flops), call time, roofline
fraction, the counter-measured HBM traffic recorded for the current kernel
sources (else null), parity against the oracle computed in this run, and the
oracle's own time on the host (median of 3 runs; a 1-thread run as well for
the fp32 and MHA batches).  Any parity failure makes the run exit with 1.

Usage: python bench.py [--steps K] [--warmup W] [--configs all|none|a,b]
       python bench.py --config NAME [...]   (one workload, no suite)
       python bench.py --mode write|prefill --config prefill_bf16
       python bench.py --mode copy  (plain device copy, for counter scaling)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import shutil
import statistics
import subprocess
import sys
import time

REPO = os.path.dirname(os.path.abspath(__file__))
if REPO not in sys.path:
    sys.path.insert(0, REPO)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix peak, AMD published
METRIC = "effective KV-read HBM GB/s (% of MI355X peak) + decode tokens/s, paged attention"
SHARED_PREFIX_PARTITION = 1024
# time a step's slot write and decode as two launches (paged_kv_write, then
# paged_decode_attention) instead of paged_decode_step (--unfused-step)
UNFUSED_STEP = False
COLD_FLUSH_BYTES = 1 << 30   # > L2 (4 MiB per XCD) + MALL (256 MiB)
STREAM_READ_BYTES = 2 << 30  # contiguous buffer of the streaming-read yardstick
# parity bars on outputs in the cache dtype (max |gpu - oracle|)
TOL = {"f32": 1e-5, "f16": 5e-3, "bf16": 5e-3}
# the workloads beside the headline: untimed steps for at least SUITE_WARM_S
# seconds (the GPU's clock settles only after tens of milliseconds of work),
# then at least SUITE_STEPS timed steps
SUITE_WARM_S = 0.15
GRAPH_STEPS = 10  # steps captured in one graph for the host-free step time
SUITE_STEPS = 100
SUITE = ("tiny_fp32", "mha_fp16", "long_bf16", "gqa_fp8", "prefix_fp16", "write_prefill_bf16",
         "prefill_bf16")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def code_text(text: str) -> str:
    """Source text without comments and with whitespace runs collapsed:
    what the compiler sees, so comment edits keep the digest."""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif text[i] in "\"'":
            q, j = text[i], i + 1
            while j < n and text[j] != q:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(text[i])
            i += 1
    return " ".join("".join(out).split())


def source_digest(files: dict | None = None) -> str:
    """Digest of the kernel sources' code (comments and layout ignored);
    ``files`` maps file name -> text, default: the csrc directory."""
    if files is None:
        csrc = os.path.join(REPO, "paged_kv_decode_13_amd", "csrc")
        files = {}
        for f in sorted(os.listdir(csrc)):
            with open(os.path.join(csrc, f), encoding="utf-8") as fh:
                files[f] = fh.read()
    h = hashlib.sha256()
    for f in sorted(files):
        h.update(f.encode() + b"\0" + code_text(files[f]).encode())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per call measured by rocprofv3 counters, if they were taken
    on the current kernel sources (else None)."""
    path = os.path.join(REPO, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest():
        return None
    return rec.get("bytes_per_launch")


def cpu_model() -> str | None:
    """The host CPU's model name as lscpu reports it (else /proc/cpuinfo),
    with its family, model and stepping numbers, which identify the part
    where the name alone is generic."""
    fields = {}
    if shutil.which("lscpu"):
        try:
            out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=20).stdout
            for ln in out.splitlines():
                if ":" in ln:
                    k, v = ln.split(":", 1)
                    fields.setdefault(k.strip(), v.strip())
        except (OSError, subprocess.SubprocessError):
            pass
    if "Model name" not in fields:
        try:
            with open("/proc/cpuinfo") as f:
                for ln in f:
                    if ":" in ln:
                        k, v = ln.split(":", 1)
                        key = {"model name": "Model name", "cpu family": "CPU family",
                               "model": "Model", "stepping": "Stepping"}.get(k.strip())
                        if key:
                            fields.setdefault(key, v.strip())
        except OSError:
            pass
    name = fields.get("Model name")
    if name is None:
        return None
    ids = [f"{k.lower()} {fields[k]}" for k in ("CPU family", "Model", "Stepping") if k in fields]
    return f"{name} ({', '.join(ids)})" if ids else name


def upload(batch, dev):
    import torch

    from paged_kv_decode_13_amd import workloads as wl

    t = {
        "q": wl.torch_view(batch.query, batch.dtype).to(dev),
        "kc": wl.torch_view(batch.key_cache, batch.cache_dtype).to(dev),
        "vc": wl.torch_view(batch.value_cache, batch.cache_dtype).to(dev),
        "bt": torch.from_numpy(batch.block_tables).to(dev),
        "cl": torch.from_numpy(batch.context_lens).to(dev),
    }
    if batch.k_scale is not None:
        t["ks"] = torch.from_numpy(batch.k_scale).to(dev)
        t["vs"] = torch.from_numpy(batch.v_scale).to(dev)
    if batch.slot_mapping is not None:
        t["nk"] = wl.torch_view(batch.new_key, batch.dtype).to(dev)
        t["nv"] = wl.torch_view(batch.new_value, batch.dtype).to(dev)
        t["slots"] = torch.from_numpy(batch.slot_mapping).to(dev)
    return t


def _pct(xs, p: float) -> float:
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(p * len(xs)))]


def _r(x, nd: int = 5):
    return None if x is None else round(float(x), nd)


# ----------------------------------------------------------------------------
# oracle side (host): the write applied to the host pools, parity, CPU time


def host_write(batch) -> None:
    """Apply the step's slot write to the host pools with the oracle (in
    place: the GPU holds its own copy), so that the oracle's decode sees the
    same history as the GPU's."""
    import oracle

    if batch.slot_mapping is None or batch.meta.get("host_written"):
        return
    if batch.cache_dtype == "e4m3":
        oracle.paged_kv_write_e4m3(batch.new_key, batch.new_value, batch.key_cache,
                                   batch.value_cache, batch.slot_mapping, batch.k_scale,
                                   batch.v_scale, batch.dtype)
    else:
        oracle.paged_kv_write(batch.new_key, batch.new_value, batch.key_cache, batch.value_cache,
                              batch.slot_mapping)
    batch.meta["host_written"] = True


def oracle_decode(batch, threads: int = 0, shared_prefix: bool = False):
    import oracle

    if shared_prefix:
        return oracle.paged_prefix_decode(batch.query, batch.key_cache, batch.value_cache,
                                          batch.meta["prefix_table"],
                                          batch.meta["shared_prefix_tokens"], batch.block_tables,
                                          batch.context_lens, batch.block_size, batch.scale,
                                          batch.dtype, threads)
    if batch.cache_dtype == "e4m3":
        return oracle.paged_decode_e4m3(batch.query, batch.key_cache, batch.value_cache,
                                        batch.k_scale, batch.v_scale, batch.block_tables,
                                        batch.context_lens, batch.block_size, batch.scale,
                                        batch.dtype, threads)
    return oracle.paged_decode(batch.query, batch.key_cache, batch.value_cache, batch.block_tables,
                               batch.context_lens, batch.block_size, batch.scale, batch.dtype,
                               threads)


def parity(gpu_out, ref, dtype: str, compared: str) -> dict:
    """max |gpu - oracle| over the compared outputs against the bar of the
    output type (NaN anywhere counts as a failure)."""
    import numpy as np
    import torch

    got = gpu_out.to(torch.float64).cpu().numpy()
    finite = bool(np.isfinite(got).all())
    err = float(np.max(np.abs(got - ref))) if finite and got.size else (0.0 if finite else float("inf"))
    tol = TOL[dtype]
    return {"max_abs_err": err, "tol": tol, "ok": bool(finite and err <= tol), "compared": compared}


def cpu_time(fn, runs: int = 3) -> float:
    """Median wall time of ``runs`` calls (steady clock)."""
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return statistics.median(ts)


def cpu_record(batch, *, runs: int = 3, one_thread: bool = False, shared_prefix: bool = False,
               alg_bytes: int | None = None) -> dict:
    """The oracle's time on the whole batch on the host cores: median of
    ``runs``; optionally also one run on one thread."""
    import oracle

    nthreads = oracle.max_threads()
    t = cpu_time(lambda: oracle_decode(batch, 0, shared_prefix), runs)
    b = batch.kv_bytes_logical() if alg_bytes is None else alg_bytes
    rec = {"kind": "oracle", "threads": nthreads, "runs": runs, "median_s": _r(t, 6),
           "decode_tokens_per_s": _r(batch.num_seqs / t, 3), "gbs": _r(b / t / 1e9, 4),
           "sample": f"the whole batch ({batch.num_seqs} sequences, {batch.total_tokens} context "
                     "tokens), fp64 gather + softmax attention"}
    if one_thread:
        t1 = cpu_time(lambda: oracle_decode(batch, 1, shared_prefix), 1)
        rec["one_thread"] = {"threads": 1, "runs": 1, "s": _r(t1, 6),
                             "decode_tokens_per_s": _r(batch.num_seqs / t1, 3),
                             "gbs": _r(b / t1 / 1e9, 4)}
    return rec


# ----------------------------------------------------------------------------
# GPU timing


def fused_step(batch, t, shared_prefix: bool = False) -> bool:
    """Whether a step's slot write rides in the decode launch
    (paged_decode_step): a batch with new tokens and a cache that is not E4M3."""
    return ("slots" in t and batch.cache_dtype in ("f32", "f16", "bf16")
            and not shared_prefix and not UNFUSED_STEP)


def step_entry(batch, t, shared_prefix: bool = False) -> str:
    """The entry point(s) one step calls."""
    if fused_step(batch, t, shared_prefix):
        return "paged_decode_step"
    return (("paged_kv_write + " if "slots" in t else "") +
            ("paged_prefix_decode_attention" if shared_prefix else
             "paged_decode_attention_fp8" if batch.cache_dtype == "e4m3" else
             "paged_decode_attention"))


def make_calls(batch, t, partition_size: int, out, ws, shared_prefix: bool = False):
    """(write, decode) closures of one step on the current stream; with the
    fused step the write is part of the decode call and ``write`` does
    nothing."""
    import torch

    import paged_kv_decode_13_amd as pkv

    fused = fused_step(batch, t, shared_prefix)
    has_write = "slots" in t and not fused
    quant = batch.cache_dtype == "e4m3"
    ptab = None
    if shared_prefix:
        plen = batch.meta["shared_prefix_tokens"]
        ptab = torch.from_numpy(batch.meta["prefix_table"]).to(t["q"].device)

    def write():
        if has_write and quant:
            pkv.paged_kv_write_fp8(t["nk"], t["nv"], t["kc"], t["vc"], t["slots"], t["ks"], t["vs"])
        elif has_write:
            pkv.paged_kv_write(t["nk"], t["nv"], t["kc"], t["vc"], t["slots"])

    def decode():
        if fused:
            pkv.paged_decode_step(t["q"], t["kc"], t["vc"], t["nk"], t["nv"], t["slots"], t["bt"],
                                  t["cl"], batch.block_size, batch.scale,
                                  max_context_len=batch.max_context_len,
                                  partition_size=partition_size, out=out, workspace=ws)
        elif quant:
            pkv.paged_decode_attention_fp8(
                t["q"], t["kc"], t["vc"], t["ks"], t["vs"], t["bt"], t["cl"], batch.block_size,
                batch.scale, max_context_len=batch.max_context_len,
                partition_size=partition_size, out=out, workspace=ws)
        elif shared_prefix:
            pkv.paged_prefix_decode_attention(
                t["q"], t["kc"], t["vc"], ptab, plen, t["bt"], t["cl"], batch.block_size,
                batch.scale, max_context_len=batch.max_context_len,
                partition_size=partition_size, out=out, workspace=ws)
        else:
            pkv.paged_decode_attention(t["q"], t["kc"], t["vc"], t["bt"], t["cl"], batch.block_size,
                                       batch.scale, max_context_len=batch.max_context_len,
                                       partition_size=partition_size, out=out, workspace=ws)

    return write, decode


def workspace_for(batch, partition_size: int, shared_prefix: bool, dev):
    import torch

    import paged_kv_decode_13_amd as pkv

    if shared_prefix:
        need = pkv.paged_prefix_decode_workspace_size(
            batch.num_seqs, batch.num_heads, batch.num_kv_heads, batch.head_dim,
            batch.max_context_len, batch.meta["shared_prefix_tokens"], partition_size)
    else:
        need = pkv.paged_decode_workspace_size(batch.num_seqs, batch.num_heads, batch.head_dim,
                                               batch.max_context_len, partition_size)
    # any contents: the library depends on none of them
    return torch.empty(max(need, 1), dtype=torch.uint8, device=dev)


def time_steps(batch, t, partition_size: int, steps: int, warmup: int, shared_prefix: bool = False,
               cold_steps: int = 0, graph: bool = False, warm_s: float = 0.0):
    """``steps`` eager steps (write + decode) timed back to back between two
    events, after ``warmup`` untimed steps (and, with warm_s > 0, untimed
    steps until that many seconds have passed); the same steps again with
    HIP events around each part (per-call medians and p99); then,
    optionally, the step captured in a HIP graph and replayed (events around
    each replay, and the back-to-back rate), and cold steps (a 1 GiB
    read-modify-write before each)."""
    import torch

    dev = t["q"].device
    out = torch.empty((batch.num_seqs, batch.num_heads, batch.head_dim), dtype=t["q"].dtype,
                      device=dev)
    ws = workspace_for(batch, partition_size, shared_prefix, dev)
    write, decode = make_calls(batch, t, partition_size, out, ws, shared_prefix)

    for _ in range(warmup):
        write()
        decode()
    torch.cuda.synchronize()
    if warm_s > 0:
        # keep stepping until the GPU has run for warm_s seconds: short
        # workloads otherwise time the clock ramp rather than steady state
        w0 = time.perf_counter()
        while time.perf_counter() - w0 < warm_s:
            for _ in range(8):
                write()
                decode()
            torch.cuda.synchronize()
    # The K timed steps run back to back between two events: an event
    # recorded between kernels costs the stream a few microseconds (two
    # events with nothing between them read about 5 us apart), so the
    # per-call events of the medians below ride on a second pass of the same
    # K steps.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        write()
        decode()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in evs:
        e[0].record()
        write()
        e[1].record()
        decode()
        e[2].record()
    torch.cuda.synchronize()
    step_ms = [e[0].elapsed_time(e[2]) for e in evs]
    write_ms = [e[0].elapsed_time(e[1]) for e in evs]
    decode_ms = [e[1].elapsed_time(e[2]) for e in evs]
    res = {
        "ms_per_step": start.elapsed_time(end) / steps,
        "wall_ms_per_step": 1e3 * wall / steps,
        "write_ms": statistics.mean(write_ms),
        "decode_ms": statistics.mean(decode_ms),
        "decode_ms_median": statistics.median(decode_ms),
        "decode_ms_p99": _pct(decode_ms, 0.99),
        "step_ms_median": statistics.median(step_ms),
        "step_ms_p99": _pct(step_ms, 0.99),
        "out": out,
    }
    if graph:
        # the same step captured in a HIP graph (no host launch gaps between
        # the write, the decode and the merge): per-replay latency (events
        # around each replay of a one-step graph), the back-to-back replay
        # rate, and a graph of GRAPH_STEPS steps, whose replay time per step
        # is the step's GPU time with no host involvement at all
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            write()
            decode()
        for _ in range(max(1, warmup)):
            g.replay()
        torch.cuda.synchronize()
        gevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(steps)]
        for a, b in gevs:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        rep = [a.elapsed_time(b) for a, b in gevs]
        res["graph_step_ms_median"] = statistics.median(rep)
        res["graph_step_ms_p99"] = _pct(rep, 0.99)
        gs, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gs.record()
        for _ in range(steps):
            g.replay()
        ge.record()
        torch.cuda.synchronize()
        res["graph_ms_per_step"] = gs.elapsed_time(ge) / steps
        del g
        gn = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gn):
            for _ in range(GRAPH_STEPS):
                write()
                decode()
        gn.replay()
        torch.cuda.synchronize()
        reps = max(2, steps // GRAPH_STEPS)
        gs.record()
        for _ in range(reps):
            gn.replay()
        ge.record()
        torch.cuda.synchronize()
        res["graph_gpu_ms_per_step"] = gs.elapsed_time(ge) / (reps * GRAPH_STEPS)
        del gn
    if cold_steps > 0:
        # cold caches: a 1 GiB read-modify-write before each step evicts L2
        # and the MALL (tables, workspace, query, recently read pages); it
        # sits outside the events, on the same stream
        scratch = torch.zeros(COLD_FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
        cevs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(cold_steps)]
        for e in cevs:
            scratch.add_(1)
            e[0].record()
            write()
            e[1].record()
            decode()
            e[2].record()
        torch.cuda.synchronize()
        del scratch
        c_step = [e[0].elapsed_time(e[2]) for e in cevs]
        c_dec = [e[1].elapsed_time(e[2]) for e in cevs]
        res["cold"] = {
            "steps": cold_steps,
            "flush_bytes": COLD_FLUSH_BYTES,
            "step_ms_median": statistics.median(c_step),
            "step_ms_p99": _pct(c_step, 0.99),
            "decode_ms_median": statistics.median(c_dec),
            "decode_ms_p99": _pct(c_dec, 0.99),
        }
    return res


def stream_read(dev, nbytes: int = STREAM_READ_BYTES, reps: int = 10, warmup: int = 3) -> dict:
    """The plain streaming-read kernel (libpkvstream.so) over one contiguous
    buffer: what a simple stream achieves on this GPU, timed with HIP events
    on the launch stream."""
    import ctypes

    import torch

    from paged_kv_decode_13_amd import build as pkv_build

    if not os.path.exists(pkv_build.STREAM_LIB_PATH):
        raise RuntimeError(f"{pkv_build.STREAM_LIB_PATH} is missing; run build() first")
    lib = ctypes.CDLL(pkv_build.STREAM_LIB_PATH)
    lib.pkv_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.pkv_stream_read.restype = ctypes.c_int
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def once():
        rc = lib.pkv_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"pkv_stream_read failed with status {rc}")

    for _ in range(warmup):
        once()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        once()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    del buf
    return {"kernel": "stream_read_kernel (contiguous, 16-byte non-temporal loads)",
            "bytes": nbytes, "ms": round(ms, 5), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 2)}


def cpu_baseline(batch, target_s: float):
    """The oracle, untouched, on an evenly spaced sample of the batch's
    sequences (the whole batch when it fits), run repeatedly for about
    ``target_s`` seconds of host work (at least three runs); the median run."""
    import numpy as np

    import oracle
    from paged_kv_decode_13_amd import workloads as wl

    order = np.arange(batch.num_seqs)
    probe = wl.subset(batch, order[:: max(1, batch.num_seqs // 8)])
    t0 = time.perf_counter()
    oracle_decode(probe)
    probe_s = max(time.perf_counter() - t0, 1e-3)
    frac = min(1.0, target_s / 3 / probe_s * probe.total_tokens / batch.total_tokens)
    step = max(1, int(round(1.0 / frac))) if frac < 1.0 else 1
    sample = batch if step == 1 else wl.subset(batch, order[::step])
    runs, secs = [], 0.0
    while len(runs) < 3 or (secs < target_s and len(runs) < 100):
        t0 = time.perf_counter()
        oracle_decode(sample)
        runs.append(time.perf_counter() - t0)
        secs += runs[-1]
    med = statistics.median(runs)
    return {
        "value": round(sample.kv_bytes_logical() / med / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": ((f"every {step}th sequence of the same batch" if step > 1 else
                    "the whole batch") +
                   f" ({sample.num_seqs} sequences, {sample.total_tokens} context tokens), "
                   f"fp64 gather + softmax attention; median of {len(runs)} runs "
                   f"({secs:.1f} s in all)"),
        "median_s": round(med, 6),
        "runs": len(runs),
        "tokens_per_s": round(sample.num_seqs / med, 3),
        "cpu_model": cpu_model(),
        "logical_cpus": os.cpu_count(),
    }


# ----------------------------------------------------------------------------
# the suite of workloads beside the headline


def _free() -> None:
    """Return cached device memory between workloads."""
    import gc

    import torch

    gc.collect()
    torch.cuda.empty_cache()


def decode_record(batch, dev, *, steps: int, warmup: int, partition_size: int | None = None,
                  shared_prefix: bool = False, traffic_key: str | None = None,
                  cpu: bool = True, one_thread: bool = False, latency: bool = False) -> dict:
    """One decode workload: time the step, check every output against the
    oracle, time the oracle on the host."""
    t = upload(batch, dev)
    ps = batch.partition_size if partition_size is None else partition_size
    r = time_steps(batch, t, ps, steps, warmup, shared_prefix, graph=True, warm_s=SUITE_WARM_S)
    host_write(batch)
    ref = oracle_decode(batch, 0, shared_prefix)
    par = parity(r["out"], ref, batch.dtype,
                 f"all {ref.size} outputs ({batch.num_seqs} sequences x {batch.num_heads} heads "
                 f"x {batch.head_dim})")
    logical = batch.kv_bytes_logical()
    alg = batch.kv_bytes_unique() if shared_prefix else logical
    call_s = r["decode_ms_median"] * 1e-3
    gbs = alg / call_s / 1e9
    traffic = load_traffic(traffic_key) if traffic_key else None
    rec = {
        "workload": batch.name,
        "entry_point": step_entry(batch, t, shared_prefix).split(" + ")[-1],
        "num_seqs": batch.num_seqs, "num_heads": batch.num_heads,
        "num_kv_heads": batch.num_kv_heads, "head_dim": batch.head_dim,
        "block_size": batch.block_size, "partition_size": ps,
        "kv_cache_dtype": batch.cache_dtype, "context_tokens": batch.total_tokens,
        "new_tokens_written": 0 if batch.slot_mapping is None else int((batch.slot_mapping >= 0).sum()),
        "call_ms_median": _r(r["decode_ms_median"]), "call_ms_p99": _r(r["decode_ms_p99"]),
        "step_ms_median": _r(r["step_ms_median"]), "step_ms_p99": _r(r["step_ms_p99"]),
        "graph_step_ms_median": _r(r["graph_step_ms_median"]),
        "graph_step_ms_p99": _r(r["graph_step_ms_p99"]),
        "graph_ms_per_step": _r(r["graph_ms_per_step"]),
        "graph_gpu_ms_per_step": _r(r["graph_gpu_ms_per_step"]),
        "steps": steps,
        "kv_bytes_logical": logical,
        "algorithmic_bytes": alg,
        "gbs": round(gbs, 2),
        "frac": round(gbs / HBM_PEAK_GBS, 4),
        "logical_gbs": round(logical / call_s / 1e9, 2),
        "decode_tokens_per_s": round(batch.num_seqs / (r["step_ms_median"] * 1e-3), 1),
        "traffic": traffic,
        "traffic_ratio": None if traffic is None else round(traffic / alg, 4),
        "parity": par,
    }
    if latency:
        rec["latency_us"] = {k: _r(1e3 * r[v], 2) for k, v in (
            ("eager_step_median", "step_ms_median"), ("eager_step_p99", "step_ms_p99"),
            ("graph_step_median", "graph_step_ms_median"), ("graph_step_p99", "graph_step_ms_p99"),
            ("graph_back_to_back", "graph_ms_per_step"),
            ("graph_gpu_step", "graph_gpu_ms_per_step"),
            ("decode_call_median", "decode_ms_median"), ("decode_call_p99", "decode_ms_p99"))}
    if cpu:
        rec["cpu_oracle"] = cpu_record(batch, one_thread=one_thread, shared_prefix=shared_prefix,
                                       alg_bytes=alg)
    return rec


def write_record(batch, dev, *, steps: int, warmup: int) -> dict:
    """The bulk prompt write alone, then both pools compared with the
    oracle's write byte for byte."""
    import numpy as np
    import torch

    import oracle

    t = upload(batch, dev)
    r = run_write(batch, t, steps, warmup)
    kc, vc = batch.key_cache.copy(), batch.value_cache.copy()
    oracle.paged_kv_write(batch.new_key, batch.new_value, kc, vc, batch.slot_mapping)
    same = (np.array_equal(t["kc"].cpu().view(torch.uint8).numpy().ravel(), kc.view(np.uint8).ravel())
            and np.array_equal(t["vc"].cpu().view(torch.uint8).numpy().ravel(),
                               vc.view(np.uint8).ravel()))
    rec = {k: r[k] for k in ("value", "unit", "ms_per_step", "roofline")}
    rec["tokens"] = int(batch.new_key.shape[0])
    rec["bytes_moved"] = 4 * batch.new_key.nbytes
    rec["traffic"] = load_traffic("write_prefill_bf16")
    rec["parity"] = {"bit_exact": bool(same), "ok": bool(same),
                     "compared": "both pools, every byte, against the oracle's write"}
    return rec


def prefill_record(batch, dev, *, steps: int, warmup: int) -> dict:
    """The bulk write plus the causal attention of every prompt token;
    parity on a deterministic sample of query rows (every prompt, its first
    and last row and the last row of 6 evenly spaced 64-token chunks, every
    head), each against the oracle's decode of that row over the history it
    sees (a causal row at position p is the decode of context p + 1)."""
    import numpy as np
    import torch

    from paged_kv_decode_13_amd import workloads as wl

    t = upload(batch, dev)
    r = run_prefill(batch, t, steps, warmup, keep_out=True)
    out = r.pop("out")
    host_write(batch)
    qsl = batch.meta["query_start_loc"]
    rows, seqs, ctxs = [], [], []
    for s in range(batch.num_seqs):
        n = int(batch.context_lens[s])
        pos = sorted({0, n - 1, *[min(n - 1, c * 64 + 63) for c in
                                  np.linspace(0, (n - 1) // 64, 6).astype(int)]})
        for p in pos:
            rows.append(int(qsl[s]) + p)
            seqs.append(s)
            ctxs.append(p + 1)
    rows = np.asarray(rows)
    sub = wl.subset(batch, np.asarray(seqs))
    sub.query = np.ascontiguousarray(batch.meta["prompt_query"][rows])
    sub.context_lens = np.asarray(ctxs, dtype=np.int32)
    sub.slot_mapping = None
    ref = oracle_decode(sub)
    got = out[torch.from_numpy(rows).to(out.device)]
    rec = {k: r[k] for k in ("value", "unit", "ms_per_step", "prompt_tokens_per_s", "write_ms",
                             "attention_ms", "algorithmic_flops", "roofline")}
    rec["parity"] = parity(got, ref, batch.dtype,
                           f"{rows.size} query rows x {batch.num_heads} heads (every prompt's "
                           "first and last row, chunk ends across the prompt)")
    return rec


def run_suite(names, dev, steps: int, warmup: int) -> dict:
    from paged_kv_decode_13_amd import workloads as wl

    recs = {}
    steps = max(steps, SUITE_STEPS)
    for name in names:
        t0 = time.time()
        if name == "tiny_fp32":
            recs[name] = decode_record(wl.make_config(name), dev, steps=max(steps, 400),
                                       warmup=warmup, one_thread=True, latency=True)
        elif name == "mha_fp16":
            recs[name] = decode_record(wl.make_config(name), dev, steps=steps, warmup=warmup,
                                       traffic_key=name, one_thread=True)
        elif name in ("long_bf16", "gqa_fp8"):
            recs[name] = decode_record(wl.make_config(name), dev, steps=steps, warmup=warmup,
                                       traffic_key=name)
        elif name == "prefix_fp16":
            for bs in wl.PREFIX_BLOCK_SIZES:
                b = wl.make_config(name, block_size=bs)
                recs[f"prefix_fp16_bs{bs}"] = decode_record(
                    b, dev, steps=steps, warmup=warmup, traffic_key=f"prefix_fp16_bs{bs}",
                    cpu=bs == 16)
                recs[f"prefix_fp16_bs{bs}_shared"] = decode_record(
                    b, dev, steps=steps, warmup=warmup, partition_size=SHARED_PREFIX_PARTITION,
                    shared_prefix=True, traffic_key=f"prefix_fp16_bs{bs}_shared", cpu=bs == 16)
        elif name == "write_prefill_bf16":
            recs[name] = write_record(wl.make_prefill_config("prefill_bf16"), dev, steps=steps,
                                      warmup=max(warmup, 600))
        elif name == "prefill_bf16":
            b = wl.add_prompt_queries(wl.make_prefill_config(name), seed=11)
            recs[name] = prefill_record(b, dev, steps=20, warmup=16)
        else:
            raise KeyError(name)
        _free()
        log(f"[suite] {name} done in {time.time() - t0:.1f}s")
    return recs


# ----------------------------------------------------------------------------
# single-workload modes


def run_write(batch, t, steps: int, warmup: int) -> dict:
    """The slot write alone (a bulk prompt write for the prefill workload),
    timed with HIP events; bytes moved = new rows read + rows written."""
    import torch

    import paged_kv_decode_13_amd as pkv

    def write():
        pkv.paged_kv_write(t["nk"], t["nv"], t["kc"], t["vc"], t["slots"])

    for _ in range(warmup):
        write()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        write()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    moved = 2 * 2 * batch.new_key.nbytes  # K and V, read and written
    gbs = moved / (ms * 1e-3) / 1e9
    return {
        "metric": "paged KV slot write GB/s (bytes read + written)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": batch.dtype,
        "data": "synthetic (seeded N(0,1) rows, generated page tables)",
        "config": {"workload": batch.name, "tokens": int(batch.new_key.shape[0]),
                   "num_kv_heads": batch.num_kv_heads, "head_dim": batch.head_dim,
                   "block_size": batch.block_size, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "kv_write_kernel", "achieved": round(gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic("write_" + batch.name)},
        "cpu_baseline": None,
    }


def prefill_flops(batch) -> int:
    """Algorithmic flops of causal attention over the prompts: query i of a
    prompt sees i + 1 tokens; scores and values each take 2 * D flops per
    (query head, visible token)."""
    import numpy as np

    n = batch.context_lens.astype(np.int64)
    visible = int((n * (n + 1) // 2).sum())
    return 4 * batch.head_dim * batch.num_heads * visible


def run_prefill(batch, t, steps: int, warmup: int, keep_out: bool = False) -> dict:
    """One prefill step: the bulk write of every prompt token's K/V through
    slot_mapping, then causal attention of every prompt token over its
    prompt (paged_prefill_attention); HIP events on the launch stream."""
    import torch

    import paged_kv_decode_13_amd as pkv

    dev = t["q"].device
    from paged_kv_decode_13_amd import workloads as wl

    pq = wl.torch_view(batch.meta["prompt_query"], batch.dtype).to(dev)
    qsl = torch.from_numpy(batch.meta["query_start_loc"]).to(dev)
    out = torch.empty_like(pq)

    def write():
        pkv.paged_kv_write(t["nk"], t["nv"], t["kc"], t["vc"], t["slots"])

    def attend():
        pkv.paged_prefill_attention(pq, t["kc"], t["vc"], t["bt"], t["cl"], qsl, batch.block_size,
                                    batch.scale, max_context_len=batch.max_context_len, out=out)

    for _ in range(warmup):
        write()
        attend()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in evs:
        e[0].record()
        write()
        e[1].record()
        attend()
        e[2].record()
    torch.cuda.synchronize()
    step_ms = statistics.median(e[0].elapsed_time(e[2]) for e in evs)
    attn_ms = statistics.median(e[1].elapsed_time(e[2]) for e in evs)
    write_ms = statistics.median(e[0].elapsed_time(e[1]) for e in evs)
    flops = prefill_flops(batch)
    tflops = flops / (attn_ms * 1e-3) / 1e12
    tokens = int(batch.context_lens.astype("int64").sum())
    res = {
        "metric": "causal paged prefill attention TFLOP/s (+ prompt tokens/s)",
        "value": round(flops / (step_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": batch.dtype,
        "data": "synthetic (seeded N(0,1) prompts and queries, generated page tables)",
        "config": {"workload": batch.name, "prompts": batch.num_seqs, "prompt_tokens": tokens,
                   "num_heads": batch.num_heads, "num_kv_heads": batch.num_kv_heads,
                   "head_dim": batch.head_dim, "block_size": batch.block_size,
                   "parallelism": "single GPU"},
        "prompt_tokens_per_s": round(tokens / (step_ms * 1e-3), 1),
        "write_ms": round(write_ms, 4),
        "attention_ms": round(attn_ms, 4),
        "algorithmic_flops": flops,
        "roofline": {"bound": "mfma", "kernel": "paged_prefill_mfma_kernel",
                     "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": load_traffic(batch.name)},
        "cpu_baseline": None,
    }
    if keep_out:
        res["out"] = out
    return res


def run_copy(size_mb: int, steps: int) -> None:
    """A plain device-to-device copy of known size (counter calibration)."""
    import torch

    n = size_mb * (1 << 20)
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy", "bytes_read_per_copy": n, "bytes_written_per_copy": n,
                      "copies": steps}), flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="gqa_bf16")
    ap.add_argument("--configs", default=None,
                    help="workloads measured beside the headline: 'all' (the default for the "
                         "GQA headline run), 'none', or a comma list of " + ",".join(SUITE))
    ap.add_argument("--block-size", type=int, default=None, help="prefix_fp16 only")
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--sweep-partitions", default=None,
                    help="comma list of partition sizes to time as well (stderr report)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--shared-prefix", action="store_true",
                    help="prefix_fp16: decode through paged_prefix_decode_attention (the shared "
                         "prefix read once per KV head for the batch)")
    ap.add_argument("--mode", default="decode", choices=["decode", "write", "copy", "prefill"])
    ap.add_argument("--copy-mb", type=int, default=1024)
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="steps timed again with L2/MALL flushed before each (0: skip)")
    ap.add_argument("--no-stream-read", action="store_true",
                    help="skip the streaming-read yardstick")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the step replayed from a captured HIP graph")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the headline's oracle comparison (profiling runs)")
    ap.add_argument("--unfused-step", action="store_true",
                    help="time a step's slot write and decode as two launches instead of "
                         "paged_decode_step")
    args = ap.parse_args()
    global UNFUSED_STEP
    UNFUSED_STEP = bool(args.unfused_step)

    if args.gpus != 1:
        print(f"bench.py measures the decode path on one GPU; --gpus {args.gpus} is not "
              "supported (there is no multi-GPU path in this library).", file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process on one GPU.", file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.mode == "copy":
        run_copy(args.copy_mb, args.steps)
        return 0

    import paged_kv_decode_13_amd as pkv
    from paged_kv_decode_13_amd import workloads as wl

    from paged_kv_decode_13_amd import build as pkv_build

    if not (os.path.exists(pkv.library_path()) and os.path.exists(pkv_build.STREAM_LIB_PATH)):
        pkv_build.build()
    headline = (args.mode == "decode" and args.config == "gqa_bf16" and args.block_size is None
                and not args.shared_prefix)
    suite_arg = args.configs if args.configs is not None else ("all" if headline else "none")
    suite = [] if suite_arg == "none" else list(SUITE) if suite_arg == "all" else \
        [s for s in suite_arg.split(",") if s]
    for s in suite:
        if s not in SUITE:
            print(f"unknown workload {s!r}; choose from {', '.join(SUITE)}", file=sys.stderr)
            return 2
    dev = torch.device("cuda:0")
    t0 = time.time()
    if args.config in wl.PREFILL_NAMES:
        batch = wl.make_prefill_config(args.config)
    else:
        batch = wl.make_config(args.config, block_size=args.block_size)
    log(f"[bench] {args.config}: {batch.num_seqs} seqs, {batch.total_tokens} context tokens, "
        f"generated in {time.time() - t0:.1f}s")
    t = upload(batch, dev)
    torch.cuda.synchronize()
    shared = bool(args.shared_prefix)
    ps = batch.partition_size if args.partition_size is None else args.partition_size
    if shared and args.partition_size is None:
        # the suffixes (0..1024 tokens) are cut finer than the whole histories:
        # measured best on the shared-prefix path
        ps = SHARED_PREFIX_PARTITION
    if shared and "prefix_table" not in batch.meta:
        print(f"{args.config} has no shared prefix", file=sys.stderr)
        return 2
    if args.mode == "prefill":
        if args.config not in wl.PREFILL_NAMES:
            print("--mode prefill runs on a prompt workload (prefill_bf16)", file=sys.stderr)
            return 2
        wl.add_prompt_queries(batch, seed=11)
        t = upload(batch, dev)
        print(json.dumps(run_prefill(batch, t, args.steps, args.warmup)), flush=True)
        return 0
    if args.mode == "write":
        if batch.slot_mapping is None:
            print(f"{args.config} writes no tokens", file=sys.stderr)
            return 2
        print(json.dumps(run_write(batch, t, args.steps, args.warmup)), flush=True)
        return 0

    if args.sweep_partitions:
        for p in [int(x) for x in args.sweep_partitions.split(",")]:
            r = time_steps(batch, t, p, max(5, args.steps // 2), 3, shared)
            gbs = batch.kv_bytes_logical() / (r["decode_ms"] * 1e-3) / 1e9
            log(f"[sweep] partition {p:6d}: decode {r['decode_ms']*1e3:8.1f} us "
                f"({gbs:7.1f} GB/s, {100 * gbs / HBM_PEAK_GBS:5.1f}% of peak), "
                f"write {r['write_ms']*1e3:6.1f} us")

    r = time_steps(batch, t, ps, args.steps, args.warmup, shared, cold_steps=args.cold_steps,
                   graph=not args.no_graph)
    log(f"[bench] timed {args.steps} steps: {r['ms_per_step']:.4f} ms/step "
        f"(decode {r['decode_ms']:.4f} ms, write {r['write_ms']:.4f} ms)")

    kv_bytes = batch.kv_bytes_logical()
    step_s = r["ms_per_step"] * 1e-3
    value = kv_bytes / step_s / 1e9
    # the roofline rates algorithmic HBM bytes: with the shared prefix read
    # once, that is the distinct cached rows, not the logical history
    alg_bytes = batch.kv_bytes_unique() if shared else kv_bytes
    achieved = alg_bytes / (r["decode_ms"] * 1e-3) / 1e9
    workload = args.config if args.block_size is None else f"{args.config}_bs{args.block_size}"
    traffic = load_traffic(workload + ("_shared" if shared else ""))
    if shared:
        kernel = ("paged_prefix_decode_attention call (prefix units and suffix decode in one "
                  "kernel + log-sum-exp merge)")
    elif fused_step(batch, t):
        kernel = "paged_decode_step call (decode kernel with the slot write" + (
            " + log-sum-exp merge)" if ps and batch.max_context_len > ps else ")")
    else:
        kernel = "paged_decode_attention call (decode kernel" + (
            " + log-sum-exp merge)" if ps and batch.max_context_len > ps else ")")

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": batch.dtype,
        "data": "synthetic (seeded N(0,1) values, generated context lengths and page tables)",
        "config": {
            "workload": batch.name,
            "num_seqs": batch.num_seqs,
            "num_heads": batch.num_heads,
            "num_kv_heads": batch.num_kv_heads,
            "head_dim": batch.head_dim,
            "block_size": batch.block_size,
            "partition_size": ps,
            "context_tokens": batch.total_tokens,
            "max_context_len": batch.max_context_len,
            "new_tokens_written": 0 if batch.slot_mapping is None else int((batch.slot_mapping >= 0).sum()),
            "kv_cache_dtype": batch.cache_dtype,
            "parallelism": "single GPU",
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "decode_tokens_per_s": round(batch.num_seqs / step_s, 1),
        "kv_bytes_logical": kv_bytes,
        "step_entry_point": step_entry(batch, t, shared),
        "write_ms": round(r["write_ms"], 5),
        "decode_ms": round(r["decode_ms"], 5),
        "decode_ms_median": round(r["decode_ms_median"], 5),
        "decode_ms_p99": round(r["decode_ms_p99"], 5),
        "step_ms_p99": round(r["step_ms_p99"], 5),
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "algorithmic_bytes": alg_bytes,
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
    }
    if "graph_ms_per_step" in r:
        line["graph"] = {
            "ms_per_step": round(r["graph_ms_per_step"], 5),
            "step_ms_median": round(r["graph_step_ms_median"], 5),
            "step_ms_p99": round(r["graph_step_ms_p99"], 5),
            "gpu_ms_per_step": round(r["graph_gpu_ms_per_step"], 5),
            "value": round(kv_bytes / (r["graph_ms_per_step"] * 1e-3) / 1e9, 2),
            "decode_tokens_per_s": round(batch.num_seqs / (r["graph_ms_per_step"] * 1e-3), 1),
        }
    if "cold" in r:
        c = dict(r["cold"])
        c["decode_gbs_median"] = round(alg_bytes / (c["decode_ms_median"] * 1e-3) / 1e9, 2)
        c["value_median"] = round(kv_bytes / (c["step_ms_median"] * 1e-3) / 1e9, 2)
        line["cold"] = {k: (round(v, 5) if isinstance(v, float) else v) for k, v in c.items()}
    if not args.no_stream_read:
        sr = stream_read(dev)
        sr["decode_frac_of_stream"] = round(achieved / sr["gbs"], 4)
        line["stream_read"] = sr
        log(f"[bench] stream read {sr['gbs']:.1f} GB/s; decode call at "
            f"{100 * sr['decode_frac_of_stream']:.1f}% of it")
    if args.block_size is not None or shared:
        line["config"]["unique_kv_bytes"] = batch.kv_bytes_unique()
    if shared:
        line["config"]["shared_prefix_tokens"] = batch.meta["shared_prefix_tokens"]
        line["config"]["entry_point"] = "paged_prefix_decode_attention"

    ok = True
    if not args.no_parity:
        # the outputs of the timed run against the oracle's, every element
        host_write(batch)
        ref = oracle_decode(batch, 0, shared)
        line["parity"] = parity(r["out"], ref, batch.dtype,
                                f"all {ref.size} outputs of the timed run")
        ok = line["parity"]["ok"]
        log(f"[bench] parity: max|gpu-oracle| = {line['parity']['max_abs_err']:.3e} "
            f"({'ok' if ok else 'FAIL'})")
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle ...")
        line["cpu_baseline"] = cpu_baseline(batch, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    del t, r
    _free()
    if suite:
        line["configs"] = run_suite(suite, dev, args.steps, args.warmup)
        bad = [k for k, v in line["configs"].items() if not v["parity"]["ok"]]
        if bad:
            log(f"[bench] parity FAILED: {', '.join(bad)}")
            ok = False
    print(json.dumps(line), flush=True)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
