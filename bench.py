#!/usr/bin/env python3
"""Decode-step benchmark for paged-KV decode attention on one MI355X.

A step is one pass of the whole hot path over one decode batch: the slot
write of each sequence's new K/V (paged_kv_write) followed by the fused paged
decode attention (paged_decode_attention, plus its log-sum-exp merge when the
context is split).  Inputs are seeded synthetic batches (see
paged_kv_decode_13_amd/workloads.py) uploaded to HBM before the timed region.

Prints ONE JSON line on stdout.  ``value`` is the effective KV-read bandwidth
of the whole step: sum(ctx) * num_kv_heads * head_dim * 2 * bytes / step time.
``roofline`` rates the decode call alone (HIP events on the launch stream)
against the 8 TB/s HBM peak.  ``graph`` times the same step replayed from
a captured HIP graph (no host launch gaps).  ``cold`` repeats the step with L2 and the MALL
flushed before each one (a 1 GiB read-modify-write outside the events);
``stream_read`` times a plain contiguous read (libpkvstream.so) as the
achievable-read yardstick.  ``cpu_baseline`` is the fp64 oracle timed on a
bounded sample of the same batch on the host cores.

Usage: python bench.py [--steps K] [--warmup W] [--config gqa_bf16]
       python bench.py --mode copy  (plain device copy, for counter scaling)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

REPO = os.path.dirname(os.path.abspath(__file__))
if REPO not in sys.path:
    sys.path.insert(0, REPO)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published
METRIC = "effective KV-read HBM GB/s (% of MI355X peak) + decode tokens/s, paged attention"
SHARED_PREFIX_PARTITION = 512
COLD_FLUSH_BYTES = 1 << 30   # > L2 (4 MiB per XCD) + MALL (256 MiB)
STREAM_READ_BYTES = 2 << 30  # contiguous buffer of the streaming-read yardstick


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
    """HBM bytes per decode launch measured by rocprofv3 counters, if they were
    taken on the current kernel sources (else None)."""
    path = os.path.join(REPO, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest():
        return None
    return rec.get("bytes_per_launch")


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


def time_steps(batch, t, partition_size: int, steps: int, warmup: int, shared_prefix: bool = False,
               cold_steps: int = 0, graph: bool = False):
    import torch

    import paged_kv_decode_13_amd as pkv

    out = torch.empty((batch.num_seqs, batch.num_heads, batch.head_dim), dtype=t["q"].dtype,
                      device=t["q"].device)
    if shared_prefix:
        plen = batch.meta["shared_prefix_tokens"]
        ptab = torch.from_numpy(batch.meta["prefix_table"]).to(t["q"].device)
        need = pkv.paged_prefix_decode_workspace_size(
            batch.num_seqs, batch.num_heads, batch.num_kv_heads, batch.head_dim,
            batch.max_context_len, plen, partition_size)
    else:
        need = pkv.paged_decode_workspace_size(batch.num_seqs, batch.num_heads, batch.head_dim,
                                               batch.max_context_len, partition_size)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device=t["q"].device)  # counter starts at zero
    has_write = "slots" in t
    quant = batch.cache_dtype == "e4m3"

    def write():
        if has_write and quant:
            pkv.paged_kv_write_fp8(t["nk"], t["nv"], t["kc"], t["vc"], t["slots"], t["ks"], t["vs"])
        elif has_write:
            pkv.paged_kv_write(t["nk"], t["nv"], t["kc"], t["vc"], t["slots"])

    def decode():
        if quant:
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

    for _ in range(warmup):
        write()
        decode()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for e in evs:
        e[0].record()
        write()
        e[1].record()
        decode()
        e[2].record()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = [e[0].elapsed_time(e[2]) for e in evs]
    write_ms = [e[0].elapsed_time(e[1]) for e in evs]
    decode_ms = [e[1].elapsed_time(e[2]) for e in evs]
    res = {
        "ms_per_step": start.elapsed_time(end) / steps,
        "wall_ms_per_step": 1e3 * wall / steps,
        "write_ms": statistics.mean(write_ms),
        "decode_ms": statistics.mean(decode_ms),
        "decode_ms_median": statistics.median(decode_ms),
        "step_ms_p99": _pct(step_ms, 0.99),
        "out": out,
    }
    if graph:
        # the same step captured once in a HIP graph and replayed: no host
        # launch gaps between the write, the decode and the merge
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            write()
            decode()
        for _ in range(max(1, warmup)):
            g.replay()
        torch.cuda.synchronize()
        gs, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gs.record()
        for _ in range(steps):
            g.replay()
        ge.record()
        torch.cuda.synchronize()
        res["graph_ms_per_step"] = gs.elapsed_time(ge) / steps
        del g
    if cold_steps > 0:
        # cold caches: a 1 GiB read-modify-write before each step evicts L2
        # and the MALL (tables, workspace, query, recently read pages); it
        # sits outside the events, on the same stream
        scratch = torch.zeros(COLD_FLUSH_BYTES // 4, dtype=torch.int32, device=t["q"].device)
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
    sequences, repeated until about ``target_s`` seconds of host work."""
    import numpy as np

    import oracle
    from paged_kv_decode_13_amd import workloads as wl

    order = np.arange(batch.num_seqs)
    probe = wl.subset(batch, order[:: max(1, batch.num_seqs // 8)])
    def run(b):
        if b.cache_dtype == "e4m3":
            oracle.paged_decode_e4m3(b.query, b.key_cache, b.value_cache, b.k_scale, b.v_scale,
                                     b.block_tables, b.context_lens, b.block_size, b.scale, b.dtype)
        else:
            oracle.paged_decode(b.query, b.key_cache, b.value_cache, b.block_tables,
                                b.context_lens, b.block_size, b.scale, b.dtype)

    t0 = time.perf_counter()
    run(probe)
    probe_s = max(time.perf_counter() - t0, 1e-3)
    frac = min(1.0, target_s / probe_s * probe.total_tokens / batch.total_tokens)
    step = max(1, int(round(1.0 / frac))) if frac < 1.0 else 1
    sample = wl.subset(batch, order[::step])
    passes, secs = 0, 0.0
    while passes == 0 or (secs < target_s and passes < 100):
        t0 = time.perf_counter()
        run(sample)
        secs += time.perf_counter() - t0
        passes += 1
    per_pass = secs / passes
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu_model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(sample.kv_bytes_logical() / per_pass / 1e9, 4),
        "unit": "GB/s",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": ((f"every {step}th sequence of the same batch" if step > 1 else
                    "the whole batch") +
                   f" ({sample.num_seqs} sequences, {sample.total_tokens} context tokens), "
                   f"fp64 gather + softmax attention, {passes} passes in {secs:.1f} s"),
        "tokens_per_s": round(sample.num_seqs / per_pass, 3),
        "cpu_model": cpu_model,
    }


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
                     "traffic": None},
        "cpu_baseline": None,
    }


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix peak, AMD published


def prefill_flops(batch) -> int:
    """Algorithmic flops of causal attention over the prompts: query i of a
    prompt sees i + 1 tokens; scores and values each take 2 * D flops per
    (query head, visible token)."""
    import numpy as np

    n = batch.context_lens.astype(np.int64)
    visible = int((n * (n + 1) // 2).sum())
    return 4 * batch.head_dim * batch.num_heads * visible


def run_prefill(batch, t, steps: int, warmup: int) -> dict:
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
    step_ms = statistics.mean(e[0].elapsed_time(e[2]) for e in evs)
    attn_ms = statistics.mean(e[1].elapsed_time(e[2]) for e in evs)
    write_ms = statistics.mean(e[0].elapsed_time(e[1]) for e in evs)
    flops = prefill_flops(batch)
    tflops = flops / (attn_ms * 1e-3) / 1e12
    tokens = int(batch.context_lens.astype("int64").sum())
    return {
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
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None},
        "cpu_baseline": None,
    }


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
    args = ap.parse_args()

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
        "write_ms": round(r["write_ms"], 5),
        "decode_ms": round(r["decode_ms"], 5),
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

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a sample ...")
        line["cpu_baseline"] = cpu_baseline(batch, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
