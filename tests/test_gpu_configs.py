"""The five named decode workloads at full size: HIP path against the fp64
oracle over every output element, in the launch configuration the benchmark
times (cache dtype out, the workload's KV partition size), and with fp32
outputs against the tighter arithmetic bound."""
import time

import numpy as np
import pytest

from paged_kv_decode_13_amd import workloads as wl
from tests.gpu_helpers import TIGHT, TOL, gpu_step, max_err, oracle_step, to_f64, upload

pytestmark = pytest.mark.gpu

CASES = [("tiny_fp32", None), ("mha_fp16", None), ("gqa_bf16", None), ("long_bf16", None)] + [
    ("prefix_fp16", bs) for bs in wl.PREFIX_BLOCK_SIZES]


@pytest.mark.parametrize("name,bs", CASES, ids=[f"{n}" + (f"-bs{b}" if b else "") for n, b in CASES])
def test_full_config(cuda, name, bs):
    t0 = time.time()
    b = wl.make_config(name, block_size=bs)
    print(f"\n[{name}] generated in {time.time() - t0:.1f}s; tokens={b.total_tokens}", flush=True)
    t0 = time.time()
    ref = oracle_step(b)
    print(f"[{name}] oracle in {time.time() - t0:.1f}s", flush=True)
    out = to_f64(gpu_step(b, upload(b, cuda)))
    err = max_err(out, ref)
    print(f"[{name}] bench launch (partition {b.partition_size}, {b.dtype} out): "
          f"max|err|={err:.3e} bar {TOL[b.dtype]}", flush=True)
    assert err <= TOL[b.dtype]
    out = to_f64(gpu_step(b, upload(b, cuda), out_dtype="f32"))
    err = max_err(out, ref)
    print(f"[{name}] fp32 out: max|err|={err:.3e} bound {TIGHT[b.dtype]}", flush=True)
    assert err <= TIGHT[b.dtype]
    out = to_f64(gpu_step(b, upload(b, cuda), partition_size=0, out_dtype="f32"))
    assert max_err(out, ref) <= TIGHT[b.dtype]
