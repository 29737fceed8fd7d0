"""Host-side pieces of bench.py that need no GPU."""
import os
import subprocess
import sys

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, REPO)

import bench  # noqa: E402


def test_code_text_drops_comments_only():
    src = 'int a = 1; // note\n/* block\n comment */ const char *s = "// kept"; char c = \'/\';'
    assert bench.code_text(src) == 'int a = 1; const char *s = "// kept"; char c = \'/\';'


def test_digest_ignores_comments_not_code():
    base = {"k.hip": "__global__ void k(int *p) {\n  p[0] = 1;  // store\n}\n"}
    commented = {"k.hip": "// a kernel\n__global__ void k(int *p) {\n  /* one */ p[0] = 1;\n}\n"}
    changed = {"k.hip": "__global__ void k(int *p) {\n  p[0] = 2;\n}\n"}
    assert bench.source_digest(base) == bench.source_digest(commented)
    assert bench.source_digest(base) != bench.source_digest(changed)
    assert bench.source_digest(base) != bench.source_digest({"other.hip": base["k.hip"]})


def test_multi_gpu_request_is_refused():
    res = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_parity_flags_errors_and_nan():
    import numpy as np
    import torch

    ref = np.zeros((2, 3), dtype=np.float64)
    ok = bench.parity(torch.full((2, 3), 4e-3), ref, "bf16", "six")
    assert ok["ok"] and abs(ok["max_abs_err"] - 4e-3) < 1e-9
    assert not bench.parity(torch.full((2, 3), 6e-3), ref, "bf16", "six")["ok"]
    assert not bench.parity(torch.full((2, 3), 2e-5), ref, "f32", "six")["ok"]
    nan = torch.zeros(2, 3)
    nan[1, 2] = float("nan")
    assert not bench.parity(nan, ref, "f16", "six")["ok"]


def test_cpu_model_is_reported():
    name = bench.cpu_model()
    assert name is None or (isinstance(name, str) and name)
