"""The oracle against what the pages and the mathematics fix (CPU only)."""
import os
import shutil
import subprocess
import sys
import tempfile

import numpy as np
import pytest

from tests import oracle_pins as pins

import oracle


@pytest.mark.parametrize("pin", pins.QUICK_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# Plausible mistakes planted in a copy of oracle.c; each must trip at least one
# pin.  (old text, new text) replacements, applied to the copy only.
PLANTED = {
    "block_id_uses_modulo": ("int64_t lb = token_index / block_size;",
                             "int64_t lb = token_index % block_size;"),
    "offset_uses_division": ("int64_t off = token_index % block_size;",
                             "int64_t off = (token_index / block_size) % block_size;"),
    "scale_dropped": ("scores[t] = scale * dot;", "scores[t] = dot;"),
    "gqa_heads_interleaved": ("int32_t h = kvh * group + g;", "int32_t h = g * num_kv_heads + kvh;"),
    "keys_summed_not_values": ("out[d] += w * values[t * head_dim + d];",
                               "out[d] += w * keys[t * head_dim + d];"),
    "softmax_not_normalised": ("double w = scores[t] / denom;", "double w = scores[t];"),
    "dot_index_wrong": ("dot += q[d] * keys[t * head_dim + d];", "dot += q[d] * keys[d];"),
    "pool_axes_swapped": ("((pb * block_size + off) * num_kv_heads + kv_head)",
                          "((off * num_blocks + pb) % (num_blocks * block_size) * num_kv_heads + kv_head)"),
    "f16_bias_off_by_one": ("mag = ldexp(1.0 + (double)frac / 1024.0, expo - 15);",
                            "mag = ldexp(1.0 + (double)frac / 1024.0, expo - 16);"),
    "write_offset_dropped": ("int64_t off = slot % block_size;", "int64_t off = 0;"),
    "max_not_subtracted_sign": ("scores[t] = exp(scores[t] - smax);", "scores[t] = exp(smax - scores[t]);"),
    "prefix_table_ignored": ("row[lb] = lb < prefix_blocks ? prefix_table[lb] : own[lb];",
                             "row[lb] = own[lb];"),
    "prefix_last_page_from_own_row": ("row[lb] = lb < prefix_blocks ? prefix_table[lb] : own[lb];",
                                      "row[lb] = lb < prefix_blocks - 1 ? prefix_table[lb] : own[lb];"),
    "prefix_pages_reversed": ("row[lb] = lb < prefix_blocks ? prefix_table[lb] : own[lb];",
                              "row[lb] = lb < prefix_blocks ? prefix_table[prefix_blocks - 1 - lb] : own[lb];"),
    "suffix_table_relative": ("row[lb] = lb < prefix_blocks ? prefix_table[lb] : own[lb];",
                              "row[lb] = lb < prefix_blocks ? prefix_table[lb] : own[lb - prefix_blocks];"),
    "prefill_query_cannot_see_itself": ("rc = oracle_attention(out + qrow, qd, keys, values, pos + 1,",
                                        "rc = oracle_attention(out + qrow, qd, keys, values, pos,"),
    "prefill_top_left_causal": ("int32_t pos = ctx - q_len + i; /* this query's position */",
                                "int32_t pos = i; /* this query's position */"),
    "prefill_sees_the_future": ("rc = oracle_attention(out + qrow, qd, keys, values, pos + 1,",
                                "rc = oracle_attention(out + qrow, qd, keys, values, ctx,"),
    "prefill_query_offset_dropped": ("int64_t qrow = ((int64_t)(q0 + i) * num_heads + head) * head_dim;",
                                     "int64_t qrow = ((int64_t)i * num_heads + head) * head_dim;"),
    "prefill_gqa_heads_interleaved": ("int32_t head = kvh * group + g;", "int32_t head = g * num_kv_heads + kvh;"),
    "e4m3_bias_off_by_one": ("mag = ldexp(1.0 + (double)frac / 8.0, expo - 7);",
                             "mag = ldexp(1.0 + (double)frac / 8.0, expo - 8);"),
    "e4m3_subnormal_as_normal": ("mag = ldexp((double)frac, -9); /* subnormal",
                                 "mag = ldexp(1.0 + (double)frac / 8.0, -7); /* subnormal"),
    "e4m3_no_saturation": ("if (a > 448.0) a = 448.0;", "if (a > 1e30) a = 448.0;"),
    "e4m3_ties_away": ("double m = rint(ldexp(a, -e) * 8.0) - 8.0;",
                       "double m = floor(ldexp(a, -e) * 8.0 + 0.5) - 8.0;"),
    "e4m3_write_divides": ("float kx = load_f32(key, i * token_elems + e, src_dtype) * kinv;",
                           "float kx = load_f32(key, i * token_elems + e, src_dtype) / k_scale[h];"),
    "e4m3_gqa_heads_interleaved": ("int32_t qh = kvh * group + g;", "int32_t qh = g * num_kv_heads + kvh;"),
    "e4m3_write_offset_dropped": ("int64_t offset = slot % block_size;", "int64_t offset = 0;"),
    "e4m3_value_scale_on_keys": ("keys[t * head_dim + d] = oracle_decode_e4m3(key_cache[row + d]) * (double)k_scale[kvh];",
                                 "keys[t * head_dim + d] = oracle_decode_e4m3(key_cache[row + d]) * (double)v_scale[kvh];"),
}


@pytest.fixture(scope="module")
def planted_dir():
    d = tempfile.mkdtemp(prefix="oracle_planted_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(PLANTED))
def test_planted_mistake_is_caught(name, planted_dir):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "oracle.c"), encoding="utf-8").read()
    old, new = PLANTED[name]
    assert src.count(old) == 1, f"mutation anchor not found once: {old}"
    mdir = os.path.join(planted_dir, name)
    os.makedirs(mdir, exist_ok=True)
    shutil.copy(os.path.join(os.path.dirname(oracle.__file__), "oracle.h"), mdir)
    with open(os.path.join(mdir, "oracle.c"), "w", encoding="utf-8") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(mdir, "liboracle.so")
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", lib,
                    os.path.join(mdir, "oracle.c"), "-lm"], check=True)
    repo = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, "-m", "tests.oracle_pins", "--lib", lib], cwd=repo,
                         capture_output=True, text=True, timeout=300)
    assert res.returncode != 0, f"planted mistake {name} passed every pin:\n{res.stdout}"


def test_unmodified_copy_passes(planted_dir):
    """Control for the planted-mistake runs: the same harness on an
    unmodified copy reports no failure."""
    mdir = os.path.join(planted_dir, "_control")
    os.makedirs(mdir, exist_ok=True)
    here = os.path.dirname(oracle.__file__)
    for f in ("oracle.c", "oracle.h"):
        shutil.copy(os.path.join(here, f), mdir)
    lib = os.path.join(mdir, "liboracle.so")
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", lib,
                    os.path.join(mdir, "oracle.c"), "-lm"], check=True)
    repo = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, "-m", "tests.oracle_pins", "--lib", lib], cwd=repo,
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr


def test_prefix_workload_independent_of_block_size():
    """The shared-prefix workload lays identical logical data out in pages of
    8, 16, 32 and 64 tokens; the paged result must not depend on the layout
    (a sample of sequences keeps this quick)."""
    from paged_kv_decode_13_amd import workloads as wl

    outs = []
    for bs in wl.PREFIX_BLOCK_SIZES:
        b = wl.subset(wl.make_config("prefix_fp16", block_size=bs), [0, 5, 77])
        outs.append(oracle.paged_decode(b.query, b.key_cache, b.value_cache, b.block_tables,
                                        b.context_lens, bs, b.scale, "f16"))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
