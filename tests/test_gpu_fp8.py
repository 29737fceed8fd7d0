"""8-bit (E4M3) KV cache: the quantising slot write and the decode over E4M3
pools against the oracle's E4M3 functions on identical inputs (MI355X)."""
import itertools

import numpy as np
import pytest

import oracle
from paged_kv_decode_13_amd import workloads as wl
from tests.gpu_helpers import (TIGHT, TOL, gpu_step, max_err, oracle_step, rounded_out_ok, to_f64,
                               upload)

pytestmark = pytest.mark.gpu


def _special_values(scale: np.float32) -> np.ndarray:
    """binary32 inputs whose scaled values hit the E4M3 grid points, the
    midpoints between them (ties), one ulp either side of the midpoints,
    the subnormal range, saturation and signed zeros."""
    table = oracle.e4m3_to_float64(np.arange(0, 0x7F, dtype=np.uint8))
    pos = np.unique(table)
    mids = (pos[1:] + pos[:-1]) / 2
    t = np.concatenate([pos, mids, [448.5, 464, 479.9, 480, 1e5], pos / 3]).astype(np.float32)
    t = np.concatenate([t, np.nextafter(t, np.float32(np.inf)), np.nextafter(t, np.float32(0))])
    # inputs x with x * fl(1/scale) near those points
    inv = np.float32(1) / scale
    x = (t / inv).astype(np.float32)
    x = np.concatenate([x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(0))])
    return np.concatenate([x, -x, np.array([0.0, -0.0], np.float32)])


@pytest.mark.parametrize("src", ["f32", "f16", "bf16"])
def test_fp8_write_is_bit_exact(cuda, src):
    import torch

    import paged_kv_decode_13_amd as pkv

    kvh, d, bs = 4, 128, 16
    ks = np.array([0.02, 1.0, 3.0, 0.0071], np.float32)
    vs = np.array([7.5, 0.011, 0.5, 2.0], np.float32)
    rng = np.random.default_rng(5)
    vals = np.concatenate([_special_values(ks[0]), _special_values(ks[2]),
                           (rng.standard_normal(60000) * rng.choice([0.01, 1, 30], 60000)).astype(np.float32)])
    n_tok = -(-vals.size // (kvh * d))
    flat = np.resize(vals, n_tok * kvh * d).astype(np.float32)
    enc = wl.encode(flat, src).reshape(n_tok, kvh, d)
    key, value = enc, np.ascontiguousarray(enc[::-1])
    nb = n_tok // bs + 3
    slots = rng.permutation(nb * bs)[:n_tok].astype(np.int64)
    slots[3] = -1
    kc = np.full((nb, bs, kvh, d), 0x55, np.uint8)
    vc = kc.copy()
    print(f"\n[fp8 write] {src}: {n_tok} tokens", flush=True)
    dev = cuda
    tk, tv = wl.torch_view(key, src).to(dev), wl.torch_view(value, src).to(dev)
    tkc, tvc = torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev)
    pkv.paged_kv_write_fp8(tk, tv, tkc, tvc, torch.from_numpy(slots).to(dev),
                           torch.from_numpy(ks).to(dev), torch.from_numpy(vs).to(dev))
    torch.cuda.synchronize()
    oracle.paged_kv_write_e4m3(key, value, kc, vc, slots, ks, vs, src)
    assert np.array_equal(tkc.cpu().numpy(), kc)
    assert np.array_equal(tvc.cpu().numpy(), vc)


def _edge_lengths(bs):
    return [1, bs - 1, bs, bs + 1, 3 * bs + 1, 0, 137, 700]


EDGE = [(dt, bs, g) for dt, bs, g in itertools.product(("f16", "bf16"), (4, 8, 16, 32, 64),
                                                       (1, 2, 4, 8))]


@pytest.mark.parametrize("dtype,bs,group", EDGE, ids=[f"{a}-bs{b}-g{c}" for a, b, c in EDGE])
def test_fp8_edge_lengths(cuda, dtype, bs, group):
    """Quantised write of each sequence's new token, then decode over the E4M3
    pools, unsplit and split; fp32 outputs to the arithmetic bound, 16-bit
    outputs to it plus their own rounding."""
    b = wl.make_batch(_edge_lengths(bs), num_heads=2 * group, num_kv_heads=2, head_dim=128,
                      block_size=bs, dtype=dtype, seed=2000 + bs * 7 + group, write_new_token=True,
                      table_slack=1, kv_dtype="e4m3")
    ref = oracle_step(b)
    assert np.array_equal(ref[5], np.zeros_like(ref[5]))
    for ps in (0, max(64, bs)):
        out = to_f64(gpu_step(b, upload(b, cuda), partition_size=ps, out_dtype="f32"))
        assert max_err(out, ref) <= TIGHT[dtype], (ps, max_err(out, ref))
        out = to_f64(gpu_step(b, upload(b, cuda), partition_size=ps))
        assert rounded_out_ok(out, ref, dtype), (ps, max_err(out, ref))


def test_fp8_out_of_range_contents(cuda):
    """A bad page id or context length gives that sequence NaN, not a fault;
    the other sequences are unchanged."""
    b = wl.make_batch([40, 300, 17, 129], num_heads=8, num_kv_heads=2, head_dim=128,
                      block_size=16, dtype="bf16", seed=77, kv_dtype="e4m3")
    ref = oracle_step(b)
    t = upload(b, cuda)
    bt = t["bt"].clone()
    bt[1, 3] = b.num_blocks + 9
    t["bt"] = bt
    cl = t["cl"].clone()
    cl[2] = b.max_context_len + 5
    t["cl"] = cl
    out = to_f64(gpu_step(b, t, out_dtype="f32", partition_size=64))
    assert np.isnan(out[1]).all() and np.isnan(out[2]).all()
    assert max_err(out[[0, 3]], ref[[0, 3]]) <= TIGHT["bf16"]


def test_fp8_deterministic_and_split_agree(cuda):
    b = wl.make_batch([3000, 15, 777, 2048], num_heads=32, num_kv_heads=8, head_dim=128,
                      block_size=32, dtype="f16", seed=91, kv_dtype="e4m3")
    t = upload(b, cuda)
    a1 = gpu_step(b, t, partition_size=0).cpu()
    a2 = gpu_step(b, t, partition_size=0).cpu()
    import torch

    assert torch.equal(a1.view(torch.int16), a2.view(torch.int16))
    ref = oracle_step(b)
    for ps in (256, 1024, 4096):
        out = to_f64(gpu_step(b, t, partition_size=ps, out_dtype="f32"))
        assert max_err(out, ref) <= TIGHT["f16"], ps


def test_fp8_full_config(cuda):
    """The GQA batch-256 workload over an E4M3 cache at full size: every output
    element against the oracle, in the launch configuration the benchmark
    times and with fp32 outputs."""
    b = wl.make_config("gqa_fp8")
    print(f"\n[gqa_fp8] {b.total_tokens} context tokens", flush=True)
    ref = oracle_step(b)
    out = to_f64(gpu_step(b, upload(b, cuda)))
    assert max_err(out, ref) <= TOL["bf16"], max_err(out, ref)
    out = to_f64(gpu_step(b, upload(b, cuda), out_dtype="f32"))
    assert max_err(out, ref) <= TIGHT["bf16"], max_err(out, ref)
