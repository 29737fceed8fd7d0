"""The fused decode step (paged_decode_step: the slot write inside the decode
launch) against the oracle's write-then-decode, through the C ABI (MI355X)."""
import itertools

import numpy as np
import pytest

import oracle
from paged_kv_decode_13_amd import workloads as wl
from tests.gpu_helpers import TIGHT, max_err, oracle_step, to_f64, upload

pytestmark = pytest.mark.gpu


def _step(b, t, *, partition_size, out_dtype="f32", workspace=None):
    import torch

    import paged_kv_decode_13_amd as pkv

    odt = getattr(torch, {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}[out_dtype])
    out = pkv.paged_decode_step(t["q"], t["kc"], t["vc"], t["nk"], t["nv"], t["slots"], t["bt"],
                                t["cl"], b.block_size, b.scale, max_context_len=b.max_context_len,
                                partition_size=partition_size, out_dtype=odt, workspace=workspace)
    torch.cuda.synchronize()
    return out


def _bits(pool) -> np.ndarray:
    import torch

    return pool.cpu().view(torch.int16).numpy().reshape(-1).view(np.uint16)


def _oracle_pools(b, slots=None):
    kc, vc = b.key_cache.copy(), b.value_cache.copy()
    oracle.paged_kv_write(b.new_key, b.new_value, kc, vc, b.slot_mapping if slots is None else slots)
    return kc, vc


CASES = [(dt, bs, g) for dt, bs, g in itertools.product(("f16", "bf16"), (4, 16, 64), (1, 4, 8))]


@pytest.mark.parametrize("dtype,bs,group", CASES, ids=[f"{a}-bs{b}-g{c}" for a, b, c in CASES])
def test_step_matches_write_then_decode(cuda, dtype, bs, group):
    """Boundary lengths (the new token first, last and inside a page, an
    empty context with no slot, several pages) through the unsplit grid
    without a workspace, the persistent grid, single partitions and runs of
    four: outputs against the oracle's write-then-decode at the fp32-path
    bound, the pools byte for byte against the oracle's write (the new rows
    start out NaN in the pool, so a read of the pool instead of the new rows
    shows)."""
    import paged_kv_decode_13_amd as pkv

    lens = [1, bs - 1, bs, bs + 1, 3 * bs + 1, 0, 137, 700, 2100]
    b = wl.make_batch(lens, num_heads=2 * group, num_kv_heads=2, head_dim=128, block_size=bs,
                      dtype=dtype, seed=4000 + bs * 3 + group, write_new_token=True)
    print(f"\n[step] {dtype} bs={bs} G={group}", flush=True)
    ref = oracle_step(b)
    kc_ref, vc_ref = _oracle_pools(b)
    for ps, ws in ((0, pkv.NO_WORKSPACE), (0, None), (64 if bs <= 64 else bs, None), (512, None)):
        t = upload(b, cuda)
        out = to_f64(_step(b, t, partition_size=ps, workspace=ws))
        assert max_err(out, ref) <= TIGHT[dtype], (ps, ws)
        assert np.array_equal(_bits(t["kc"]), kc_ref.reshape(-1).view(np.uint16)), ps
        assert np.array_equal(_bits(t["vc"]), vc_ref.reshape(-1).view(np.uint16)), ps


VALU_CASES = [("f32", 128, 16, 1), ("f32", 128, 4, 8), ("f32", 64, 64, 4), ("f16", 64, 16, 8),
              ("bf16", 64, 8, 2)]


@pytest.mark.parametrize("dtype,dim,bs,group", VALU_CASES,
                         ids=[f"{a}-d{b}-bs{c}-g{d}" for a, b, c, d in VALU_CASES])
def test_step_vector_kernel(cuda, dtype, dim, bs, group):
    """The step on the caches the vector-ALU kernel serves (binary32, or
    head_dim 64): the same boundary lengths, the unsplit grid without a
    workspace and split partitions, outputs against the oracle's
    write-then-decode and the pools byte for byte."""
    import paged_kv_decode_13_amd as pkv

    lens = [1, bs - 1, bs, bs + 1, 3 * bs + 1, 0, 137, 700, 2100]
    b = wl.make_batch(lens, num_heads=2 * group, num_kv_heads=2, head_dim=dim, block_size=bs,
                      dtype=dtype, seed=4100 + dim + bs * 3 + group, write_new_token=True)
    print(f"\n[step] {dtype} d={dim} bs={bs} G={group}", flush=True)
    ref = oracle_step(b)
    kc_ref, vc_ref = _oracle_pools(b)
    for ps, ws in ((0, pkv.NO_WORKSPACE), (128 if bs <= 64 else bs, None), (512, None)):
        t = upload(b, cuda)
        out = to_f64(_step(b, t, partition_size=ps, workspace=ws))
        assert max_err(out, ref) <= TIGHT[dtype], (ps, ws)
        assert np.array_equal(_bits(t["kc"]), kc_ref.reshape(-1).view(np.uint16)), ps
        assert np.array_equal(_bits(t["vc"]), vc_ref.reshape(-1).view(np.uint16)), ps


def test_step_slot_rules(cuda):
    """A negative slot stores nothing and attends over the history as it
    is; a slot that is not the sequence's position ctx - 1 makes exactly
    that sequence NaN and is not written; an empty context with a slot
    stores nothing and gives zeros; 16-bit outputs."""
    import torch

    lens = [40, 300, 17, 1025, 0]
    b = wl.make_batch(lens, num_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                      dtype="bf16", seed=77, write_new_token=True)
    slots = b.slot_mapping.copy()
    # sequence 0 takes no new row: its position ctx - 1 keeps a finite row
    # (the batch leaves the new tokens' rows NaN until they are written)
    s0 = int(slots[0])
    b.key_cache[s0 // 16, s0 % 16] = b.new_value[0]
    b.value_cache[s0 // 16, s0 % 16] = b.new_key[0]
    slots[0] = -1
    slots[2] = int(slots[2]) - 1      # sequence 2 points one row early
    slots[4] = int(slots[1]) + 1      # an empty context given a slot
    t = upload(b, cuda)
    t["slots"] = torch.from_numpy(slots).to(cuda)
    out = to_f64(_step(b, t, partition_size=256))
    # reference: write the valid slots only (sequence 2's is refused), then decode
    ok = slots.copy()
    ok[2] = ok[4] = -1
    kc, vc = _oracle_pools(b, ok)
    ref = oracle.paged_decode(b.query, kc, vc, b.block_tables, b.context_lens, b.block_size,
                              b.scale, b.dtype)
    assert np.isnan(out[2]).all()
    assert (out[4] == 0).all()
    keep = [0, 1, 3, 4]
    assert max_err(out[keep], ref[keep]) <= TIGHT["bf16"]
    assert np.array_equal(_bits(t["kc"]), kc.reshape(-1).view(np.uint16))
    assert np.array_equal(_bits(t["vc"]), vc.reshape(-1).view(np.uint16))


def test_step_full_gqa_workload(cuda):
    """The 256-sequence GQA batch with its new tokens, every output element,
    at the partition size the bench times, and the pools after the step."""
    b = wl.make_config("gqa_bf16")
    print(f"\n[step] gqa_bf16 full: {b.num_seqs} seqs", flush=True)
    ref = oracle_step(b)
    t = upload(b, cuda)
    out = to_f64(_step(b, t, partition_size=b.partition_size))
    assert max_err(out, ref) <= TIGHT["bf16"]
    kc, vc = _oracle_pools(b)
    assert np.array_equal(_bits(t["kc"]), kc.reshape(-1).view(np.uint16))
    assert np.array_equal(_bits(t["vc"]), vc.reshape(-1).view(np.uint16))


def test_step_replays_in_graph(cuda):
    """paged_decode_step captured in a HIP graph and replayed after new
    queries and new rows were copied in: every replay bit for bit equal to
    an eager call on the same inputs, pools included."""
    import torch

    import paged_kv_decode_13_amd as pkv

    b = wl.make_batch([1, 15, 16, 17, 300, 1025, 4000, 2048], num_heads=32, num_kv_heads=8,
                      head_dim=128, block_size=16, dtype="bf16", seed=78, write_new_token=True)
    t = upload(b, cuda)
    out = torch.empty((b.num_seqs, b.num_heads, b.head_dim), dtype=torch.float32, device=cuda)
    need = pkv.paged_decode_workspace_size(b.num_seqs, b.num_heads, b.head_dim, b.max_context_len, 512)
    ws = torch.full((max(need, 1),), 255, dtype=torch.uint8, device=cuda)

    def step():
        pkv.paged_decode_step(t["q"], t["kc"], t["vc"], t["nk"], t["nv"], t["slots"], t["bt"], t["cl"],
                              b.block_size, b.scale, max_context_len=b.max_context_len,
                              partition_size=512, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for i in range(3):
        for key, shape in (("q", b.query.shape), ("nk", b.new_key.shape), ("nv", b.new_value.shape)):
            t[key].copy_(torch.from_numpy(
                wl.encode(rng.standard_normal(int(np.prod(shape))).astype(np.float32), "bf16")
                .reshape(shape)).view(torch.bfloat16).to(cuda))
        step()
        torch.cuda.synchronize()
        eager, kc_e, vc_e = out.clone(), t["kc"].clone(), t["vc"].clone()
        out.fill_(float("nan"))
        ws.fill_(250 + i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), i
        assert torch.equal(t["kc"].view(torch.int16), kc_e.view(torch.int16)), i
        assert torch.equal(t["vc"].view(torch.int16), vc_e.view(torch.int16)), i
