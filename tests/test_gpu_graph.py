"""The decode step (slot write + decode attention, split partitions and the
log-sum-exp merge included), and the shared-prefix call, captured in a HIP
graph and replayed (MI355X).

The library allocates nothing and clears nothing with memset (the
persistent decode kernel clears its own work counter when it starts), so a
captured step can be replayed as is.
Each replay is checked against an eager call on the same inputs, bit for
bit, with eager work (which also scribbles over the workspace) and
synchronisations between the replays, and the first against the oracle."""
import numpy as np
import pytest

import oracle
from paged_kv_decode_13_amd import workloads as wl
from tests.gpu_helpers import TIGHT, max_err, to_f64, upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv", [None, "e4m3"], ids=["bf16", "e4m3"])
def test_decode_step_replays_in_graph(cuda, kv):
    import torch

    import paged_kv_decode_13_amd as pkv

    batch = wl.make_batch([1, 15, 16, 17, 300, 1025, 4000, 2048], num_heads=32, num_kv_heads=8,
                          head_dim=128, block_size=16, dtype="bf16", seed=77, write_new_token=True,
                          partition_size=512, kv_dtype=kv)
    print(f"\n[graph] {kv or 'bf16'} cache: {batch.num_seqs} seqs", flush=True)
    dev = cuda
    t = upload(batch, dev)
    quant = kv == "e4m3"
    out = torch.empty((batch.num_seqs, batch.num_heads, batch.head_dim), dtype=torch.float32,
                      device=dev)
    need = pkv.paged_decode_workspace_size(batch.num_seqs, batch.num_heads, batch.head_dim,
                                           batch.max_context_len, batch.partition_size)
    ws = torch.full((max(need, 1),), 255, dtype=torch.uint8, device=dev)

    def step():
        if quant:
            pkv.paged_kv_write_fp8(t["nk"], t["nv"], t["kc"], t["vc"], t["slots"], t["ks"], t["vs"])
            pkv.paged_decode_attention_fp8(t["q"], t["kc"], t["vc"], t["ks"], t["vs"], t["bt"],
                                           t["cl"], batch.block_size, batch.scale,
                                           max_context_len=batch.max_context_len,
                                           partition_size=batch.partition_size, out=out,
                                           workspace=ws)
        else:
            pkv.paged_kv_write(t["nk"], t["nv"], t["kc"], t["vc"], t["slots"])
            pkv.paged_decode_attention(t["q"], t["kc"], t["vc"], t["bt"], t["cl"], batch.block_size,
                                       batch.scale, max_context_len=batch.max_context_len,
                                       partition_size=batch.partition_size, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    # eager result against the oracle
    kc, vc = batch.key_cache.copy(), batch.value_cache.copy()
    if quant:
        oracle.paged_kv_write_e4m3(batch.new_key, batch.new_value, kc, vc, batch.slot_mapping,
                                   batch.k_scale, batch.v_scale, batch.dtype)
        ref = oracle.paged_decode_e4m3(batch.query, kc, vc, batch.k_scale, batch.v_scale,
                                       batch.block_tables, batch.context_lens, batch.block_size,
                                       batch.scale, batch.dtype)
    else:
        oracle.paged_kv_write(batch.new_key, batch.new_value, kc, vc, batch.slot_mapping)
        ref = oracle.paged_decode(batch.query, kc, vc, batch.block_tables, batch.context_lens,
                                  batch.block_size, batch.scale, batch.dtype)
    assert max_err(to_f64(out), ref) <= TIGHT["bf16"]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    for i in range(4):
        # new queries (eager), then the eager step and the replay on them
        t["q"].copy_(torch.from_numpy(
            wl.encode(rng.standard_normal(batch.query.size).astype(np.float32), "bf16")
            .reshape(batch.query.shape)).view(torch.bfloat16).to(dev))
        step()
        torch.cuda.synchronize()
        eager = out.clone()
        out.fill_(float("nan"))
        ws.fill_(250 + i)  # a stale work counter and partials before the replay
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), i


def test_shared_prefix_call_replays_in_graph(cuda):
    """The shared-prefix call with two suffix partitions per sequence (prefix
    units and the suffix decode in one launch, then the merge) captured and
    replayed: every replay bit for bit equal to an eager call."""
    import torch

    import paged_kv_decode_13_amd as pkv

    prefix = 2048
    b = wl.make_prefix_batch([0, 1, prefix - 1, prefix, prefix + 1, prefix + 600, prefix + 952,
                              prefix + 52] * 4, prefix, num_heads=32, num_kv_heads=8,
                             head_dim=128, block_size=16, dtype="f16", seed=78,
                             partition_size=512)
    print(f"\n[graph] shared prefix: {b.num_seqs} seqs", flush=True)
    dev = cuda
    t = upload(b, dev)
    pt = torch.from_numpy(b.meta["prefix_table"]).to(dev)
    out = torch.empty((b.num_seqs, b.num_heads, b.head_dim), dtype=torch.float32, device=dev)
    need = pkv.paged_prefix_decode_workspace_size(b.num_seqs, b.num_heads, b.num_kv_heads,
                                                  b.head_dim, b.max_context_len, prefix, 512)
    ws = torch.full((max(need, 1),), 255, dtype=torch.uint8, device=dev)

    def step():
        pkv.paged_prefix_decode_attention(t["q"], t["kc"], t["vc"], pt, prefix, t["bt"], t["cl"],
                                          b.block_size, b.scale, max_context_len=b.max_context_len,
                                          partition_size=512, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = oracle.paged_prefix_decode(b.query, b.key_cache, b.value_cache, b.meta["prefix_table"],
                                     prefix, b.block_tables, b.context_lens, b.block_size, b.scale,
                                     b.dtype)
    assert max_err(to_f64(out), ref) <= TIGHT["f16"]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    for i in range(4):
        t["q"].copy_(torch.from_numpy(
            wl.encode(rng.standard_normal(b.query.size).astype(np.float32), "f16")
            .reshape(b.query.shape)).view(torch.float16).to(dev))
        step()
        torch.cuda.synchronize()
        eager = out.clone()
        out.fill_(float("nan"))
        ws.fill_(250 + i)  # a stale work counter and partials before the replay
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), i
