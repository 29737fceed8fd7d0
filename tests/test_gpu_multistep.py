"""An engine loop on the GPU (MI355X): consecutive decode steps, each
writing every sequence's new token at its slot -- on a fresh page whenever
its position opens one -- and then decoding, through the C ABI; the oracle
runs the same steps on host copies of the pool.

Pages: "实现教学版 PagedAttention：从 block table 读取历史 KV cache", sections
"写入 slot 和读取 block table 必须一致" (the write and the read must use the
same slot for a token) and "PagedAttention 如何接入 mini vLLM" (a step writes
the new K/V, then attends over the history through the block table)."""
import numpy as np
import pytest

import oracle
from paged_kv_decode_13_amd import workloads as wl
from tests.gpu_helpers import TIGHT, max_err, to_f64

pytestmark = pytest.mark.gpu

# (dtype, cache dtype, heads, KV heads, head_dim, block_size, initial lengths, steps, partition)
CASES = {
    "bf16_gqa_bs16": ("bf16", None, 32, 8, 128, 16, [0, 1, 15, 16, 17, 255, 1000, 2047], 40, 0),
    "f16_gqa_bs4_split": ("f16", None, 32, 8, 128, 4, [0, 3, 4, 5, 63, 500], 24, 256),
    "bf16_mha_bs32": ("bf16", None, 16, 16, 128, 32, [31, 32, 33, 700], 36, 512),
    "e4m3_gqa_bs16": ("bf16", "e4m3", 32, 8, 128, 16, [1, 16, 300, 1500], 20, 512),
    "f32_d64_bs8": ("f32", None, 8, 2, 64, 8, [0, 7, 8, 100], 16, 0),
}


@pytest.mark.parametrize("case", list(CASES), ids=list(CASES))
def test_engine_steps_match_oracle(cuda, case):
    import torch

    import paged_kv_decode_13_amd as pkv

    dtype, kv, h, kvh, d, bs, ctx0, nsteps, ps = CASES[case]
    batch, steps = wl.make_decode_steps(ctx0, nsteps, num_heads=h, num_kv_heads=kvh, head_dim=d,
                                        block_size=bs, dtype=dtype, seed=97, kv_dtype=kv,
                                        partition_size=ps)
    quant = kv == "e4m3"
    print(f"\n[multistep] {case}: {batch.num_seqs} seqs, {nsteps} steps", flush=True)
    dev = cuda
    kc_h, vc_h = batch.key_cache.copy(), batch.value_cache.copy()
    cdt = batch.cache_dtype
    kc = wl.torch_view(kc_h, cdt).to(dev)
    vc = wl.torch_view(vc_h, cdt).to(dev)
    if quant:
        ks, vs = torch.from_numpy(batch.k_scale).to(dev), torch.from_numpy(batch.v_scale).to(dev)
    bound = int(steps[-1]["context_lens"].max())  # a static bound, as an engine would pass
    for k, st in enumerate(steps):
        q = wl.torch_view(st["query"], dtype).to(dev)
        nk = wl.torch_view(st["new_key"], dtype).to(dev)
        nv = wl.torch_view(st["new_value"], dtype).to(dev)
        slots = torch.from_numpy(st["slot_mapping"]).to(dev)
        bt = torch.from_numpy(st["block_tables"]).to(dev)
        cl = torch.from_numpy(st["context_lens"]).to(dev)
        if quant:
            pkv.paged_kv_write_fp8(nk, nv, kc, vc, slots, ks, vs)
            out = pkv.paged_decode_attention_fp8(q, kc, vc, ks, vs, bt, cl, bs, batch.scale,
                                                 max_context_len=bound, partition_size=ps,
                                                 out_dtype=torch.float32)
            oracle.paged_kv_write_e4m3(st["new_key"], st["new_value"], kc_h, vc_h, st["slot_mapping"],
                                       batch.k_scale, batch.v_scale, dtype)
            ref = oracle.paged_decode_e4m3(st["query"], kc_h, vc_h, batch.k_scale, batch.v_scale,
                                           st["block_tables"], st["context_lens"], bs, batch.scale,
                                           dtype)
        else:
            pkv.paged_kv_write(nk, nv, kc, vc, slots)
            out = pkv.paged_decode_attention(q, kc, vc, bt, cl, bs, batch.scale,
                                             max_context_len=bound, partition_size=ps,
                                             out_dtype=torch.float32)
            oracle.paged_kv_write(st["new_key"], st["new_value"], kc_h, vc_h, st["slot_mapping"])
            ref = oracle.paged_decode(st["query"], kc_h, vc_h, st["block_tables"],
                                      st["context_lens"], bs, batch.scale, dtype)
        torch.cuda.synchronize()
        err = max_err(to_f64(out), ref)
        assert err <= TIGHT[dtype], (case, k, err)
    # the pools after the last step, byte for byte
    for dev_pool, host_pool in ((kc, kc_h), (vc, vc_h)):
        got = dev_pool.cpu().contiguous().view(torch.uint8).numpy()
        assert np.array_equal(got.reshape(-1), host_pool.view(np.uint8).reshape(-1)), case
