"""paged_decode_attention_noalloc (the entry point that allocates nothing,
its scratch a static device array) against paged_decode_attention with a
caller workspace: two calls in a row through the C ABI, the second with a
smaller batch, each bit for bit equal to the workspace entry point and
within the fp32-output bound of the oracle; an unsplit call; a request too
large for the scratch is refused."""
import ctypes

import numpy as np
import pytest

from paged_kv_decode_13_amd import workloads as wl
from tests.gpu_helpers import TIGHT, max_err, oracle_step, to_f64, upload

pytestmark = pytest.mark.gpu

WORKSPACE_ERR = 6


def _noalloc_call(lib, b, t, out, ps):
    import torch

    st = lib.paged_decode_attention_noalloc(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(t["q"].data_ptr()),
        ctypes.c_void_p(t["kc"].data_ptr()), ctypes.c_void_p(t["vc"].data_ptr()),
        ctypes.c_void_p(t["bt"].data_ptr()), ctypes.c_void_p(t["cl"].data_ptr()), b.num_seqs,
        b.num_heads, b.num_kv_heads, b.head_dim, b.block_size, b.max_blocks_per_seq, b.num_blocks,
        b.max_context_len, ctypes.c_float(b.scale), ps, 2 if b.dtype == "bf16" else 1, 0,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def test_noalloc_matches_workspace_entry_point(cuda):
    import torch

    import paged_kv_decode_13_amd as pkv

    lib = pkv._load()
    cases = [
        # (lengths, heads, kv heads, dtype, block, partition)
        ([1 + (i * 997) % 6000 for i in range(64)], 32, 8, "bf16", 16, 512),
        ([0, 1, 15, 17, 300, 1025, 2049, 33], 16, 2, "f16", 32, 256),  # smaller, after the first
        ([5, 700, 64, 3000], 8, 8, "bf16", 16, 0),                       # unsplit: the counter only
    ]
    for lens, h, kvh, dtype, bs, ps in cases:
        print(f"\n[noalloc] {len(lens)} seqs, {h}/{kvh} heads, {dtype}, block {bs}, partition {ps}",
              flush=True)
        b = wl.make_batch(lens, num_heads=h, num_kv_heads=kvh, head_dim=128, block_size=bs,
                          dtype=dtype, seed=len(lens) + h)
        t = upload(b, cuda)
        need = pkv.paged_decode_workspace_size(b.num_seqs, h, 128, b.max_context_len, ps)
        assert need <= pkv.NOALLOC_SCRATCH_BYTES
        out = torch.full((b.num_seqs, h, 128), float("nan"), dtype=torch.float32, device=cuda)
        assert _noalloc_call(lib, b, t, out, ps) == 0
        ws = torch.empty(need, dtype=torch.uint8, device=cuda)
        ref_gpu = pkv.paged_decode_attention(t["q"], t["kc"], t["vc"], t["bt"], t["cl"], bs, b.scale,
                                             max_context_len=b.max_context_len, partition_size=ps,
                                             out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_gpu)
        assert max_err(to_f64(out), oracle_step(b)) <= TIGHT[dtype]


def test_noalloc_refuses_what_does_not_fit(cuda):
    import torch

    import paged_kv_decode_13_amd as pkv

    lens = [1 + (i * 61) % 4000 for i in range(256)]
    b = wl.make_batch(lens, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      dtype="bf16", seed=9)
    t = upload(b, cuda)
    ps = 128  # 32 partitions per head: far more partials than the scratch holds
    assert pkv.paged_decode_workspace_size(b.num_seqs, 32, 128, b.max_context_len, ps) > \
        pkv.NOALLOC_SCRATCH_BYTES
    out = torch.zeros((b.num_seqs, 32, 128), dtype=torch.float32, device=cuda)
    assert _noalloc_call(pkv._load(), b, t, out, ps) == WORKSPACE_ERR
    with pytest.raises(pkv.PagedKVError, match="WORKSPACE"):
        pkv.paged_decode_attention_noalloc(t["q"], t["kc"], t["vc"], t["bt"], t["cl"], 16, b.scale,
                                           max_context_len=b.max_context_len, partition_size=ps,
                                           out=out)
    torch.cuda.synchronize()
    assert int(out.count_nonzero()) == 0  # nothing was launched
