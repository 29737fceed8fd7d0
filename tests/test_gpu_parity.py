"""HIP path against the fp64 oracle on identical seeded inputs (MI355X)."""
import itertools

import numpy as np
import pytest

import oracle
from paged_kv_decode_13_amd import workloads as wl
from tests.gpu_helpers import (TIGHT, TOL, gpu_step, max_err, oracle_step, rounded_out_ok,
                               to_f64, upload)

pytestmark = pytest.mark.gpu


def _edge_lengths(bs):
    # boundary lengths of the pages' correctness list plus an empty context
    return [1, bs - 1, bs, bs + 1, 3 * bs + 1, 0, 137, 700]


EDGE_CASES = [(dt, bs, g, d) for dt, bs, g, d in itertools.product(
    ("f32", "f16", "bf16"), (4, 8, 16, 32, 64), (1, 2, 4, 8), (64, 128))]


@pytest.mark.parametrize("dtype,bs,group,head_dim", EDGE_CASES,
                         ids=[f"{a}-bs{b}-g{c}-d{d}" for a, b, c, d in EDGE_CASES])
def test_edge_lengths(cuda, dtype, bs, group, head_dim):
    """Heterogeneous batch of boundary context lengths, unsplit and split.
    fp32 outputs are held to the arithmetic bound; cache-dtype outputs to
    that bound plus the rounding of the output itself (short contexts give
    |out| up to ~3, where half a bf16 ulp is 7.8e-3)."""
    seed = 1000 + bs * 7 + group * 3 + head_dim
    b = wl.make_batch(_edge_lengths(bs), num_heads=2 * group, num_kv_heads=2, head_dim=head_dim,
                      block_size=bs, dtype=dtype, seed=seed, write_new_token=True, table_slack=1)
    ref = oracle_step(b)
    assert np.array_equal(ref[5], np.zeros_like(ref[5]))  # empty context -> zeros
    for ps in (0, max(64, bs)):
        t = upload(b, cuda)
        out = to_f64(gpu_step(b, t, partition_size=ps, out_dtype="f32"))
        err = max_err(out, ref)
        assert err <= TIGHT[dtype], (ps, err)
        out = to_f64(gpu_step(b, upload(b, cuda), partition_size=ps))
        assert rounded_out_ok(out, ref, dtype), (ps, max_err(out, ref))


def test_write_is_bit_exact(cuda):
    import torch

    import paged_kv_decode_13_amd as pkv

    for dtype, d, bs in (("f32", 64, 4), ("f16", 128, 16), ("bf16", 128, 32), ("bf16", 64, 64)):
        b = wl.make_batch([5, 1, 40, 17, 64], num_heads=8, num_kv_heads=4, head_dim=d,
                          block_size=bs, dtype=dtype, seed=77, write_new_token=True)
        b.slot_mapping[1] = -1  # skipped token
        t = upload(b, cuda)
        pkv.paged_kv_write(t["nk"], t["nv"], t["kc"], t["vc"], t["slots"])
        torch.cuda.synchronize()
        kc, vc = b.key_cache.copy(), b.value_cache.copy()
        oracle.paged_kv_write(b.new_key, b.new_value, kc, vc, b.slot_mapping)
        assert np.array_equal(t["kc"].cpu().view(torch.uint8).numpy().ravel(), kc.view(np.uint8).ravel())
        assert np.array_equal(t["vc"].cpu().view(torch.uint8).numpy().ravel(), vc.view(np.uint8).ravel())


def test_split_partition_sizes_agree(cuda):
    b = wl.make_batch([1, 300, 2049, 4000], num_heads=16, num_kv_heads=4, head_dim=128,
                      block_size=16, dtype="bf16", seed=5)
    ref = oracle_step(b)
    t = upload(b, cuda)
    outs = {}
    for ps in (0, 16, 64, 512, 4096, 8192):
        outs[ps] = to_f64(gpu_step(b, t, partition_size=ps, out_dtype="f32"))
        assert max_err(outs[ps], ref) <= TIGHT["bf16"], ps
    # a partition covering every context is the unsplit launch: same bits
    assert np.array_equal(outs[0], outs[4096]) and np.array_equal(outs[0], outs[8192])


def test_deterministic(cuda):
    import torch

    b = wl.make_batch([777, 3000, 12], num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                      dtype="bf16", seed=9)
    t = upload(b, cuda)
    a1 = gpu_step(b, t, partition_size=512).cpu()
    a2 = gpu_step(b, t, partition_size=512).cpu()
    assert a1.view(torch.int16).equal(a2.view(torch.int16))


def test_attend_then_write(cuda):
    """The other ordering of a step: attend over ctx tokens, then store the new
    token at position ctx (its slot lies past the attended context)."""
    import torch

    import paged_kv_decode_13_amd as pkv

    b = wl.make_batch([9, 16, 33], num_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                      dtype="f16", seed=21, write_new_token=True, table_slack=1)
    ctx = b.context_lens - 1  # attend before the token exists
    t = upload(b, cuda)
    t["cl"] = torch.from_numpy(ctx.astype(np.int32)).to(cuda)
    out = pkv.paged_decode_attention(t["q"], t["kc"], t["vc"], t["bt"], t["cl"], 16, b.scale,
                                     max_context_len=int(ctx.max()), out_dtype=torch.float32)
    pkv.paged_kv_write(t["nk"], t["nv"], t["kc"], t["vc"], t["slots"])
    torch.cuda.synchronize()
    ref = oracle_step(b, write=False, context_lens=ctx.astype(np.int32))
    assert max_err(to_f64(out), ref) <= TIGHT["f16"]
    # the written rows now hold the new token and are read at position ctx
    kc = b.key_cache.copy()
    vc = b.value_cache.copy()
    oracle.paged_kv_write(b.new_key, b.new_value, kc, vc, b.slot_mapping)
    assert np.array_equal(t["kc"].cpu().view(torch.int16).numpy().view(np.uint16), kc)


def test_out_of_range_contents_give_nan_not_faults(cuda):
    """Lengths past the host bound and page ids past the pool are caught in
    the kernel: that sequence's output is NaN, nothing is read out of range,
    the other sequences are unaffected."""
    import torch

    b = wl.make_batch([40, 50, 60], num_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                      dtype="bf16", seed=2)
    ref = oracle_step(b)
    t = upload(b, cuda)
    cl = b.context_lens.copy()
    cl[0] = 61  # beyond max_context_len = 60
    t["cl"] = torch.from_numpy(cl).to(cuda)
    bt = b.block_tables.copy()
    bt[2, 1] = b.num_blocks + 1000  # page id past the pool
    t["bt"] = torch.from_numpy(bt).to(cuda)
    for ps in (0, 16):
        out = to_f64(gpu_step(b, t, partition_size=ps, out_dtype="f32", max_context_len=60))
        assert np.isnan(out[0]).all() and np.isnan(out[2]).all()
        assert max_err(out[1], ref[1]) <= TIGHT["bf16"]
    # an out-of-range slot is skipped by the write
    import paged_kv_decode_13_amd as pkv

    before = t["kc"].clone()
    nk = torch.ones((1, 2, 128), dtype=torch.bfloat16, device=cuda)
    bad = torch.tensor([b.num_blocks * 16 + 3], dtype=torch.int64, device=cuda)
    pkv.paged_kv_write(nk, nk, t["kc"], t["vc"], bad)
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int16), t["kc"].view(torch.int16))  # bits: NaN rows too


def test_parity_is_sensitive_to_mutations(cuda):
    """A wrong table entry, length or slot must break parity."""
    import torch

    b = wl.make_batch([33, 90, 200], num_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                      dtype="bf16", seed=8, write_new_token=True)
    ref = oracle_step(b)
    # one table entry pointing at another sequence's page
    t = upload(b, cuda)
    bt = b.block_tables.copy()
    bt[1, 2] = b.block_tables[2, 0]
    t["bt"] = torch.from_numpy(bt).to(cuda)
    assert max_err(to_f64(gpu_step(b, t, out_dtype="f32")), ref) > TIGHT["bf16"]
    # a context one token short
    t = upload(b, cuda)
    cl = b.context_lens.copy()
    cl[2] -= 1
    t["cl"] = torch.from_numpy(cl).to(cuda)
    assert max_err(to_f64(gpu_step(b, t, out_dtype="f32")), ref) > TIGHT["bf16"]
    # a slot one row off: the poisoned target row stays NaN
    t = upload(b, cuda)
    sl = b.slot_mapping.copy()
    sl[0] += 1
    t["slots"] = torch.from_numpy(sl).to(cuda)
    assert max_err(to_f64(gpu_step(b, t, out_dtype="f32")), ref) > TIGHT["bf16"]


def test_workspace_any_initial_contents(cuda):
    """One workspace serves consecutive calls of different shapes, and before
    every call it is overwritten with arbitrary bytes (the counter area
    included: all ones, random, a count just below the call's last ticket):
    no call depends on what an earlier call left there."""
    import torch

    import paged_kv_decode_13_amd as pkv

    ws = torch.empty(1 << 22, dtype=torch.uint8, device=cuda)
    gen = torch.Generator(device="cpu").manual_seed(5)
    cases = [([300, 17, 4000], 8, 2, 512), ([5000], 32, 8, 1024), ([1, 2, 3, 64, 65], 16, 4, 0),
             ([2049, 99], 8, 8, 2048)]
    fills = ["ones", "random", "near_last"]
    for i, (lens, h, kvh, ps) in enumerate(cases * 2):
        b = wl.make_batch(lens, num_heads=h, num_kv_heads=kvh, head_dim=128, block_size=16,
                          dtype="f16", seed=len(lens) + h)
        t = upload(b, cuda)
        assert pkv.paged_decode_workspace_size(b.num_seqs, h, 128, b.max_context_len, ps) <= ws.numel()
        fill = fills[i % len(fills)]
        if fill == "ones":
            ws.fill_(255)
        elif fill == "random":
            ws.copy_(torch.randint(0, 256, (ws.numel(),), dtype=torch.uint8, generator=gen))
        else:
            ws.fill_(0)
            ws[:4].view(torch.int32).fill_(3)  # a small stale count
        out = pkv.paged_decode_attention(t["q"], t["kc"], t["vc"], t["bt"], t["cl"], 16, b.scale,
                                         max_context_len=b.max_context_len, partition_size=ps,
                                         out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        assert max_err(to_f64(out), oracle_step(b)) <= TIGHT["f16"], (i, fill)


@pytest.mark.parametrize("kv", [None, "e4m3"], ids=["f16", "e4m3"])
def test_unsplit_without_workspace(cuda, kv):
    """An unsplit call with no workspace (one workgroup per (sequence, KV
    head), no counter) matches the oracle for every group size; a split call
    without one is refused."""
    import torch

    import paged_kv_decode_13_amd as pkv

    lens = [0, 1, 15, 16, 17, 300, 1025, 2500]
    for g in (1, 2, 4, 8):
        b = wl.make_batch(lens, num_heads=4 * g, num_kv_heads=4, head_dim=128, block_size=16,
                          dtype="f16", seed=40 + g, write_new_token=True, kv_dtype=kv)
        t = upload(b, cuda)
        if kv:
            pkv.paged_kv_write_fp8(t["nk"], t["nv"], t["kc"], t["vc"], t["slots"], t["ks"], t["vs"])
            out = pkv.paged_decode_attention_fp8(
                t["q"], t["kc"], t["vc"], t["ks"], t["vs"], t["bt"], t["cl"], 16, b.scale,
                max_context_len=b.max_context_len, out_dtype=torch.float32,
                workspace=pkv.NO_WORKSPACE)
        else:
            pkv.paged_kv_write(t["nk"], t["nv"], t["kc"], t["vc"], t["slots"])
            out = pkv.paged_decode_attention(t["q"], t["kc"], t["vc"], t["bt"], t["cl"], 16, b.scale,
                                             max_context_len=b.max_context_len,
                                             out_dtype=torch.float32, workspace=pkv.NO_WORKSPACE)
        torch.cuda.synchronize()
        assert max_err(to_f64(out), oracle_step(b)) <= TIGHT["f16"], g
    with pytest.raises(pkv.PagedKVError, match="WORKSPACE"):
        if kv:
            pkv.paged_decode_attention_fp8(t["q"], t["kc"], t["vc"], t["ks"], t["vs"], t["bt"],
                                           t["cl"], 16, b.scale, max_context_len=b.max_context_len,
                                           partition_size=512, workspace=pkv.NO_WORKSPACE)
        else:
            pkv.paged_decode_attention(t["q"], t["kc"], t["vc"], t["bt"], t["cl"], 16, b.scale,
                                       max_context_len=b.max_context_len, partition_size=512,
                                       workspace=pkv.NO_WORKSPACE)


def test_unit_order_edges(cuda):
    """Unit order (whole partitions first, then the partial last partitions
    longest first, by a counting sort every workgroup repeats): lengths that
    are exact multiples of the partition (no partial unit), all-partial
    batches, empty contexts, a 300-sequence batch (two sorting rounds, the
    second partial) whose tails fall in every length class, the largest
    batch one call accepts, and a merge over a row count that is not a
    multiple of four."""
    import torch

    cases = [([512, 1024, 2048], 512), ([3, 5, 200, 0, 511], 512), ([0, 0, 700, 1536], 256),
             ([(i * 53) % 1000 for i in range(300)], 512),
             ([1 + (i * 37) % 300 for i in range(4096)], 128)]
    for lens, ps in cases:
        b = wl.make_batch(lens, num_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                          dtype="bf16", seed=len(lens))
        ref = oracle_step(b)
        out = to_f64(gpu_step(b, upload(b, cuda), partition_size=ps, out_dtype="f32"))
        assert max_err(out, ref) <= TIGHT["bf16"], (len(lens), ps)
    # 1367 sequences x 3 heads = 4101 rows: the merge takes four rows per
    # workgroup from 4096 rows on, and the last workgroup holds one
    b = wl.make_batch([1 + (i * 29) % 90 for i in range(1367)], num_heads=3, num_kv_heads=3,
                      head_dim=128, block_size=16, dtype="bf16", seed=1367)
    ref = oracle_step(b)
    out = to_f64(gpu_step(b, upload(b, cuda), partition_size=16, out_dtype="f32"))
    assert max_err(out, ref) <= TIGHT["bf16"]
    import paged_kv_decode_13_amd as pkv

    with pytest.raises(pkv.PagedKVError):
        b = wl.make_batch([4] * 4097, num_heads=2, num_kv_heads=2, head_dim=128, block_size=16,
                          dtype="bf16", seed=1)
        gpu_step(b, upload(b, cuda), partition_size=0)


def test_bulk_prefill_write_then_decode(cuda):
    """A prompt-sized write (every token of every prompt) is bit-exact, and a
    decode over the prompts then reads exactly the written rows."""
    import torch

    import paged_kv_decode_13_amd as pkv

    for dtype, d, bs, kvh in (("bf16", 128, 16, 8), ("f16", 64, 4, 2), ("f32", 128, 32, 1)):
        b = wl.make_prefill([700, 1, 16, 2049], num_heads=4 * kvh, num_kv_heads=kvh, head_dim=d,
                            block_size=bs, dtype=dtype, seed=3)
        t = upload(b, cuda)
        pkv.paged_kv_write(t["nk"], t["nv"], t["kc"], t["vc"], t["slots"])
        torch.cuda.synchronize()
        kc, vc = b.key_cache.copy(), b.value_cache.copy()
        oracle.paged_kv_write(b.new_key, b.new_value, kc, vc, b.slot_mapping)
        assert np.array_equal(t["kc"].cpu().view(torch.uint8).numpy().ravel(), kc.view(np.uint8).ravel())
        assert np.array_equal(t["vc"].cpu().view(torch.uint8).numpy().ravel(), vc.view(np.uint8).ravel())
        out = to_f64(gpu_step(b, t, write=False, partition_size=512 if bs <= 32 else 0,
                              out_dtype="f32"))
        assert max_err(out, oracle_step(b)) <= TIGHT[dtype], dtype


@pytest.mark.parametrize("kv,bs,ps", [(None, 16, 256), (None, 4, 64), (None, 32, 512),
                                      ("e4m3", 16, 128)],
                         ids=["bf16-bs16-p256", "bf16-bs4-p64", "bf16-bs32-p512", "e4m3-bs16-p128"])
def test_partition_runs(cuda, kv, bs, ps):
    """Short partitions go in runs of four whole partitions per work unit,
    one wave per partition, each wave writing its partial directly; the rest
    of a span is one unit per partition.  Lengths at and around run
    boundaries (exactly one run, a run and a partial partition, two runs, a
    run and three singles, fewer than four partitions), every group size;
    then a bad page inside a run makes exactly that sequence NaN."""
    import torch

    run = 4 * ps
    lens = [run, run + 1, 2 * run, run + 3 * ps, 3 * ps, ps - 1, 0, 5 * run + 17, run - bs]
    for g in (1, 2, 4, 8):
        b = wl.make_batch(lens, num_heads=4 * g, num_kv_heads=4, head_dim=128, block_size=bs,
                          dtype="bf16", seed=60 + g, write_new_token=True, partition_size=ps,
                          kv_dtype=kv)
        out = to_f64(gpu_step(b, upload(b, cuda), out_dtype="f32"))
        assert max_err(out, oracle_step(b)) <= TIGHT["bf16"], (g, kv, bs, ps)
    b = wl.make_batch(lens, num_heads=16, num_kv_heads=4, head_dim=128, block_size=bs,
                      dtype="bf16", seed=71, write_new_token=True, partition_size=ps, kv_dtype=kv)
    ref = oracle_step(b)
    t = upload(b, cuda)
    bt = b.block_tables.copy()
    bt[2, (run + ps) // bs] = b.num_blocks + 5  # inside the second run of sequence 2
    t["bt"] = torch.from_numpy(bt).to(cuda)
    out = to_f64(gpu_step(b, t, out_dtype="f32"))
    assert np.isnan(out[2]).all()
    keep = [i for i in range(len(lens)) if i != 2]
    assert max_err(out[keep], ref[keep]) <= TIGHT["bf16"]
