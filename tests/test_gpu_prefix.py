"""Shared-prefix decode (paged_prefix_decode_attention) against the fp64
oracle's shared-prefix decode on identical seeded inputs (MI355X)."""
import itertools

import numpy as np
import pytest

import oracle
from paged_kv_decode_13_amd import workloads as wl
from tests.gpu_helpers import (TIGHT, TOL, gpu_prefix_step, max_err, oracle_prefix_step,
                               rounded_out_ok, to_f64, upload)

pytestmark = pytest.mark.gpu


def _lengths(prefix_len, bs):
    # empty, inside the prefix, exactly the prefix, one past it, a ragged
    # suffix, a suffix of whole pages, a long suffix
    return [0, max(1, prefix_len // 3), prefix_len, prefix_len + 1, prefix_len + 3 * bs + 5,
            prefix_len + 4 * bs, prefix_len + 700, 1, prefix_len - 1 if prefix_len > 1 else 2]


# (prefix tokens, sequences): prefixes of a ragged last 64-token chunk, of
# several chunks and splits, and longer than one split; the batch sizes give
# ragged 64-row blocks
EDGE = [(dt, bs, g) for dt, bs, g in itertools.product(("f16", "bf16"), (4, 8, 16, 32, 64),
                                                       (1, 2, 4, 8))]


@pytest.mark.parametrize("dtype,bs,group", EDGE, ids=[f"{a}-bs{b}-g{c}" for a, b, c in EDGE])
def test_prefix_edges(cuda, dtype, bs, group):
    prefix_len = {4: 200, 8: 520, 16: 1024, 32: 96, 64: 2112}[bs]
    lens = _lengths(prefix_len, bs) * 3  # 27 sequences: ragged row blocks for every G
    b = wl.make_prefix_batch(lens, prefix_len, num_heads=2 * group, num_kv_heads=2, head_dim=128,
                             block_size=bs, dtype=dtype, seed=500 + bs + group)
    print(f"\n[prefix-edge] {dtype} bs={bs} G={group} prefix={prefix_len}", flush=True)
    ref = oracle_prefix_step(b)
    for ps in (0, max(64, bs)):
        out = to_f64(gpu_prefix_step(b, upload(b, cuda), partition_size=ps, out_dtype="f32"))
        assert max_err(out, ref) <= TIGHT[dtype], (ps, max_err(out, ref))
        assert np.array_equal(out[0], np.zeros_like(out[0]))
        out = to_f64(gpu_prefix_step(b, upload(b, cuda), partition_size=ps))
        assert rounded_out_ok(out, ref, dtype), (ps, max_err(out, ref))


def test_prefix_equals_plain_decode_on_same_history(cuda):
    """With the prefix ids also written into every table row, the plain decode
    and the shared-prefix decode see the same history; both match the
    oracle, and the oracle's two readings agree bit for bit."""
    b = wl.make_prefix_batch([300, 1200, 1025, 1800, 64], 1024, num_heads=32, num_kv_heads=8,
                             head_dim=128, block_size=16, dtype="bf16", seed=9,
                             own_prefix_entries="copy")
    ref = oracle_prefix_step(b)
    plain = oracle.paged_decode(b.query, b.key_cache, b.value_cache, b.block_tables,
                                b.context_lens, 16, b.scale, "bf16")
    assert np.array_equal(ref, plain)
    import paged_kv_decode_13_amd as pkv

    t = upload(b, cuda)
    out_p = to_f64(gpu_prefix_step(b, t, out_dtype="f32"))
    import torch

    out_d = to_f64(pkv.paged_decode_attention(t["q"], t["kc"], t["vc"], t["bt"], t["cl"], 16,
                                              b.scale, max_context_len=b.max_context_len,
                                              out_dtype=torch.float32))
    assert max_err(out_p, ref) <= TIGHT["bf16"] and max_err(out_d, ref) <= TIGHT["bf16"]


def test_prefix_out_of_range_contents(cuda):
    """A bad prefix page id makes NaN exactly the sequences that reach that
    page; a context past max_context_len makes that sequence NaN; the rest
    match the oracle."""
    bs, plen = 16, 512
    lens = [100, 200, 300, 400, 700, 30]
    b = wl.make_prefix_batch(lens, plen, num_heads=16, num_kv_heads=4, head_dim=128,
                             block_size=bs, dtype="f16", seed=31)
    ref = oracle_prefix_step(b)
    pt = b.meta["prefix_table"].copy()
    pt[15] = b.num_blocks + 100  # tokens 240..255 of the prefix
    t = upload(b, cuda)
    out = to_f64(gpu_prefix_step(b, t, prefix_table=pt, out_dtype="f32"))
    reach = np.array(lens) > 15 * bs
    assert np.isnan(out[reach]).all()
    assert max_err(out[~reach], ref[~reach]) <= TIGHT["f16"]
    import torch

    cl = t["cl"].clone()
    cl[2] = b.max_context_len + 1
    t["cl"] = cl
    out = to_f64(gpu_prefix_step(b, t, out_dtype="f32"))
    assert np.isnan(out[2]).all()
    keep = [0, 1, 3, 4, 5]
    assert max_err(out[keep], ref[keep]) <= TIGHT["f16"]
    torch.cuda.synchronize()


def test_prefix_deterministic_any_workspace_contents(cuda):
    """Three calls on one workspace with two suffix partitions per sequence,
    i.e. through the launch that runs the prefix units beside the persistent
    suffix grid, the workspace overwritten with arbitrary bytes before each
    (the counter area included): identical outputs."""
    import torch

    import paged_kv_decode_13_amd as pkv

    b = wl.make_prefix_batch([2100, 2048, 3000, 10, 2500] * 8, 2048, num_heads=32, num_kv_heads=8,
                             head_dim=128, block_size=32, dtype="bf16", seed=12, partition_size=512)
    t = upload(b, cuda)
    need = pkv.paged_prefix_decode_workspace_size(b.num_seqs, 32, 8, 128, b.max_context_len, 2048,
                                                  512)
    ws = torch.empty(need, dtype=torch.uint8, device=cuda)
    pt = torch.from_numpy(b.meta["prefix_table"]).to(cuda)
    outs = []
    for fill in (255, 7, 0):
        ws.fill_(fill)
        outs.append(pkv.paged_prefix_decode_attention(
            t["q"], t["kc"], t["vc"], pt, 2048, t["bt"], t["cl"], 32, b.scale,
            max_context_len=b.max_context_len, partition_size=512, workspace=ws).clone())
        torch.cuda.synchronize()
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    assert torch.equal(outs[0].view(torch.int16), outs[2].view(torch.int16))
    ref = oracle_prefix_step(b)
    assert max_err(to_f64(outs[0]), ref) <= TOL["bf16"]


@pytest.mark.parametrize("bs", wl.PREFIX_BLOCK_SIZES)
def test_prefix_full_config(cuda, bs):
    """The 128-sequence shared-prefix workload at full size through the
    shared-prefix entry point, every output element against the oracle, in
    the launch configuration the benchmark times and with fp32 outputs."""
    b = wl.make_config("prefix_fp16", block_size=bs)
    print(f"\n[prefix_fp16 bs={bs}] shared-prefix entry point", flush=True)
    ref = oracle_prefix_step(b)
    out = to_f64(gpu_prefix_step(b, upload(b, cuda)))
    assert max_err(out, ref) <= TOL["f16"], max_err(out, ref)
    out = to_f64(gpu_prefix_step(b, upload(b, cuda), out_dtype="f32", partition_size=0))
    assert max_err(out, ref) <= TIGHT["f16"], max_err(out, ref)


def test_prefix_more_units_than_fit_beside_the_suffix_grid(cuda):
    """768 sequences sharing a 1024-token prefix with 128-token suffix
    partitions: 48 row blocks x 8 KV heads = 384 prefix units share the
    launch with the persistent suffix grid, more than the CUs can hold beside
    it, so part of the suffix grid starts only as prefix units finish.
    Includes sequences shorter than the prefix and empty ones."""
    rng = np.random.default_rng(7681)
    prefix = 1024
    ctx = prefix + rng.integers(0, 300, size=768, endpoint=True)
    ctx[:8] = [0, 1, 500, prefix - 1, prefix, prefix + 1, prefix + 128, prefix + 129]
    b = wl.make_prefix_batch(ctx, prefix, num_heads=32, num_kv_heads=8, head_dim=128,
                             block_size=16, dtype="f16", seed=7681, partition_size=128)
    ref = oracle_prefix_step(b)
    out = to_f64(gpu_prefix_step(b, upload(b, cuda), out_dtype="f32"))
    assert max_err(out, ref) <= TIGHT["f16"], max_err(out, ref)
    out = to_f64(gpu_prefix_step(b, upload(b, cuda)))
    assert rounded_out_ok(out, ref, "f16"), max_err(out, ref)


def test_prefix_largest_batch(cuda):
    """The largest batch one call accepts (4096 sequences) through the
    shared-prefix call: the unit-order tables then fill most of a
    workgroup's LDS beside the prefix/decode union (one workgroup per CU),
    and the prefix units far outnumber the resident workgroups."""
    prefix = 256
    lens = [(i * 37) % (prefix + 120) for i in range(4096)]
    b = wl.make_prefix_batch(lens, prefix, num_heads=8, num_kv_heads=2, head_dim=128,
                             block_size=16, dtype="bf16", seed=4096, partition_size=64)
    ref = oracle_prefix_step(b)
    out = to_f64(gpu_prefix_step(b, upload(b, cuda), out_dtype="f32"))
    assert max_err(out, ref) <= TIGHT["bf16"], max_err(out, ref)


def test_prefix_entry_point_without_a_prefix(cuda):
    """prefix_len == 0 (no prefix table): the call is the plain decode.
    Unsplit, each sequence's epilogue stores its output itself; split, the
    partials go through the merge with no prefix slots before them."""
    lens = [0, 1, 15, 16, 17, 300, 1025, 2048, 4000]
    b = wl.make_prefix_batch(lens * 2, 0, num_heads=16, num_kv_heads=4, head_dim=128,
                             block_size=16, dtype="bf16", seed=4242)
    ref = oracle_prefix_step(b)
    assert np.array_equal(ref[0], np.zeros_like(ref[0]))
    for ps in (0, 256):
        out = to_f64(gpu_prefix_step(b, upload(b, cuda), partition_size=ps, out_dtype="f32"))
        assert max_err(out, ref) <= TIGHT["bf16"], (ps, max_err(out, ref))
        out = to_f64(gpu_prefix_step(b, upload(b, cuda), partition_size=ps))
        assert rounded_out_ok(out, ref, "bf16"), (ps, max_err(out, ref))
