"""Causal multi-token paged attention (paged_prefill_attention) against the
oracle's prefill on identical seeded inputs (MI355X)."""
import itertools

import numpy as np
import pytest

import oracle
from paged_kv_decode_13_amd import workloads as wl
from tests.gpu_helpers import TIGHT, TOL, abs_pool, max_err, single_rounding_ok, to_f64, upload

pytestmark = pytest.mark.gpu

TORCH_DT = {"f16": "float16", "bf16": "bfloat16", "f32": "float32"}


def _gpu_prefill(b, t, out_dtype=None, max_context_len=None):
    import torch

    import paged_kv_decode_13_amd as pkv

    dev = t["q"].device
    pq = wl.torch_view(b.meta["prompt_query"], b.dtype).to(dev)
    qsl = torch.from_numpy(b.meta["query_start_loc"]).to(dev)
    odt = None if out_dtype is None else getattr(torch, TORCH_DT[out_dtype])
    out = pkv.paged_prefill_attention(pq, t["kc"], t["vc"], t["bt"], t["cl"], qsl, b.block_size,
                                      b.scale, max_context_len=max_context_len or b.max_context_len,
                                      out_dtype=odt)
    torch.cuda.synchronize()
    return out


def _oracle_prefill(b, kc=None, vc=None):
    return oracle.paged_prefill(b.meta["prompt_query"], b.key_cache if kc is None else kc,
                                b.value_cache if vc is None else vc, b.block_tables,
                                b.context_lens, b.meta["query_start_loc"], b.block_size, b.scale,
                                b.dtype)


def _weighted_abs_v(b):
    """Per output element, the softmax-weighted mean of |v| over the row's
    history: the oracle's prefill over the pool with |V|."""
    return _oracle_prefill(b, vc=abs_pool(b.value_cache, b.dtype))


EDGE = [(dt, bs, g) for dt, bs, g in itertools.product(("f16", "bf16"), (4, 8, 16, 32, 64),
                                                       (1, 2, 4, 8))]


@pytest.mark.parametrize("dtype,bs,group", EDGE, ids=[f"{a}-bs{b}-g{c}" for a, b, c in EDGE])
def test_prefill_edges(cuda, dtype, bs, group):
    """Whole prompts of ragged lengths (one past 2048 tokens, so several
    staged page segments at block 4), chunked prefills continuing a cached
    history, single-query rows, an empty sequence and q_len = ctx = 1.
    binary32 outputs (two-term probabilities) within 1e-4; 16-bit outputs
    (probabilities rounded once) within the single-rounding bound."""
    ctx = [1, 37, 64, 65, 200, 300, 2100, 70, 0, 5]
    ql = [1, 37, 64, 13, 200, 1, 40, 70, 0, 5]
    b = wl.make_prefill_attention(ctx, ql, num_heads=2 * group, num_kv_heads=2, head_dim=128,
                                  block_size=bs, dtype=dtype, seed=3000 + bs + group)
    print(f"\n[prefill-edge] {dtype} bs={bs} G={group}", flush=True)
    ref = _oracle_prefill(b)
    out = to_f64(_gpu_prefill(b, upload(b, cuda), out_dtype="f32"))
    assert max_err(out, ref) <= TIGHT[dtype], max_err(out, ref)
    out = to_f64(_gpu_prefill(b, upload(b, cuda)))
    assert single_rounding_ok(out, ref, dtype, _weighted_abs_v(b)), max_err(out, ref)


def test_prefill_single_queries_match_decode(cuda):
    """q_len = 1 for every sequence: the prefill entry point and the decode
    entry point both match the oracle's decode."""
    import torch

    import paged_kv_decode_13_amd as pkv

    ctx = [5, 700, 1500, 33]
    b = wl.make_prefill_attention(ctx, [1, 1, 1, 1], num_heads=32, num_kv_heads=8, head_dim=128,
                                  block_size=16, dtype="bf16", seed=5)
    q = b.meta["prompt_query"]
    ref = oracle.paged_decode(q, b.key_cache, b.value_cache, b.block_tables, b.context_lens, 16,
                              b.scale, "bf16")
    t = upload(b, cuda)
    out = to_f64(_gpu_prefill(b, t, out_dtype="f32"))
    assert max_err(out, ref) <= TIGHT["bf16"]
    dec = pkv.paged_decode_attention(wl.torch_view(q, "bf16").to(cuda), t["kc"], t["vc"], t["bt"],
                                     t["cl"], 16, b.scale, max_context_len=b.max_context_len,
                                     out_dtype=torch.float32)
    assert max_err(to_f64(dec), ref) <= TIGHT["bf16"]


def test_prefill_out_of_range_contents(cuda):
    """A bad page id makes NaN exactly the rows that reach it; q_len > ctx or
    a context past max_context_len makes the sequence's rows NaN; a query
    range outside the packed rows is skipped; the rest match the oracle."""
    import torch

    ctx = [100, 300, 50, 80]
    ql = [100, 60, 50, 10]
    b = wl.make_prefill_attention(ctx, ql, num_heads=8, num_kv_heads=2, head_dim=128,
                                  block_size=16, dtype="f16", seed=9)
    ref = _oracle_prefill(b)
    t = upload(b, cuda)
    bt = t["bt"].clone()
    bt[1, 15] = b.num_blocks + 3  # tokens 240..255 of sequence 1
    t["bt"] = bt
    out = to_f64(_gpu_prefill(b, t, out_dtype="f32"))
    qsl = b.meta["query_start_loc"]
    pos1 = 300 - 60 + np.arange(60)
    rows1 = np.arange(qsl[1], qsl[2])
    reach = pos1 >= 240
    assert np.isnan(out[rows1[reach]]).all()
    assert max_err(out[rows1[~reach]], ref[rows1[~reach]]) <= TIGHT["f16"]
    others = np.r_[qsl[0]:qsl[1], qsl[2]:qsl[4]]
    assert max_err(out[others], ref[others]) <= TIGHT["f16"]
    # a context shorter than the sequence's query count, and one past max_context_len
    t = upload(b, cuda)
    cl = t["cl"].clone()
    cl[2] = 40  # q_len 50 > 40
    cl[3] = b.max_context_len + 1
    t["cl"] = cl
    out = to_f64(_gpu_prefill(b, t, out_dtype="f32"))
    assert np.isnan(out[qsl[2]:qsl[4]]).all()
    assert max_err(out[qsl[0]:qsl[2]], ref[qsl[0]:qsl[2]]) <= TIGHT["f16"]
    torch.cuda.synchronize()


def test_prefill_full_workload_decimated(cuda):
    """The prompt workload at full size (32 prompts of 1024..8192 tokens):
    the bulk write of every prompt token through slot_mapping, then causal
    attention of every prompt token.  Compared element by element over a
    deterministic decimation: every sequence, every query head (so every KV
    head), the first and the last query row of every 64-token chunk -- which
    touches every 32-token row tile of the kernel, each tile's diagonal
    included -- each against the oracle's decode of that row over the
    history it sees (a causal row at position p attends to tokens 0..p, the
    decode of context p + 1), at the 5e-3 bar of 16-bit caches."""
    import torch

    import paged_kv_decode_13_amd as pkv

    b = wl.add_prompt_queries(wl.make_prefill_config("prefill_bf16"), seed=11)
    t = upload(b, cuda)
    pkv.paged_kv_write(t["nk"], t["nv"], t["kc"], t["vc"], t["slots"])
    out = _gpu_prefill(b, t)
    torch.cuda.synchronize()
    kc, vc = b.key_cache.copy(), b.value_cache.copy()
    oracle.paged_kv_write(b.new_key, b.new_value, kc, vc, b.slot_mapping)
    qsl = b.meta["query_start_loc"]
    rows, seqs, ctxs = [], [], []
    for s_ in range(b.num_seqs):
        n = int(b.context_lens[s_])
        for c0 in range(0, n, 64):
            for pos in sorted({c0, min(n - 1, c0 + 63)}):
                rows.append(int(qsl[s_]) + pos)
                seqs.append(s_)
                ctxs.append(pos + 1)
    rows = np.asarray(rows)
    seqs = np.asarray(seqs)
    print(f"\n[prefill_bf16] {rows.size} query rows x {b.num_heads} heads", flush=True)
    ref = oracle.paged_decode(np.ascontiguousarray(b.meta["prompt_query"][rows]), kc, vc,
                              np.ascontiguousarray(b.block_tables[seqs]),
                              np.asarray(ctxs, dtype=np.int32), b.block_size, b.scale, "bf16")
    got = to_f64(out[torch.from_numpy(rows).to(out.device)])
    err = max_err(got, ref)
    print(f"[prefill_bf16] max|err| {err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_pool_past_4gib(cuda):
    """A pool larger than 4 GiB with the batch's pages at its top (every K/V
    byte read lies past the 4 GiB mark): the prefill's 64-bit addressing
    (pools under 4 GiB use 32-bit offsets from the pool's base) and the
    decode's, against the oracle on the same rows in the batch's own compact
    pool."""
    import torch

    from tests.gpu_helpers import gpu_step, oracle_step

    b = wl.make_prefill_attention([300, 1000, 64, 0, 777], [300, 17, 64, 0, 5], num_heads=8,
                                  num_kv_heads=2, head_dim=128, block_size=16, dtype="bf16",
                                  seed=4242)
    nb = b.key_cache.shape[0]
    page_bytes = b.block_size * b.num_kv_heads * b.head_dim * 2
    big = (9 << 29) // page_bytes + nb  # 4.5 GiB of pages below the batch's
    base = big - nb
    assert base * page_bytes > (4 << 30)
    print(f"\n[pool-past-4gib] {big} pages of {page_bytes} B", flush=True)
    t = upload(b, cuda)
    kc = torch.zeros((big,) + tuple(t["kc"].shape[1:]), dtype=t["kc"].dtype, device=cuda)
    vc = torch.zeros_like(kc)
    kc[base:] = t["kc"]
    vc[base:] = t["vc"]
    table = b.block_tables.astype(np.int64)
    table = np.where((table >= 0) & (table < nb), table + base, table).astype(np.int32)
    t.update(kc=kc, vc=vc, bt=torch.from_numpy(table).to(cuda))
    ref = _oracle_prefill(b)
    out = to_f64(_gpu_prefill(b, t, out_dtype="f32"))
    assert max_err(out, ref) <= TIGHT["bf16"], max_err(out, ref)
    out = to_f64(_gpu_prefill(b, t))
    assert single_rounding_ok(out, ref, "bf16", _weighted_abs_v(b)), max_err(out, ref)
    dref = oracle_step(b, write=False)
    for ps in (0, 64):
        dout = to_f64(gpu_step(b, t, partition_size=ps, out_dtype="f32", write=False))
        assert max_err(dout, dref) <= TIGHT["bf16"], (ps, max_err(dout, dref))
    del kc, vc
    torch.cuda.empty_cache()
