"""Seeded synthetic decode batches.

This module only draws inputs: random values, context lengths, page
assignments and the slot of each step's new token.  It holds none of the
attention arithmetic, imports neither the GPU binding nor the oracle, and is
the one module both sides may share.

Shapes and distributions follow the five decode workloads this library is
measured on (all values N(0, 1), drawn as binary32 and rounded to the storage
type round-to-nearest-even):

  tiny_fp32    1 seq, context 37, block 4, 4/4 heads, head_dim 64, pool of 16
               blocks, table = 10 ids of a seeded permutation, fp32, plus one
               new token written through slot_mapping;
  mha_fp16     32 seqs, 32/32 heads, head_dim 128, block 16, contexts uniform
               in [1, 4096], fp16; 512-token KV partitions;
  gqa_bf16     256 seqs, 32/8 heads, head_dim 128, block 16, contexts
               log-uniform in [128, 16000], bf16, one new token per sequence;
               5120-token KV partitions (8192 for its E4M3-cache variant);
  long_bf16    4 seqs x 32768, 64/8 heads, head_dim 128, block 32, bf16,
               512-token KV partitions;
  prefix_fp16  128 seqs sharing one 2048-token prefix (same physical pages)
               plus unique suffixes uniform in [0, 1024]; 32/8 heads,
               head_dim 128, fp16, block 8/16/32/64 on identical logical data;
               1024-token KV partitions.
(The partition sizes of the workloads without a prescribed one are the
fastest of 256..16384 measured on MI355X; the long-context workload's 512
is part of its definition.)

Pages of every table are disjoint runs of a shuffled pool sized to fit
(except the shared prefix), so consecutive logical blocks are never
physically adjacent by construction.  With ``poison=True`` every row no valid
context reaches is NaN -- the spare pool block, the slots past the context
in each last page, and the slot a new token is about to be written to -- so
an over-read or a missed write shows up as NaN in the output.

Storage: float32 arrays for fp32; uint16 bit patterns for fp16 / bf16.
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, field

import numpy as np

DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}
NAN_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0, "e4m3": 0x7F}

CONFIG_NAMES = ("tiny_fp32", "mha_fp16", "gqa_bf16", "long_bf16", "prefix_fp16")
PREFILL_NAMES = ("prefill_bf16",)
# the GQA batch-256 workload over an 8-bit (E4M3) cache: same lengths and
# page tables as gqa_bf16 (same seed), bf16 queries, per-KV-head scales
QUANT_NAMES = ("gqa_fp8",)
CONFIG_SEEDS = {name: i + 1 for i, name in enumerate(CONFIG_NAMES)}
CONFIG_SEEDS["gqa_fp8"] = CONFIG_SEEDS["gqa_bf16"]
PREFIX_BLOCK_SIZES = (8, 16, 32, 64)

_CHUNK = 1 << 22  # elements per independently seeded chunk of a large fill


@dataclass
class DecodeBatch:
    """One decode step's inputs (host arrays)."""

    name: str
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    query: np.ndarray  # [B, H, D]
    key_cache: np.ndarray  # [NB, bs, KVH, D]
    value_cache: np.ndarray
    block_tables: np.ndarray  # int32 [B, MB]
    context_lens: np.ndarray  # int32 [B]
    scale: float  # a binary32 value
    new_key: np.ndarray | None = None  # [T, KVH, D]
    new_value: np.ndarray | None = None
    slot_mapping: np.ndarray | None = None  # int64 [T]
    partition_size: int = 0
    poison_block: int | None = None
    unique_tokens: int | None = None  # distinct cached tokens (shared prefix counted once)
    meta: dict = field(default_factory=dict)
    kv_dtype: str | None = None  # cache element type when it differs from dtype ("e4m3")
    k_scale: np.ndarray | None = None  # float32 [KVH]: E4M3 caches only
    v_scale: np.ndarray | None = None

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.meta.get("num_blocks", self.key_cache.shape[0]))

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def cache_dtype(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def elem_bytes(self) -> int:
        """Bytes of one cached K or V element."""
        return DTYPE_BYTES[self.cache_dtype]

    @property
    def total_tokens(self) -> int:
        return int(self.context_lens.astype(np.int64).sum())

    def kv_bytes_logical(self) -> int:
        """K and V bytes the decode must read: sum(ctx) * KVH * D * 2 * b."""
        return self.total_tokens * self.num_kv_heads * self.head_dim * 2 * self.elem_bytes

    def kv_bytes_unique(self) -> int:
        toks = self.total_tokens if self.unique_tokens is None else self.unique_tokens
        return toks * self.num_kv_heads * self.head_dim * 2 * self.elem_bytes


# ----------------------------------------------------------------------------
# random fills


def _normal_f32(seed_seq: np.random.SeedSequence, n: int, threads: int | None = None) -> np.ndarray:
    """n standard normals as float32, drawn in fixed-size independently seeded
    chunks so the result does not depend on the thread count."""
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, math.ceil(n / _CHUNK))
    seeds = seed_seq.spawn(nchunks)

    def fill(i: int) -> None:
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        np.random.Generator(np.random.PCG64(seeds[i])).standard_normal(
            hi - lo, dtype=np.float32, out=out[lo:hi])

    if nchunks == 1:
        fill(0)
    else:
        workers = threads or min(16, os.cpu_count() or 1)
        with _cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def encode(values_f32: np.ndarray, dtype: str) -> np.ndarray:
    """binary32 values -> storage array for ``dtype`` (round to nearest even)."""
    values_f32 = np.ascontiguousarray(values_f32, dtype=np.float32)
    if dtype == "f32":
        return values_f32
    if dtype == "f16":
        return values_f32.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(values_f32).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dtype)


def _random_storage(seed_seq, shape, dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    flat = _normal_f32(seed_seq, n)
    step = 1 << 26
    for lo in range(0, n, step):
        out[lo:lo + step] = encode(flat[lo:lo + step], dtype)
    return out.reshape(shape)


def _random_e4m3(seed_seq, shape, scales: np.ndarray) -> np.ndarray:
    """E4M3 codes of N(0,1) values divided by their KV head's scale (the
    head is axis -2 of ``shape``), saturated to +-448 and rounded by torch's
    float8_e4m3fn conversion."""
    import torch

    n = int(np.prod(shape))
    d, kvh = shape[-1], shape[-2]
    out = np.empty(n, dtype=np.uint8)
    flat = _normal_f32(seed_seq, n)
    inv = (np.float32(1) / scales.astype(np.float32)).astype(np.float32)
    step = (1 << 26) // (kvh * d) * (kvh * d)
    for lo in range(0, n, step):
        x = flat[lo:lo + step].reshape(-1, kvh, d) * inv[None, :, None]
        x = np.clip(x, -448.0, 448.0).astype(np.float32)
        out[lo:lo + step] = torch.from_numpy(x.reshape(-1)).to(torch.float8_e4m3fn).view(
            torch.uint8).numpy()
    return out.reshape(shape)


def nan_value(dtype: str):
    if dtype == "f32":
        return np.array([NAN_BITS["f32"]], dtype=np.uint32).view(np.float32)[0]
    if dtype == "e4m3":
        return np.uint8(NAN_BITS["e4m3"])
    return np.uint16(NAN_BITS[dtype])


def storage_dtype(dtype: str):
    return {"f32": np.float32, "e4m3": np.uint8}.get(dtype, np.uint16)


# ----------------------------------------------------------------------------
# page assignment


def _disjoint_tables(rng: np.random.Generator, blocks_per_seq: np.ndarray):
    """Shuffle a pool of exactly sum(blocks_per_seq) ids and hand each sequence
    a consecutive run of the shuffled list.  One extra id (the last) is the
    spare block that pads every table."""
    total = int(blocks_per_seq.sum())
    ids = rng.permutation(total).astype(np.int32)
    spare = total
    mb = max(1, int(blocks_per_seq.max()) if blocks_per_seq.size else 1)
    tables = np.full((blocks_per_seq.size, mb), spare, dtype=np.int32)
    pos = 0
    for s, n in enumerate(blocks_per_seq):
        tables[s, :n] = ids[pos:pos + n]
        pos += int(n)
    return tables, total + 1, spare


def _row_index(tables: np.ndarray, seq: int, token: int, block_size: int) -> int:
    """Flat row (physical_block * block_size + offset) a seeded layout assigns
    to one logical token -- the slot a block allocator hands out."""
    return int(tables[seq, token // block_size]) * block_size + token % block_size


def _poison_rows(cache: np.ndarray, rows: np.ndarray, dtype: str) -> None:
    flat = cache.reshape(-1, cache.shape[2], cache.shape[3])
    flat[rows] = nan_value(dtype)


def _tail_rows(tables, context_lens, block_size) -> np.ndarray:
    """Rows past each context inside its last page."""
    rows = []
    for s, ctx in enumerate(context_lens):
        ctx = int(ctx)
        if ctx % block_size:
            last = int(tables[s, (ctx - 1) // block_size])
            rows.extend(last * block_size + o for o in range(ctx % block_size, block_size))
    return np.asarray(rows, dtype=np.int64)


# ----------------------------------------------------------------------------
# generic batch builder


def make_batch(context_lens, *, num_heads: int, num_kv_heads: int, head_dim: int,
               block_size: int, dtype: str, seed: int, write_new_token: bool = False,
               poison: bool = True, partition_size: int = 0, name: str = "custom",
               table_slack: int = 0, values: bool = True, kv_dtype: str | None = None) -> DecodeBatch:
    """A decode batch over disjoint shuffled pages.

    With ``write_new_token`` each sequence with a non-empty context gets one new
    K/V row whose slot is its logical position ``ctx - 1`` (the token is
    written first, then attended to); its pool row starts out NaN when
    ``poison`` is set.  ``table_slack`` adds spare table columns (padded with
    the spare block id).  ``values=False`` builds the layout only (lengths,
    tables, slots); the value arrays are then zero-size placeholders."""
    ctx = np.asarray(context_lens, dtype=np.int64).reshape(-1)
    if ctx.size and ctx.min() < 0:
        raise ValueError("context lengths must be >= 0")
    ss = np.random.SeedSequence(seed)
    s_perm, s_q, s_k, s_v, s_nk, s_nv = ss.spawn(6)
    rng = np.random.Generator(np.random.PCG64(s_perm))
    bps = (ctx + block_size - 1) // block_size
    tables, nb, spare = _disjoint_tables(rng, bps)
    if table_slack:
        tables = np.concatenate(
            [tables, np.full((tables.shape[0], table_slack), spare, np.int32)], axis=1)
    b = ctx.size
    shape = (nb, block_size, num_kv_heads, head_dim)
    cdt = kv_dtype or dtype
    k_scale = v_scale = None
    if cdt == "e4m3":
        # per-KV-head scales in [1/64, 1/32]: N(0,1) values stay well inside +-448
        s_ks, s_vs = ss.spawn(2)
        k_scale = np.random.Generator(np.random.PCG64(s_ks)).uniform(
            1 / 64, 1 / 32, num_kv_heads).astype(np.float32)
        v_scale = np.random.Generator(np.random.PCG64(s_vs)).uniform(
            1 / 64, 1 / 32, num_kv_heads).astype(np.float32)
    if values:
        if cdt == "e4m3":
            kc = _random_e4m3(s_k, shape, k_scale)
            vc = _random_e4m3(s_v, shape, v_scale)
        else:
            kc = _random_storage(s_k, shape, dtype)
            vc = _random_storage(s_v, shape, dtype)
        q = _random_storage(s_q, (b, num_heads, head_dim), dtype)
    else:
        kc = vc = np.zeros((0, block_size, num_kv_heads, head_dim), storage_dtype(cdt))
        q = np.zeros((0, num_heads, head_dim), storage_dtype(dtype))
    batch = DecodeBatch(name=name, dtype=dtype, num_heads=num_heads, num_kv_heads=num_kv_heads,
                        head_dim=head_dim, block_size=block_size, query=q, key_cache=kc,
                        value_cache=vc, block_tables=tables,
                        context_lens=ctx.astype(np.int32),
                        scale=float(np.float32(1.0 / math.sqrt(head_dim))),
                        partition_size=partition_size, poison_block=spare,
                        kv_dtype=kv_dtype if cdt != dtype else None, k_scale=k_scale,
                        v_scale=v_scale)
    if write_new_token:
        slots = np.array([_row_index(tables, s, int(c) - 1, block_size) if c > 0 else -1
                          for s, c in enumerate(ctx)], dtype=np.int64)
        if values:
            batch.new_key = _random_storage(s_nk, (b, num_kv_heads, head_dim), dtype)
            batch.new_value = _random_storage(s_nv, (b, num_kv_heads, head_dim), dtype)
        batch.slot_mapping = slots
    batch.meta["num_blocks"] = nb
    if poison and values:
        rows = [np.arange(spare * block_size, (spare + 1) * block_size, dtype=np.int64),
                _tail_rows(tables, ctx, block_size)]
        if write_new_token:
            rows.append(batch.slot_mapping[batch.slot_mapping >= 0])
        rows = np.concatenate(rows)
        _poison_rows(kc, rows, cdt)
        _poison_rows(vc, rows, cdt)
    return batch


def make_decode_steps(context_lens, steps: int, *, num_heads: int, num_kv_heads: int,
                      head_dim: int, block_size: int, dtype: str, seed: int,
                      kv_dtype: str | None = None, partition_size: int = 0):
    """Inputs of ``steps`` consecutive decode steps of an engine loop: every
    sequence appends one token per step.  The token at position p goes to
    slot table[p // block_size] * block_size + p % block_size, and a sequence
    whose next position opens a page first takes a fresh page id from a
    shuffled free list (extra pages, NaN-filled until written), as a block
    allocator would; the table grows accordingly.

    Returns ``(batch, per_step)``: ``batch`` holds the initial pool and
    tables (already widened to the final length), and each ``per_step``
    entry holds that step's ``query``, ``new_key``, ``new_value``,
    ``slot_mapping`` and the ``block_tables`` / ``context_lens`` after its
    token is appended (what the decode of that step reads)."""
    ctx0 = np.asarray(context_lens, dtype=np.int64).reshape(-1)
    batch = make_batch(ctx0, num_heads=num_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                       block_size=block_size, dtype=dtype, seed=seed, poison=True,
                       partition_size=partition_size, name="decode_steps", kv_dtype=kv_dtype)
    cdt = batch.cache_dtype
    final = ctx0 + steps
    width = max(1, int(((final + block_size - 1) // block_size).max()))
    spare = batch.poison_block
    tables = np.full((ctx0.size, width), spare, np.int32)
    tables[:, :batch.block_tables.shape[1]] = batch.block_tables
    # pages the steps open, appended to the pool, NaN until written
    opened = int(sum(((f + block_size - 1) // block_size) - ((c + block_size - 1) // block_size)
                     for c, f in zip(ctx0, final)))
    nb0 = batch.key_cache.shape[0]
    extra = np.full((opened,) + batch.key_cache.shape[1:], nan_value(cdt), storage_dtype(cdt))
    batch.key_cache = np.concatenate([batch.key_cache, extra])
    batch.value_cache = np.concatenate([batch.value_cache, extra.copy()])
    batch.meta["num_blocks"] = nb0 + opened
    batch.block_tables = tables.copy()
    ss = np.random.SeedSequence([seed, 17])
    s_free, s_steps = ss.spawn(2)
    free = list(np.random.Generator(np.random.PCG64(s_free)).permutation(
        np.arange(nb0, nb0 + opened, dtype=np.int32)))
    ctx = ctx0.copy()
    b = ctx.size
    per_step = []
    for k, sk in enumerate(s_steps.spawn(steps)):
        s_q, s_nk, s_nv = sk.spawn(3)
        slots = np.empty(b, np.int64)
        for s in range(b):
            pos = int(ctx[s])
            if pos % block_size == 0:
                tables[s, pos // block_size] = free.pop()
            slots[s] = _row_index(tables, s, pos, block_size)
            ctx[s] += 1
        per_step.append({
            "query": _random_storage(s_q, (b, num_heads, head_dim), dtype),
            "new_key": _random_storage(s_nk, (b, num_kv_heads, head_dim), dtype),
            "new_value": _random_storage(s_nv, (b, num_kv_heads, head_dim), dtype),
            "slot_mapping": slots,
            "block_tables": tables.copy(),
            "context_lens": ctx.astype(np.int32),
        })
    return batch, per_step


# ----------------------------------------------------------------------------
# the five named workloads


def _tiny_fp32(seed: int, poison: bool) -> DecodeBatch:
    ss = np.random.SeedSequence(seed)
    s_perm, s_q, s_k, s_v, s_nk, s_nv = ss.spawn(6)
    rng = np.random.Generator(np.random.PCG64(s_perm))
    bs, nb, ctx, kvh, d = 4, 16, 37, 4, 64
    table = rng.permutation(nb)[:10].astype(np.int32)
    shape = (nb, bs, kvh, d)
    kc = _random_storage(s_k, shape, "f32")
    vc = _random_storage(s_v, shape, "f32")
    q = _random_storage(s_q, (1, 4, d), "f32")
    slot = _row_index(table[None, :], 0, ctx - 1, bs)
    batch = DecodeBatch(name="tiny_fp32", dtype="f32", num_heads=4, num_kv_heads=kvh,
                        head_dim=d, block_size=bs, query=q, key_cache=kc, value_cache=vc,
                        block_tables=table[None, :].copy(),
                        context_lens=np.array([ctx], np.int32),
                        scale=float(np.float32(1.0 / math.sqrt(d))),
                        new_key=_random_storage(s_nk, (1, kvh, d), "f32"),
                        new_value=_random_storage(s_nv, (1, kvh, d), "f32"),
                        slot_mapping=np.array([slot], np.int64))
    if poison:
        unused = np.setdiff1d(np.arange(nb), table)
        rows = np.concatenate([np.arange(u * bs, (u + 1) * bs) for u in unused]
                              + [np.array([slot])]).astype(np.int64)
        _poison_rows(kc, rows, "f32")
        _poison_rows(vc, rows, "f32")
        batch.poison_block = int(unused[0])
    return batch


def _prefix_fp16(seed: int, block_size: int, poison: bool) -> DecodeBatch:
    """Logical data is drawn independently of the block size and then laid out
    in pages of ``block_size`` tokens, so every block size sees the same
    sequences."""
    if block_size not in PREFIX_BLOCK_SIZES:
        raise ValueError("prefix_fp16 runs at block sizes 8, 16, 32, 64")
    ss = np.random.SeedSequence(seed)
    s_len, s_perm, s_q, s_pk, s_pv, s_sk, s_sv = ss.spawn(7)
    b, h, kvh, d, prefix = 128, 32, 8, 128, 2048
    suffix = np.random.Generator(np.random.PCG64(s_len)).integers(0, 1024, size=b, endpoint=True)
    ctx = (prefix + suffix).astype(np.int64)
    n_suffix = int(suffix.sum())
    pk = _random_storage(s_pk, (prefix, kvh, d), "f16")
    pv = _random_storage(s_pv, (prefix, kvh, d), "f16")
    sk = _random_storage(s_sk, (n_suffix, kvh, d), "f16")
    sv = _random_storage(s_sv, (n_suffix, kvh, d), "f16")
    q = _random_storage(s_q, (b, h, d), "f16")
    # pages: prefix pages shared by all tables, then unique suffix pages
    n_pre = prefix // block_size
    suf_pages = (suffix + block_size - 1) // block_size
    total = n_pre + int(suf_pages.sum())
    perm_seed = np.random.SeedSequence([seed, block_size])
    ids = np.random.Generator(np.random.PCG64(perm_seed)).permutation(total).astype(np.int32)
    spare = total
    mb = n_pre + int(suf_pages.max())
    tables = np.full((b, mb), spare, dtype=np.int32)
    tables[:, :n_pre] = ids[:n_pre]
    pos = n_pre
    for s in range(b):
        n = int(suf_pages[s])
        tables[s, n_pre:n_pre + n] = ids[pos:pos + n]
        pos += n
    nb = total + 1
    kc = np.empty((nb, block_size, kvh, d), np.uint16)
    vc = np.empty_like(kc)
    kc[...] = nan_value("f16")
    vc[...] = nan_value("f16")
    kflat = kc.reshape(-1, kvh, d)
    vflat = vc.reshape(-1, kvh, d)
    t = np.arange(prefix)
    rows = tables[0, t // block_size].astype(np.int64) * block_size + t % block_size
    kflat[rows] = pk
    vflat[rows] = pv
    lo = 0
    for s in range(b):
        n = int(suffix[s])
        if n:
            t = prefix + np.arange(n)
            rows = tables[s, t // block_size].astype(np.int64) * block_size + t % block_size
            kflat[rows] = sk[lo:lo + n]
            vflat[rows] = sv[lo:lo + n]
        lo += n
    if not poison:
        # rows never reached by a context get finite values instead of NaN
        kflat[np.isnan(kflat.view(np.float16))] = 0
        vflat[np.isnan(vflat.view(np.float16))] = 0
    return DecodeBatch(name="prefix_fp16", dtype="f16", num_heads=h, num_kv_heads=kvh,
                       head_dim=d, block_size=block_size, query=q, key_cache=kc,
                       value_cache=vc, block_tables=tables,
                       context_lens=ctx.astype(np.int32),
                       scale=float(np.float32(1.0 / math.sqrt(d))),
                       partition_size=1024, poison_block=spare,
                       unique_tokens=prefix + n_suffix,
                       meta={"shared_prefix_tokens": prefix,
                             "prefix_table": np.ascontiguousarray(tables[0, :n_pre])})


def make_prefix_batch(context_lens, prefix_len: int, *, num_heads: int, num_kv_heads: int,
                      head_dim: int, block_size: int, dtype: str, seed: int,
                      partition_size: int = 0, own_prefix_entries: str = "invalid",
                      name: str = "prefix") -> DecodeBatch:
    """Sequences sharing a ``prefix_len``-token prompt prefix held in shared
    pages (``meta["prefix_table"]``), each followed by its own shuffled pages
    up to its context length; a sequence shorter than the prefix sees the
    first ``ctx`` prefix tokens.  ``own_prefix_entries`` fills the first
    prefix_len / block_size entries of every table row: "copy" (the shared
    ids, as a plain paged table would hold them), "poison" (the NaN spare
    page) or "invalid" (an id outside the pool) -- the shared-prefix decode
    must not read them.  Rows past each context in its last own page and the
    spare page are NaN."""
    if prefix_len % block_size:
        raise ValueError("the shared prefix is whole pages")
    ctx = np.asarray(context_lens, dtype=np.int64).reshape(-1)
    ss = np.random.SeedSequence(seed)
    s_perm, s_q, s_k, s_v = ss.spawn(4)
    rng = np.random.Generator(np.random.PCG64(s_perm))
    n_pre = prefix_len // block_size
    suf_pages = (np.maximum(ctx - prefix_len, 0) + block_size - 1) // block_size
    total = n_pre + int(suf_pages.sum())
    ids = rng.permutation(total).astype(np.int32)
    spare = total
    nb = total + 1
    mb = max(1, n_pre + int(suf_pages.max(initial=0)))
    tables = np.full((ctx.size, mb), spare, dtype=np.int32)
    fill = {"copy": None, "poison": spare, "invalid": nb + 7}[own_prefix_entries]
    tables[:, :n_pre] = ids[:n_pre] if fill is None else fill
    pos = n_pre
    for s in range(ctx.size):
        n = int(suf_pages[s])
        tables[s, n_pre:n_pre + n] = ids[pos:pos + n]
        pos += n
    shape = (nb, block_size, num_kv_heads, head_dim)
    kc = _random_storage(s_k, shape, dtype)
    vc = _random_storage(s_v, shape, dtype)
    q = _random_storage(s_q, (ctx.size, num_heads, head_dim), dtype)
    rows = [np.arange(spare * block_size, (spare + 1) * block_size, dtype=np.int64)]
    for s, c in enumerate(ctx):
        c = int(c)
        if c > prefix_len and c % block_size:
            last = int(tables[s, (c - 1) // block_size])
            rows.append(np.arange(last * block_size + c % block_size, (last + 1) * block_size))
    rows = np.concatenate(rows).astype(np.int64)
    _poison_rows(kc, rows, dtype)
    _poison_rows(vc, rows, dtype)
    batch = DecodeBatch(name=name, dtype=dtype, num_heads=num_heads, num_kv_heads=num_kv_heads,
                        head_dim=head_dim, block_size=block_size, query=q, key_cache=kc,
                        value_cache=vc, block_tables=tables, context_lens=ctx.astype(np.int32),
                        scale=float(np.float32(1.0 / math.sqrt(head_dim))),
                        partition_size=partition_size, poison_block=spare,
                        unique_tokens=min(prefix_len, int(ctx.max(initial=0)))
                        + int(np.maximum(ctx - prefix_len, 0).sum()))
    batch.meta.update(num_blocks=nb, shared_prefix_tokens=prefix_len,
                      prefix_table=np.ascontiguousarray(ids[:n_pre]))
    return batch


def make_config(name: str, *, block_size: int | None = None, seed: int | None = None,
                poison: bool = True, values: bool = True) -> DecodeBatch:
    """One of the five named decode workloads (seeded; default seed per name).
    ``values=False`` (not for tiny_fp32 / prefix_fp16) builds the layout only."""
    seed = CONFIG_SEEDS[name] if seed is None else seed
    if name == "tiny_fp32":
        return _tiny_fp32(seed, poison)
    if name == "prefix_fp16":
        return _prefix_fp16(seed, 16 if block_size is None else block_size, poison)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    if name == "mha_fp16":
        ctx = rng.integers(1, 4096, size=32, endpoint=True)
        return make_batch(ctx, num_heads=32, num_kv_heads=32, head_dim=128, block_size=16,
                          dtype="f16", seed=seed, poison=poison, partition_size=512,
                          name=name, values=values)
    if name in ("gqa_bf16", "gqa_fp8"):
        ctx = np.floor(np.exp(rng.uniform(math.log(128), math.log(16000), size=256)))
        ctx = np.clip(ctx, 128, 16000).astype(np.int64)
        return make_batch(ctx, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                          dtype="bf16", seed=seed, write_new_token=True, poison=poison,
                          partition_size=8192 if name == "gqa_fp8" else 5120, name=name,
                          values=values, kv_dtype="e4m3" if name == "gqa_fp8" else None)
    if name == "long_bf16":
        return make_batch(np.full(4, 32768), num_heads=64, num_kv_heads=8, head_dim=128,
                          block_size=32, dtype="bf16", seed=seed, poison=poison,
                          partition_size=512, name=name, values=values)
    raise KeyError(name)


def make_prefill(prompt_lens, *, num_heads: int, num_kv_heads: int, head_dim: int,
                 block_size: int, dtype: str, seed: int, name: str = "prefill",
                 partition_size: int = 0) -> DecodeBatch:
    """A prompt-sized write: every token of every prompt gets its K/V row and
    the slot of its logical position in the sequence's (shuffled) pages.  The
    pool starts all NaN -- nothing is cached yet -- so after the write a
    decode over the prompt reads exactly the written rows."""
    ctx = np.asarray(prompt_lens, dtype=np.int64).reshape(-1)
    ss = np.random.SeedSequence(seed)
    s_perm, s_q, s_k, s_v = ss.spawn(4)
    rng = np.random.Generator(np.random.PCG64(s_perm))
    bps = (ctx + block_size - 1) // block_size
    tables, nb, spare = _disjoint_tables(rng, bps)
    tokens = int(ctx.sum())
    slots = np.empty(tokens, dtype=np.int64)
    pos = 0
    for s, c in enumerate(ctx):
        t = np.arange(int(c))
        slots[pos:pos + c] = tables[s, t // block_size].astype(np.int64) * block_size + t % block_size
        pos += int(c)
    sdt = storage_dtype(dtype)
    kc = np.empty((nb, block_size, num_kv_heads, head_dim), sdt)
    kc[...] = nan_value(dtype)
    vc = kc.copy()
    return DecodeBatch(name=name, dtype=dtype, num_heads=num_heads, num_kv_heads=num_kv_heads,
                       head_dim=head_dim, block_size=block_size,
                       query=_random_storage(s_q, (ctx.size, num_heads, head_dim), dtype),
                       key_cache=kc, value_cache=vc, block_tables=tables,
                       context_lens=ctx.astype(np.int32),
                       scale=float(np.float32(1.0 / math.sqrt(head_dim))),
                       new_key=_random_storage(s_k, (tokens, num_kv_heads, head_dim), dtype),
                       new_value=_random_storage(s_v, (tokens, num_kv_heads, head_dim), dtype),
                       slot_mapping=slots, partition_size=partition_size, poison_block=spare)


def make_prefill_config(name: str, *, seed: int | None = None) -> DecodeBatch:
    """prefill_bf16: 32 prompts with lengths uniform in [1024, 8192] written
    into GQA-shaped pages (8 KV heads, head_dim 128, block 16, bf16) --
    the step just before decode, measured as a copy."""
    if name != "prefill_bf16":
        raise KeyError(name)
    seed = 11 if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    lens = rng.integers(1024, 8192, size=32, endpoint=True)
    return make_prefill(lens, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                        dtype="bf16", seed=seed, name=name, partition_size=2048)


def make_prefill_attention(context_lens, query_lens, *, num_heads: int, num_kv_heads: int,
                           head_dim: int, block_size: int, dtype: str, seed: int,
                           name: str = "prefill_attention") -> DecodeBatch:
    """A causal multi-token attention batch: every sequence's whole
    ``context_lens`` history is in a shuffled page pool (rows past each
    context and the spare page NaN), and its ``query_lens`` new queries are
    its last positions.  ``meta["prompt_query"]`` [sum(q_len), H, D] and
    ``meta["query_start_loc"]`` [B + 1] hold the packed queries."""
    ctx = np.asarray(context_lens, dtype=np.int64).reshape(-1)
    ql = np.asarray(query_lens, dtype=np.int64).reshape(-1)
    if ql.shape != ctx.shape or (ql > ctx).any() or (ql < 0).any():
        raise ValueError("each query count must lie in [0, context_len]")
    batch = make_batch(ctx, num_heads=num_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                       block_size=block_size, dtype=dtype, seed=seed, name=name)
    s_pq = np.random.SeedSequence([seed, 17])
    batch.meta["prompt_query"] = _random_storage(s_pq, (int(ql.sum()), num_heads, head_dim), dtype)
    batch.meta["query_start_loc"] = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    return batch


def add_prompt_queries(batch: DecodeBatch, seed: int) -> DecodeBatch:
    """Queries for every token of every prompt of a prefill batch (q_len =
    context_len), for the causal prefill attention after the prompt write."""
    ctx = batch.context_lens.astype(np.int64)
    s_pq = np.random.SeedSequence([seed, 17])
    batch.meta["prompt_query"] = _random_storage(
        s_pq, (int(ctx.sum()), batch.num_heads, batch.head_dim), batch.dtype)
    batch.meta["query_start_loc"] = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)
    return batch


def subset(batch: DecodeBatch, seqs) -> DecodeBatch:
    """The same pool restricted to some sequences (tables, lengths, queries
    and new tokens sliced; the pool is shared, not copied)."""
    seqs = np.asarray(seqs, dtype=np.int64)
    out = DecodeBatch(**{**batch.__dict__})
    out.query = np.ascontiguousarray(batch.query[seqs])
    out.block_tables = np.ascontiguousarray(batch.block_tables[seqs])
    out.context_lens = np.ascontiguousarray(batch.context_lens[seqs])
    if batch.slot_mapping is not None:
        out.new_key = np.ascontiguousarray(batch.new_key[seqs])
        out.new_value = np.ascontiguousarray(batch.new_value[seqs])
        out.slot_mapping = np.ascontiguousarray(batch.slot_mapping[seqs])
    out.unique_tokens = None
    out.meta = dict(batch.meta, subset=len(seqs))
    return out


def torch_view(a: np.ndarray, dtype: str):
    """A CPU torch tensor sharing ``a``'s memory, typed as ``dtype``."""
    import torch

    if dtype == "e4m3":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8))
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16)
