"""Paged-KV decode oracle -- TEST INFRASTRUCTURE ONLY.

A plain fp64 CPU implementation (C, built with gcc, no HIP) of what
single-query decode attention over a paged KV cache computes, written the way
the teaching version on the pages does it: gather the history through the
block table, then ordinary softmax attention.  Only ``tests/``, the smoke check
and the benchmark's CPU-baseline leg may import this package.  It shares no
code with the GPU library and never imports it.

Pages cited in this package:
  [P1] "从正确到更快：PagedAttention 的优化路线"
  [P2] "实现教学版 PagedAttention：从 block table 读取历史 KV cache"
  [P3] "算子与编译器：推理 Attention 与 KV Kernel"

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
(worked mapping printed on [P2], library attention, closed forms, brute force,
invariances, exhaustive element decoding).  No function is parity unpinned.

Array conventions: float32 arrays hold binary32 data; 16-bit data (binary16 or
bfloat16) is held as ``uint16`` bit patterns and needs an explicit ``dtype``
tag ('f16' or 'bf16'); quantised caches hold OCP E4M3 codes as ``uint8``.
"""
from __future__ import annotations

import contextlib
import ctypes
import functools
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (OpenMP over sequences)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(lib):
    p, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_f16.restype = dbl
    lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_bf16.restype = dbl
    lib.oracle_block_address.argtypes = [p, i32, i64, i32, p, p, p]
    lib.oracle_paged_gather.argtypes = [p, p, p, p, p, i32, i32, i32, i64, i32, i32, i32, ctypes.c_int]
    lib.oracle_attention.argtypes = [p, p, p, p, i32, i32, dbl]
    lib.oracle_paged_decode.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i64,
                                        dbl, ctypes.c_int, ctypes.c_int]
    lib.oracle_paged_prefix_decode.argtypes = [p, p, p, p, p, i32, p, p, i32, i32, i32, i32, i32,
                                               i32, i64, dbl, ctypes.c_int, ctypes.c_int]
    lib.oracle_paged_kv_write.argtypes = [p, p, p, p, p, i64, i32, i32, i32, i64, ctypes.c_int]
    lib.oracle_paged_prefill.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i64,
                                         dbl, ctypes.c_int, ctypes.c_int]
    lib.oracle_decode_e4m3.argtypes = [ctypes.c_uint8]
    lib.oracle_decode_e4m3.restype = dbl
    lib.oracle_encode_e4m3.argtypes = [ctypes.c_float]
    lib.oracle_encode_e4m3.restype = ctypes.c_uint8
    lib.oracle_paged_kv_write_e4m3.argtypes = [p, p, p, p, p, p, p, i64, i32, i32, i32, i64, ctypes.c_int]
    lib.oracle_paged_decode_e4m3.argtypes = [p, p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i64,
                                             dbl, ctypes.c_int, ctypes.c_int]
    lib.oracle_max_threads.argtypes = []
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Test hook: route this module's calls to another build of oracle.c
    (used to check that the pins catch deliberately planted mistakes)."""
    global _lib
    saved = _lib
    _lib = _bind(ctypes.CDLL(os.path.abspath(path)))
    _decode_table.cache_clear()
    try:
        yield
    finally:
        _lib = saved
        _decode_table.cache_clear()


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def _elem_check(a: np.ndarray, dtype: str) -> None:
    want = np.float32 if dtype == "f32" else np.uint16
    if a.dtype != want:
        raise TypeError(f"{dtype} data must be held as {np.dtype(want).name}, got {a.dtype}")


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def decode_f16(bits: int) -> float:
    return float(_load().oracle_decode_f16(int(bits)))


def decode_bf16(bits: int) -> float:
    return float(_load().oracle_decode_bf16(int(bits)))


@functools.lru_cache(maxsize=2)
def _decode_table(dtype: str) -> np.ndarray:
    fn = decode_f16 if dtype == "f16" else decode_bf16
    return np.array([fn(b) for b in range(65536)], dtype=np.float64)


def to_float64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Decode stored elements to fp64 with the oracle's own element decoders."""
    _elem_check(a, dtype)
    if dtype == "f32":
        return a.astype(np.float64)
    return _decode_table(dtype)[a]


def block_address(block_table, token_index: int, block_size: int):
    """[P2] "从逻辑 token 到物理 block": (logical_block_id, block_offset,
    physical_block_id) of one logical token."""
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    out = np.zeros(3, dtype=np.int64)
    rc = _load().oracle_block_address(_ptr(bt), bt.size, int(token_index), int(block_size),
                                      out[0:].ctypes.data, out[1:].ctypes.data,
                                      out[2:].ctypes.data)
    _check(rc, "block_address")
    return int(out[0]), int(out[1]), int(out[2])


def paged_gather(key_cache, value_cache, block_table, context_len: int, kv_head: int, dtype: str):
    """[P2] "单个 Sequence 的 paged gather": contiguous fp64 keys and values
    [context_len, head_dim] of one KV head, in logical token order."""
    _elem_check(key_cache, dtype)
    _elem_check(value_cache, dtype)
    nb, bs, kvh, d = key_cache.shape
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    keys = np.zeros((context_len, d), dtype=np.float64)
    values = np.zeros((context_len, d), dtype=np.float64)
    rc = _load().oracle_paged_gather(_ptr(keys), _ptr(values), _ptr(key_cache), _ptr(value_cache),
                                     _ptr(bt), bt.size, int(context_len), bs, nb, kvh,
                                     int(kv_head), d, DTYPE_CODE[dtype])
    _check(rc, "paged_gather")
    return keys, values


def attention(q, keys, values, scale: float):
    """[P2] "从 gather 后的 K/V 做 attention": one query head against
    contiguous fp64 keys/values."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    keys = np.ascontiguousarray(keys, dtype=np.float64)
    values = np.ascontiguousarray(values, dtype=np.float64)
    ctx, d = keys.shape
    out = np.zeros(d, dtype=np.float64)
    rc = _load().oracle_attention(_ptr(out), _ptr(q), _ptr(keys), _ptr(values), ctx, d,
                                  float(scale))
    _check(rc, "attention")
    return out


def paged_decode(query, key_cache, value_cache, block_tables, context_lens, block_size: int,
                 scale: float, dtype: str, num_threads: int = 0):
    """[P2] "扩展到 batch": fp64 output [num_seqs, num_heads, head_dim].

    ``scale`` is widened from the binary32 value the GPU receives."""
    for a in (query, key_cache, value_cache):
        _elem_check(a, dtype)
    nb, bs, kvh, d = key_cache.shape
    if bs != block_size:
        raise ValueError("block_size does not match the pool shape")
    b, h, dq = query.shape
    assert dq == d and value_cache.shape == key_cache.shape
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    assert bt.ndim == 2 and bt.shape[0] == b and cl.shape == (b,)
    out = np.zeros((b, h, d), dtype=np.float64)
    rc = _load().oracle_paged_decode(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
                                     _ptr(bt), _ptr(cl), b, h, kvh, d, bs, bt.shape[1], nb,
                                     float(np.float32(scale)), DTYPE_CODE[dtype], int(num_threads))
    _check(rc, "paged_decode")
    return out


def paged_prefix_decode(query, key_cache, value_cache, prefix_table, prefix_len: int,
                        block_tables, context_lens, block_size: int, scale: float, dtype: str,
                        num_threads: int = 0):
    """[P3] "4.1 为什么页面化会改变 kernel 设计" / "6. Prefix Cache 与 Attention
    Kernel 的关系": decode where tokens t < ``prefix_len`` of every sequence
    live in the shared pages ``prefix_table`` and later tokens in the
    sequence's own ``block_tables`` row (whose first prefix_len / block_size
    entries are ignored).  fp64 output [num_seqs, num_heads, head_dim]."""
    for a in (query, key_cache, value_cache):
        _elem_check(a, dtype)
    nb, bs, kvh, d = key_cache.shape
    if bs != block_size:
        raise ValueError("block_size does not match the pool shape")
    b, h, dq = query.shape
    assert dq == d and value_cache.shape == key_cache.shape
    pt = np.ascontiguousarray(prefix_table, dtype=np.int32).reshape(-1)
    if pt.size == 0:
        pt = np.zeros(1, dtype=np.int32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    assert bt.ndim == 2 and bt.shape[0] == b and cl.shape == (b,)
    out = np.zeros((b, h, d), dtype=np.float64)
    rc = _load().oracle_paged_prefix_decode(
        _ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache), _ptr(pt), int(prefix_len),
        _ptr(bt), _ptr(cl), b, h, kvh, d, bs, bt.shape[1], nb, float(np.float32(scale)),
        DTYPE_CODE[dtype], int(num_threads))
    _check(rc, "paged_prefix_decode")
    return out


def paged_prefill(query, key_cache, value_cache, block_tables, context_lens, query_start_loc,
                  block_size: int, scale: float, dtype: str, num_threads: int = 0):
    """[P2] "attention mask 在哪里": multi-token paged attention with a causal
    mask.  ``query`` [total_queries, H, D] packs each sequence's q_len =
    query_start_loc[s+1] - query_start_loc[s] queries, the last q_len
    positions of its context; fp64 output of the same shape."""
    for a in (query, key_cache, value_cache):
        _elem_check(a, dtype)
    nb, bs, kvh, d = key_cache.shape
    if bs != block_size:
        raise ValueError("block_size does not match the pool shape")
    tq, h, dq = query.shape
    assert dq == d and value_cache.shape == key_cache.shape
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    qsl = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    b = cl.shape[0]
    assert bt.ndim == 2 and bt.shape[0] == b and qsl.shape == (b + 1,) and qsl[-1] == tq
    out = np.zeros((tq, h, d), dtype=np.float64)
    rc = _load().oracle_paged_prefill(_ptr(out), _ptr(query), _ptr(key_cache), _ptr(value_cache),
                                      _ptr(bt), _ptr(cl), _ptr(qsl), b, h, kvh, d, bs, bt.shape[1],
                                      nb, float(np.float32(scale)), DTYPE_CODE[dtype],
                                      int(num_threads))
    _check(rc, "paged_prefill")
    return out


def paged_kv_write(key, value, key_cache, value_cache, slot_mapping) -> None:
    """[P2] "写入 slot 和读取 block table 必须一致": in-place byte copy of
    each token's K/V rows to its slot (negative slots skipped)."""
    nb, bs, kvh, d = key_cache.shape
    t = key.shape[0]
    assert key.shape == (t, kvh, d) and value.shape == key.shape
    assert key.dtype == key_cache.dtype == value.dtype == value_cache.dtype
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    assert sm.shape == (t,)
    rc = _load().oracle_paged_kv_write(_ptr(key), _ptr(value), _ptr(key_cache), _ptr(value_cache),
                                       _ptr(sm), t, kvh, d, bs, nb, key.dtype.itemsize)
    _check(rc, "paged_kv_write")


def decode_e4m3(bits: int) -> float:
    """One OCP E4M3 code as a float (NaN for 0x7F / 0xFF)."""
    return float(_load().oracle_decode_e4m3(int(bits)))


def encode_e4m3(values) -> np.ndarray:
    """binary32 values -> E4M3 codes (saturating at 448, ties to even)."""
    v = np.ascontiguousarray(values, dtype=np.float32).reshape(-1)
    enc = _load().oracle_encode_e4m3
    return np.array([enc(float(x)) for x in v], dtype=np.uint8).reshape(np.shape(values))


@functools.lru_cache(maxsize=1)
def _e4m3_table() -> np.ndarray:
    return np.array([decode_e4m3(b) for b in range(256)], dtype=np.float64)


def e4m3_to_float64(codes: np.ndarray) -> np.ndarray:
    """Decode E4M3 codes with the oracle's own decoder."""
    if codes.dtype != np.uint8:
        raise TypeError("E4M3 codes are held as uint8")
    return _e4m3_table()[codes]


def paged_kv_write_e4m3(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale,
                        src_dtype: str) -> None:
    """Quantised slot write: codes = encode(x * (1 / scale[kv head]))."""
    _elem_check(key, src_dtype)
    _elem_check(value, src_dtype)
    nb, bs, kvh, d = key_cache.shape
    assert key_cache.dtype == np.uint8 and value_cache.dtype == np.uint8
    t = key.shape[0]
    assert key.shape == (t, kvh, d) and value.shape == key.shape
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    ks = np.ascontiguousarray(k_scale, dtype=np.float32)
    vs = np.ascontiguousarray(v_scale, dtype=np.float32)
    assert sm.shape == (t,) and ks.shape == (kvh,) and vs.shape == (kvh,)
    rc = _load().oracle_paged_kv_write_e4m3(_ptr(key), _ptr(value), _ptr(key_cache),
                                            _ptr(value_cache), _ptr(sm), _ptr(ks), _ptr(vs), t, kvh,
                                            d, bs, nb, DTYPE_CODE[src_dtype])
    _check(rc, "paged_kv_write_e4m3")


def paged_decode_e4m3(query, key_cache, value_cache, k_scale, v_scale, block_tables,
                      context_lens, block_size: int, scale: float, dtype: str,
                      num_threads: int = 0):
    """Decode over E4M3 caches with per-KV-head scales; ``dtype`` is the
    query's element type.  fp64 output [num_seqs, num_heads, head_dim]."""
    _elem_check(query, dtype)
    nb, bs, kvh, d = key_cache.shape
    assert key_cache.dtype == np.uint8 and value_cache.shape == key_cache.shape
    if bs != block_size:
        raise ValueError("block_size does not match the pool shape")
    b, h, dq = query.shape
    assert dq == d
    ks = np.ascontiguousarray(k_scale, dtype=np.float32)
    vs = np.ascontiguousarray(v_scale, dtype=np.float32)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    assert ks.shape == (kvh,) and vs.shape == (kvh,)
    assert bt.ndim == 2 and bt.shape[0] == b and cl.shape == (b,)
    out = np.zeros((b, h, d), dtype=np.float64)
    rc = _load().oracle_paged_decode_e4m3(_ptr(out), _ptr(query), _ptr(key_cache),
                                          _ptr(value_cache), _ptr(ks), _ptr(vs), _ptr(bt), _ptr(cl),
                                          b, h, kvh, d, bs, bt.shape[1], nb, float(np.float32(scale)),
                                          DTYPE_CODE[dtype], int(num_threads))
    _check(rc, "paged_decode_e4m3")
    return out
