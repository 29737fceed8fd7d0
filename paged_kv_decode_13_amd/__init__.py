"""Python binding of libpagedkv: paged-KV single-query decode attention on gfx950.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/pagedkv.h``.  PyTorch provides
device memory and the stream.  There is no fallback: if the library is not
built, or a tensor is not on a GPU, the call raises.

Entry points (same names as the C ABI):
  paged_kv_write(key, value, key_cache, value_cache, slot_mapping)
  paged_decode_attention(query, key_cache, value_cache, block_tables,
                         context_lens, block_size, scale, *, max_context_len,
                         partition_size=0, out=None, out_dtype=None,
                         workspace=None)
  paged_decode_workspace_size(num_seqs, num_heads, head_dim, max_context_len,
                              partition_size)
  paged_prefix_decode_attention(query, key_cache, value_cache, prefix_table,
                                prefix_len, block_tables, context_lens,
                                block_size, scale, *, max_context_len,
                                partition_size=0, out=None, out_dtype=None,
                                workspace=None)
  paged_prefix_decode_workspace_size(num_seqs, num_heads, num_kv_heads,
                                     head_dim, max_context_len, prefix_len,
                                     partition_size)
  paged_kv_write_fp8(key, value, key_cache, value_cache, slot_mapping,
                     k_scale, v_scale)
  paged_decode_attention_fp8(query, key_cache, value_cache, k_scale, v_scale,
                             block_tables, context_lens, block_size, scale,
                             *, max_context_len, partition_size=0, out=None,
                             out_dtype=None, workspace=None)
  paged_prefill_attention(query, key_cache, value_cache, block_tables,
                          context_lens, query_start_loc, block_size, scale,
                          *, max_context_len, out=None, out_dtype=None)
  paged_decode_attention_noalloc(query, key_cache, value_cache, block_tables,
                                 context_lens, block_size, scale, *,
                                 max_context_len, partition_size=0, out,
                                 out_dtype=None)
E4M3 caches are uint8 or torch.float8_e4m3fn tensors.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "paged_kv_write",
    "paged_decode_attention",
    "paged_decode_step",
    "paged_decode_workspace_size",
    "paged_prefix_decode_attention",
    "paged_prefix_decode_workspace_size",
    "paged_kv_write_fp8",
    "paged_decode_attention_fp8",
    "paged_prefill_attention",
    "paged_decode_attention_noalloc",
    "NOALLOC_SCRATCH_BYTES",
    "library_path",
    "PagedKVError",
    "NO_WORKSPACE",
]

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG_DIR, "libpagedkv.so")

PKV_F32, PKV_F16, PKV_BF16 = 0, 1, 2
# PKV_NOALLOC_SCRATCH_BYTES of include/pagedkv.h: the static scratch of
# paged_decode_attention_noalloc on each GPU
NOALLOC_SCRATCH_BYTES = 32 << 20
_STATUS = {0: "PKV_OK", 1: "PKV_ERR_NULL", 2: "PKV_ERR_SHAPE", 3: "PKV_ERR_DTYPE",
           4: "PKV_ERR_UNSUPPORTED", 5: "PKV_ERR_ALIGN", 6: "PKV_ERR_WORKSPACE", 7: "PKV_ERR_HIP"}

_lib = None


class PagedKVError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        self.name = _STATUS.get(status, str(status))
        msg = _load().pkv_status_string(status).decode()
        super().__init__(f"{what}: {self.name} ({msg})")


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"libpagedkv.so is not built ({_LIB_PATH}); run "
            "`python -m paged_kv_decode_13_amd.build` (there is no fallback path)")
    lib = ctypes.CDLL(_LIB_PATH)
    p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.paged_kv_write.argtypes = [p, p, p, p, p, i64, i32, i32, i32, i64, ctypes.c_int, p]
    lib.paged_kv_write.restype = ctypes.c_int
    lib.paged_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.paged_decode_workspace_size.restype = sz
    lib.paged_decode_attention.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i64,
                                           i32, ctypes.c_float, i32, ctypes.c_int, ctypes.c_int,
                                           p, sz, p]
    lib.paged_decode_attention.restype = ctypes.c_int
    lib.paged_decode_step.argtypes = [p, p, p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i64,
                                      i32, ctypes.c_float, i32, ctypes.c_int, ctypes.c_int, p, sz, p]
    lib.paged_decode_step.restype = ctypes.c_int
    lib.paged_prefix_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.paged_prefix_decode_workspace_size.restype = sz
    lib.paged_prefix_decode_attention.argtypes = [p, p, p, p, p, i32, p, p, i32, i32, i32, i32, i32,
                                                  i32, i64, i32, ctypes.c_float, i32, ctypes.c_int,
                                                  ctypes.c_int, p, sz, p]
    lib.paged_prefix_decode_attention.restype = ctypes.c_int
    lib.paged_kv_write_fp8.argtypes = [p, p, p, p, p, p, p, i64, i32, i32, i32, i64, ctypes.c_int, p]
    lib.paged_kv_write_fp8.restype = ctypes.c_int
    lib.paged_decode_attention_fp8.argtypes = [p, p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32,
                                               i64, i32, ctypes.c_float, i32, ctypes.c_int,
                                               ctypes.c_int, p, sz, p]
    lib.paged_decode_attention_fp8.restype = ctypes.c_int
    lib.paged_prefill_attention.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32,
                                            i64, i32, ctypes.c_float, ctypes.c_int, ctypes.c_int, p]
    lib.paged_prefill_attention.restype = ctypes.c_int
    lib.paged_decode_attention_noalloc.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, i32,
                                                   i64, i32, ctypes.c_float, i32, ctypes.c_int,
                                                   ctypes.c_int, p]
    lib.paged_decode_attention_noalloc.restype = ctypes.c_int
    lib.pkv_status_string.argtypes = [ctypes.c_int]
    lib.pkv_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _torch():
    import torch

    return torch


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.float32:
        return PKV_F32
    if dt == torch.float16:
        return PKV_F16
    if dt == torch.bfloat16:
        return PKV_BF16
    raise TypeError(f"unsupported dtype {dt}")


def _gpu(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream_handle(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


class _NoWorkspace:
    def __repr__(self) -> str:
        return "NO_WORKSPACE"


# Pass as ``workspace=`` to make an unsplit decode call without a workspace
# (the C ABI's NULL workspace: one workgroup per (sequence, KV head), no
# work counter).  A split call needs a workspace and raises.
NO_WORKSPACE = _NoWorkspace()


def _workspace(need: int, workspace, device):
    """(pointer, bytes) of the call's workspace: the caller's buffer, NULL
    for NO_WORKSPACE, or a fresh uninitialised one (no call depends on a
    workspace's earlier contents)."""
    torch = _torch()
    if workspace is NO_WORKSPACE:
        return None, 0
    if workspace is None:
        if not need:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    else:
        _gpu(workspace, "workspace")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def paged_kv_write(key, value, key_cache, value_cache, slot_mapping) -> None:
    """Store token i's K/V rows ``key[i]``/``value[i]`` ([num_kv_heads,
    head_dim]) at ``slot_mapping[i]`` (int64, physical_block * block_size +
    offset; negative = skip) of the paged pools, on the current stream."""
    torch = _torch()
    lib = _load()
    for t, n in ((key, "key"), (value, "value"), (key_cache, "key_cache"),
                 (value_cache, "value_cache"), (slot_mapping, "slot_mapping")):
        _gpu(t, n)
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    nb, bs, kvh, d = key_cache.shape
    tokens = key.shape[0]
    if tuple(key.shape) != (tokens, kvh, d) or value.shape != key.shape:
        raise ValueError("key/value must be [num_tokens, num_kv_heads, head_dim] of the pool")
    if value_cache.shape != key_cache.shape or slot_mapping.shape != (tokens,):
        raise ValueError("inconsistent shapes")
    if not (key.dtype == value.dtype == key_cache.dtype == value_cache.dtype):
        raise TypeError("key, value and the caches must share one dtype")
    st = lib.paged_kv_write(key.data_ptr(), value.data_ptr(), key_cache.data_ptr(),
                            value_cache.data_ptr(), slot_mapping.data_ptr(), tokens, kvh, d, bs,
                            nb, _dtype_code(key.dtype), _stream_handle(key.device))
    if st != 0:
        raise PagedKVError(st, "paged_kv_write")


def paged_decode_workspace_size(num_seqs: int, num_heads: int, head_dim: int,
                                max_context_len: int, partition_size: int) -> int:
    return int(_load().paged_decode_workspace_size(num_seqs, num_heads, head_dim,
                                                   max_context_len, partition_size))


def paged_decode_attention(query, key_cache, value_cache, block_tables, context_lens,
                           block_size: int, scale: float, *, max_context_len: int,
                           partition_size: int = 0, out=None, out_dtype=None, workspace=None):
    """Decode attention of ``query`` [num_seqs, num_heads, head_dim] over the
    paged pools [num_blocks, block_size, num_kv_heads, head_dim] through
    ``block_tables`` (int32 [num_seqs, max_blocks]) and ``context_lens``
    (int32 [num_seqs]).  Returns ``out`` [num_seqs, num_heads, head_dim] in
    ``out_dtype`` (default: the cache dtype).  ``max_context_len`` is a host
    upper bound of ``context_lens``; ``partition_size`` > 0 splits contexts
    into KV partitions merged by log-sum-exp.  ``workspace`` (a GPU buffer of
    at least ``paged_decode_workspace_size`` bytes, any contents) may be
    passed to avoid an allocation per call; ``NO_WORKSPACE`` runs an unsplit
    call without one."""
    torch = _torch()
    lib = _load()
    for t, n in ((query, "query"), (key_cache, "key_cache"), (value_cache, "value_cache"),
                 (block_tables, "block_tables"), (context_lens, "context_lens")):
        _gpu(t, n)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    nb, bs, kvh, d = key_cache.shape
    if bs != block_size:
        raise ValueError("block_size does not match key_cache.shape[1]")
    b, h, dq = query.shape
    if dq != d or value_cache.shape != key_cache.shape:
        raise ValueError("inconsistent shapes")
    if block_tables.dim() != 2 or block_tables.shape[0] != b or tuple(context_lens.shape) != (b,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs]")
    if not (query.dtype == key_cache.dtype == value_cache.dtype):
        raise TypeError("query and caches must share one dtype")
    dt = _dtype_code(query.dtype)
    odt = query.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((b, h, d), dtype=odt, device=query.device)
    else:
        _gpu(out, "out")
        if tuple(out.shape) != (b, h, d):
            raise ValueError("out must be [num_seqs, num_heads, head_dim]")
        odt = out.dtype
    need = paged_decode_workspace_size(b, h, d, int(max_context_len), int(partition_size))
    ws_ptr, ws_bytes = _workspace(need, workspace, query.device)
    st = lib.paged_decode_attention(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), b, h, kvh, d, bs,
        block_tables.shape[1], nb, int(max_context_len), float(scale), int(partition_size), dt,
        _dtype_code(odt), ws_ptr, ws_bytes, _stream_handle(query.device))
    if st != 0:
        raise PagedKVError(st, "paged_decode_attention")
    return out


def paged_decode_step(query, key_cache, value_cache, new_key, new_value, slot_mapping, block_tables,
                      context_lens, block_size: int, scale: float, *, max_context_len: int,
                      partition_size: int = 0, out=None, out_dtype=None, workspace=None):
    """One decode step in one launch: sequence s's new K/V rows
    ``new_key[s]``/``new_value[s]`` ([num_kv_heads, head_dim]) are stored at
    ``slot_mapping[s]`` (int64; negative: none), which must be the slot of
    its position ``context_lens[s] - 1``, and ``query`` attends over the
    history including them: the result of ``paged_kv_write`` then
    ``paged_decode_attention``.  A sequence whose slot is not that position's
    gets NaN and its rows are not stored.  The caches, head sizes and
    groups of ``paged_decode_attention``."""
    torch = _torch()
    lib = _load()
    for t, n in ((query, "query"), (key_cache, "key_cache"), (value_cache, "value_cache"),
                 (new_key, "new_key"), (new_value, "new_value"), (slot_mapping, "slot_mapping"),
                 (block_tables, "block_tables"), (context_lens, "context_lens")):
        _gpu(t, n)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    nb, bs, kvh, d = key_cache.shape
    if bs != block_size:
        raise ValueError("block_size does not match key_cache.shape[1]")
    b, h, dq = query.shape
    if dq != d or value_cache.shape != key_cache.shape:
        raise ValueError("inconsistent shapes")
    if block_tables.dim() != 2 or block_tables.shape[0] != b or tuple(context_lens.shape) != (b,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs]")
    if tuple(new_key.shape) != (b, kvh, d) or new_value.shape != new_key.shape:
        raise ValueError("new_key/new_value must be [num_seqs, num_kv_heads, head_dim]")
    if tuple(slot_mapping.shape) != (b,):
        raise ValueError("slot_mapping must be [num_seqs]")
    if not (query.dtype == key_cache.dtype == value_cache.dtype == new_key.dtype == new_value.dtype):
        raise TypeError("query, new rows and caches must share one dtype")
    dt = _dtype_code(query.dtype)
    odt = query.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((b, h, d), dtype=odt, device=query.device)
    else:
        _gpu(out, "out")
        if tuple(out.shape) != (b, h, d):
            raise ValueError("out must be [num_seqs, num_heads, head_dim]")
        odt = out.dtype
    need = paged_decode_workspace_size(b, h, d, int(max_context_len), int(partition_size))
    ws_ptr, ws_bytes = _workspace(need, workspace, query.device)
    st = lib.paged_decode_step(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        new_key.data_ptr(), new_value.data_ptr(), slot_mapping.data_ptr(), block_tables.data_ptr(),
        context_lens.data_ptr(), b, h, kvh, d, bs, block_tables.shape[1], nb, int(max_context_len),
        float(scale), int(partition_size), dt, _dtype_code(odt), ws_ptr, ws_bytes,
        _stream_handle(query.device))
    if st != 0:
        raise PagedKVError(st, "paged_decode_step")
    return out


def paged_decode_attention_noalloc(query, key_cache, value_cache, block_tables, context_lens,
                                   block_size: int, scale: float, *, max_context_len: int,
                                   partition_size: int = 0, out, out_dtype=None):
    """``paged_decode_attention`` through the entry point that allocates
    nothing: the split partials live in the library's static scratch of
    ``NOALLOC_SCRATCH_BYTES`` per GPU (larger requests raise PKV_ERR_WORKSPACE).
    ``out`` is required, so the call allocates nothing here either.  Calls
    whose kernels can overlap on one GPU share that scratch and race."""
    torch = _torch()
    lib = _load()
    for t, n in ((query, "query"), (key_cache, "key_cache"), (value_cache, "value_cache"),
                 (block_tables, "block_tables"), (context_lens, "context_lens"), (out, "out")):
        _gpu(t, n)
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    nb, bs, kvh, d = key_cache.shape
    if bs != block_size:
        raise ValueError("block_size does not match key_cache.shape[1]")
    b, h, dq = query.shape
    if dq != d or value_cache.shape != key_cache.shape:
        raise ValueError("inconsistent shapes")
    if block_tables.dim() != 2 or block_tables.shape[0] != b or tuple(context_lens.shape) != (b,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs]")
    if not (query.dtype == key_cache.dtype == value_cache.dtype):
        raise TypeError("query and caches must share one dtype")
    if tuple(out.shape) != (b, h, d):
        raise ValueError("out must be [num_seqs, num_heads, head_dim]")
    if out_dtype is not None and out.dtype != out_dtype:
        raise TypeError("out_dtype does not match out")
    st = lib.paged_decode_attention_noalloc(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), b, h, kvh, d, bs, block_tables.shape[1],
        nb, int(max_context_len), float(scale), int(partition_size), _dtype_code(query.dtype),
        _dtype_code(out.dtype), _stream_handle(query.device))
    if st != 0:
        raise PagedKVError(st, "paged_decode_attention_noalloc")
    return out


def paged_prefix_decode_workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int,
                                       head_dim: int, max_context_len: int, prefix_len: int,
                                       partition_size: int) -> int:
    return int(_load().paged_prefix_decode_workspace_size(num_seqs, num_heads, num_kv_heads,
                                                          head_dim, max_context_len, prefix_len,
                                                          partition_size))


def paged_prefix_decode_attention(query, key_cache, value_cache, prefix_table, prefix_len: int,
                                  block_tables, context_lens, block_size: int, scale: float, *,
                                  max_context_len: int, partition_size: int = 0, out=None,
                                  out_dtype=None, workspace=None):
    """Decode attention for a batch whose sequences share a prompt prefix:
    tokens t < ``prefix_len`` (a multiple of ``block_size``) of every sequence
    live in the pages ``prefix_table`` (int32 [prefix_len / block_size]),
    later tokens in the sequence's own ``block_tables`` row (whose first
    prefix_len / block_size entries are not read).  The prefix is read once
    per KV head for the whole batch.  Other arguments as
    ``paged_decode_attention``; 16-bit caches, head_dim 128."""
    torch = _torch()
    lib = _load()
    for t, n in ((query, "query"), (key_cache, "key_cache"), (value_cache, "value_cache"),
                 (prefix_table, "prefix_table"), (block_tables, "block_tables"),
                 (context_lens, "context_lens")):
        _gpu(t, n)
    if prefix_table.dtype != torch.int32 or block_tables.dtype != torch.int32 \
            or context_lens.dtype != torch.int32:
        raise TypeError("prefix_table, block_tables and context_lens must be int32")
    nb, bs, kvh, d = key_cache.shape
    if bs != block_size:
        raise ValueError("block_size does not match key_cache.shape[1]")
    b, h, dq = query.shape
    if dq != d or value_cache.shape != key_cache.shape:
        raise ValueError("inconsistent shapes")
    if block_tables.dim() != 2 or block_tables.shape[0] != b or tuple(context_lens.shape) != (b,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs]")
    if prefix_table.numel() * block_size < prefix_len:
        raise ValueError("prefix_table holds fewer pages than prefix_len needs")
    if not (query.dtype == key_cache.dtype == value_cache.dtype):
        raise TypeError("query and caches must share one dtype")
    dt = _dtype_code(query.dtype)
    odt = query.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((b, h, d), dtype=odt, device=query.device)
    else:
        _gpu(out, "out")
        if tuple(out.shape) != (b, h, d):
            raise ValueError("out must be [num_seqs, num_heads, head_dim]")
        odt = out.dtype
    need = paged_prefix_decode_workspace_size(b, h, kvh, d, int(max_context_len), int(prefix_len),
                                              int(partition_size))
    ws_ptr, ws_bytes = _workspace(need, workspace, query.device)
    st = lib.paged_prefix_decode_attention(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        prefix_table.data_ptr(), int(prefix_len), block_tables.data_ptr(), context_lens.data_ptr(),
        b, h, kvh, d, bs, block_tables.shape[1], nb, int(max_context_len), float(scale),
        int(partition_size), dt, _dtype_code(odt), ws_ptr, ws_bytes, _stream_handle(query.device))
    if st != 0:
        raise PagedKVError(st, "paged_prefix_decode_attention")
    return out


def _e4m3_cache(t, name: str):
    torch = _torch()
    _gpu(t, name)
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError(f"{name} must hold E4M3 codes (uint8 or float8_e4m3fn)")
    return t


def _scales(k_scale, v_scale, kvh: int):
    torch = _torch()
    for t, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        _gpu(t, n)
        if t.dtype != torch.float32 or tuple(t.shape) != (kvh,):
            raise ValueError(f"{n} must be float32 [num_kv_heads]")


def paged_kv_write_fp8(key, value, key_cache, value_cache, slot_mapping, k_scale, v_scale) -> None:
    """Quantise token i's K/V rows ``key[i]``/``value[i]`` (f32/f16/bf16,
    [num_kv_heads, head_dim]) with the per-KV-head scales into the E4M3 pools
    at ``slot_mapping[i]``."""
    torch = _torch()
    lib = _load()
    for t, n in ((key, "key"), (value, "value"), (slot_mapping, "slot_mapping")):
        _gpu(t, n)
    _e4m3_cache(key_cache, "key_cache")
    _e4m3_cache(value_cache, "value_cache")
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    nb, bs, kvh, d = key_cache.shape
    tokens = key.shape[0]
    if tuple(key.shape) != (tokens, kvh, d) or value.shape != key.shape or key.dtype != value.dtype:
        raise ValueError("key/value must be [num_tokens, num_kv_heads, head_dim] of the pool, one dtype")
    if value_cache.shape != key_cache.shape or slot_mapping.shape != (tokens,):
        raise ValueError("inconsistent shapes")
    _scales(k_scale, v_scale, kvh)
    st = lib.paged_kv_write_fp8(key.data_ptr(), value.data_ptr(), key_cache.data_ptr(),
                                value_cache.data_ptr(), slot_mapping.data_ptr(), k_scale.data_ptr(),
                                v_scale.data_ptr(), tokens, kvh, d, bs, nb, _dtype_code(key.dtype),
                                _stream_handle(key.device))
    if st != 0:
        raise PagedKVError(st, "paged_kv_write_fp8")


def paged_decode_attention_fp8(query, key_cache, value_cache, k_scale, v_scale, block_tables,
                               context_lens, block_size: int, scale: float, *,
                               max_context_len: int, partition_size: int = 0, out=None,
                               out_dtype=None, workspace=None):
    """``paged_decode_attention`` over E4M3 pools with per-KV-head scales;
    ``query`` is f16 or bf16 and sets the output type (or ``out_dtype``
    float32)."""
    torch = _torch()
    lib = _load()
    for t, n in ((query, "query"), (block_tables, "block_tables"), (context_lens, "context_lens")):
        _gpu(t, n)
    _e4m3_cache(key_cache, "key_cache")
    _e4m3_cache(value_cache, "value_cache")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    nb, bs, kvh, d = key_cache.shape
    if bs != block_size:
        raise ValueError("block_size does not match key_cache.shape[1]")
    b, h, dq = query.shape
    if dq != d or value_cache.shape != key_cache.shape:
        raise ValueError("inconsistent shapes")
    if block_tables.dim() != 2 or block_tables.shape[0] != b or tuple(context_lens.shape) != (b,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], context_lens [num_seqs]")
    _scales(k_scale, v_scale, kvh)
    dt = _dtype_code(query.dtype)
    odt = query.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((b, h, d), dtype=odt, device=query.device)
    else:
        _gpu(out, "out")
        if tuple(out.shape) != (b, h, d):
            raise ValueError("out must be [num_seqs, num_heads, head_dim]")
        odt = out.dtype
    need = paged_decode_workspace_size(b, h, d, int(max_context_len), int(partition_size))
    ws_ptr, ws_bytes = _workspace(need, workspace, query.device)
    st = lib.paged_decode_attention_fp8(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        k_scale.data_ptr(), v_scale.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(),
        b, h, kvh, d, bs, block_tables.shape[1], nb, int(max_context_len), float(scale),
        int(partition_size), dt, _dtype_code(odt), ws_ptr, ws_bytes, _stream_handle(query.device))
    if st != 0:
        raise PagedKVError(st, "paged_decode_attention_fp8")
    return out


def paged_prefill_attention(query, key_cache, value_cache, block_tables, context_lens,
                            query_start_loc, block_size: int, scale: float, *,
                            max_context_len: int, out=None, out_dtype=None):
    """Causal multi-token attention over the paged pools: ``query``
    [total_queries, num_heads, head_dim] packs each sequence's new queries
    (``query_start_loc`` int32 [num_seqs + 1]), the last positions of its
    ``context_lens`` history, whose K/V are already in the pools."""
    torch = _torch()
    lib = _load()
    for t, n in ((query, "query"), (key_cache, "key_cache"), (value_cache, "value_cache"),
                 (block_tables, "block_tables"), (context_lens, "context_lens"),
                 (query_start_loc, "query_start_loc")):
        _gpu(t, n)
    if (block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32
            or query_start_loc.dtype != torch.int32):
        raise TypeError("block_tables, context_lens and query_start_loc must be int32")
    nb, bs, kvh, d = key_cache.shape
    if bs != block_size:
        raise ValueError("block_size does not match key_cache.shape[1]")
    tq, h, dq = query.shape
    b = context_lens.shape[0]
    if dq != d or value_cache.shape != key_cache.shape:
        raise ValueError("inconsistent shapes")
    if block_tables.dim() != 2 or block_tables.shape[0] != b or tuple(query_start_loc.shape) != (b + 1,):
        raise ValueError("block_tables must be [num_seqs, max_blocks], query_start_loc [num_seqs + 1]")
    if not (query.dtype == key_cache.dtype == value_cache.dtype):
        raise TypeError("query and caches must share one dtype")
    dt = _dtype_code(query.dtype)
    odt = query.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((tq, h, d), dtype=odt, device=query.device)
    else:
        _gpu(out, "out")
        if tuple(out.shape) != (tq, h, d):
            raise ValueError("out must be [total_queries, num_heads, head_dim]")
        odt = out.dtype
    st = lib.paged_prefill_attention(
        out.data_ptr(), query.data_ptr(), key_cache.data_ptr(), value_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), query_start_loc.data_ptr(), b, tq, h, kvh,
        d, bs, block_tables.shape[1], nb, int(max_context_len), float(scale), dt, _dtype_code(odt),
        _stream_handle(query.device))
    if st != 0:
        raise PagedKVError(st, "paged_prefill_attention")
    return out
