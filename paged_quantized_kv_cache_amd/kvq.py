"""Thin ctypes binding of libkvq.so (C ABI in include/kvq.h).

Argument marshalling only: shapes are read off torch tensors, pointers and the
current HIP stream are passed through, status codes become exceptions.  Every
step of the computation runs in the library's HIP kernels; there is no CPU or
PyTorch fallback -- if ``libkvq.so`` is missing, every call raises.

Pool tensors (per layer) have shape [num_blocks][Hkv][block_size][head_dim]
with element int8 (INT8), uint8 (FP8 E4M3 bytes) or float16 (FP16); the
element order inside each (block, head) tile is the library's K / V tile
layout (include/kvq.h), not row-major.  INT8 scales
[num_blocks][Hkv][block_size][head_dim/G] fp32; FP8 scales [Hkv] fp32.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_FP16, KVQ_INT8, KVQ_FP8_E4M3, KVQ_FP8_E5M2, KVQ_INT4 = 0, 1, 2, 3, 4
# kvq_paged_prefill split modes
PREFILL_SPLIT_MODES = {"auto": 0, "walk": 1, "split": 2}
FORMATS = {"fp16": KVQ_FP16, "int8": KVQ_INT8, "fp8": KVQ_FP8_E4M3, "e5m2": KVQ_FP8_E5M2,
           "int4": KVQ_INT4}
# INT8 pools hold excess-128 bytes (code + 128), FP8 pools E4M3 / E5M2 bytes,
# INT4 pools two excess-8 nibbles per byte (a pool's last axis is head_dim / 2).
POOL_DTYPES = {"fp16": torch.float16, "int8": torch.uint8, "fp8": torch.uint8,
               "e5m2": torch.uint8, "int4": torch.uint8}


def scale_mode(fmt: str, group_size: int) -> str:
    """'group' (per token-group scales written by the cache write),
    'head' (static per KV head), 'channel' (static per KV head and channel)
    or 'none'."""
    if fmt == "fp16":
        return "none"
    if group_size > 0:
        return "group"
    return "channel" if fmt == "int8" else "head"


STATUS = {0: "KVQ_OK", -1: "KVQ_ERR_INVALID_ARG", -2: "KVQ_ERR_UNSUPPORTED",
          -3: "KVQ_ERR_WORKSPACE", -4: "KVQ_ERR_HIP"}
EXPORTS = ("kvq_status_string", "kvq_version", "kvq_cache_write",
           "kvq_paged_decode", "kvq_decode_workspace_size", "kvq_copy_blocks",
           "kvq_swap_block_bytes", "kvq_swap_out", "kvq_swap_in", "kvq_paged_prefill",
           "kvq_prefill_workspace_size", "kvq_cache_write_heads", "kvq_paged_decode_heads",
           "kvq_paged_decode_noalloc")


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (what, STATUS.get(status, status),
                                          _status_string(status)))


_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """Load libkvq.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    "libkvq.so is missing (%s); build it with "
                    "`python -c 'import __graft_entry__ as g; g.build()'`" % LIB_PATH)
            L = ctypes.CDLL(LIB_PATH)
            P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
            L.kvq_status_string.restype = ctypes.c_char_p
            L.kvq_status_string.argtypes = [i32]
            L.kvq_version.restype = i32
            L.kvq_version.argtypes = []
            L.kvq_cache_write.restype = i32
            L.kvq_cache_write.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32,
                                          i32, P, P, P, P, P]
            L.kvq_paged_decode.restype = i32
            L.kvq_paged_decode.argtypes = [P, P, P, P, P, P, i32, P, i32, i32,
                                           i32, i32, i32, i32, i32, i32, i32,
                                           ctypes.c_float, i32, P, P,
                                           ctypes.c_size_t, P]
            L.kvq_paged_decode_noalloc.restype = i32
            L.kvq_paged_decode_noalloc.argtypes = [P, P, P, P, P, P, i32, P, i32, i32,
                                                   i32, i32, i32, i32, i32, i32, i32,
                                                   ctypes.c_float, i32, P, P]
            L.kvq_cache_write_heads.restype = i32
            L.kvq_cache_write_heads.argtypes = [P, P, P, i32, i32, P, i32, i32, i32, i32,
                                                i32, i32, P, P, P, P, P]
            L.kvq_paged_decode_heads.restype = i32
            L.kvq_paged_decode_heads.argtypes = [P, P, P, P, P, P, i32, P, i32, i32, i32,
                                                 i32, P, i32, i32, i32, i32, i32, i32,
                                                 ctypes.c_float, i32, P, P, ctypes.c_size_t,
                                                 P]
            L.kvq_paged_prefill.restype = i32
            L.kvq_paged_prefill.argtypes = [P, P, i32, P, P, P, P, P, i32, P, i32, i32,
                                            i32, i32, i32, i32, i32, i32, i32,
                                            ctypes.c_float, i32, P, P, ctypes.c_size_t, P]
            L.kvq_prefill_workspace_size.restype = ctypes.c_size_t
            L.kvq_prefill_workspace_size.argtypes = [i32] * 8
            L.kvq_decode_workspace_size.restype = ctypes.c_size_t
            L.kvq_decode_workspace_size.argtypes = [i32] * 7
            L.kvq_copy_blocks.restype = i32
            L.kvq_copy_blocks.argtypes = [P, i32, i32, i32, i32, i32, i32, i32,
                                          P, P, P, P, P]
            L.kvq_swap_block_bytes.restype = ctypes.c_size_t
            L.kvq_swap_block_bytes.argtypes = [i32] * 5
            L.kvq_swap_out.restype = i32
            L.kvq_swap_out.argtypes = [P, i32, i32, i32, i32, i32, i32, i32,
                                       P, P, P, P, P, i64, P]
            L.kvq_swap_in.restype = i32
            L.kvq_swap_in.argtypes = [P, i32, i32, i32, i32, i32, i32, i32,
                                      P, i64, P, P, P, P, P]
            _lib = L
    return _lib


def _status_string(status: int) -> str:
    try:
        return lib().kvq_status_string(status).decode()
    except Exception:  # pragma: no cover - only used for messages
        return "?"


def _check(status: int, what: str) -> None:
    if status != 0:
        raise KvqError(status, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _fmt(fmt) -> int:
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


# ------------------------------------------------------------------ pools
def alloc_pools(num_blocks: int, num_kv_heads: int, block_size: int,
                head_dim: int, fmt: str, group_size: int = 0, device="cuda"):
    """Allocate one layer's (k_pool, v_pool, k_scale, v_scale) with torch.

    Per-group scales: [num_blocks][Hkv][block_size][head_dim/G] (written by
    the cache write).  Static scales are returned as ones, for the caller to
    fill: [Hkv] per head (FP8), [Hkv][head_dim] per channel (INT8).  FP16 has
    no scales (None)."""
    dt = POOL_DTYPES[fmt]
    last = head_dim // 2 if fmt == "int4" else head_dim
    kp = torch.empty((num_blocks, num_kv_heads, block_size, last), dtype=dt, device=device)
    vp = torch.empty((num_blocks, num_kv_heads, block_size, last), dtype=dt, device=device)
    mode = scale_mode(fmt, group_size)
    if mode == "group":
        ng = head_dim // group_size
        ks = torch.empty((num_blocks, num_kv_heads, block_size, ng), dtype=torch.float32, device=device)
        vs = torch.empty_like(ks)
    elif mode == "head":
        ks = torch.ones(num_kv_heads, dtype=torch.float32, device=device)
        vs = torch.ones_like(ks)
    elif mode == "channel":
        ks = torch.ones((num_kv_heads, head_dim), dtype=torch.float32, device=device)
        vs = torch.ones_like(ks)
    else:
        ks = vs = None
    return kp, vp, ks, vs


def _pool_geometry(k_pool: torch.Tensor, fmt: str):
    num_blocks, hkv, bs, d = k_pool.shape
    if fmt == "int4":
        d *= 2
    if k_pool.dtype != POOL_DTYPES[fmt]:
        raise TypeError("pool dtype %s does not match format %s" % (k_pool.dtype, fmt))
    return num_blocks, hkv, bs, d


# ------------------------------------------------------------------ calls
def kvq_cache_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                    k_pool: torch.Tensor, v_pool: torch.Tensor,
                    k_scale: Optional[torch.Tensor], v_scale: Optional[torch.Tensor],
                    fmt: str, group_size: int = 0, stream=None) -> None:
    """Quantize k, v ``[T][Hkv][D]`` fp16 into their slots (see kvq.h)."""
    num_blocks, hkv, bs, d = _pool_geometry(k_pool, fmt)
    T = k.shape[0]
    if k.dtype != torch.float16 or v.dtype != torch.float16:
        raise TypeError("k and v must be float16")
    if k.shape != (T, hkv, d) or v.shape != k.shape:
        raise ValueError("k/v shape %s does not match the pool" % (tuple(k.shape),))
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != T:
        raise ValueError("slot_mapping must be int64 [T]")
    for t in (k, v, slot_mapping, k_pool, v_pool):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    st = lib().kvq_cache_write(_ptr(k), _ptr(v), _ptr(slot_mapping), T, hkv, d, bs,
                               num_blocks, _fmt(fmt), group_size, _ptr(k_pool),
                               _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
                               _stream(stream))
    _check(st, "kvq_cache_write")


def kvq_decode_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                              head_dim: int, block_size: int, max_context_len: int,
                              split_tokens: int = 0) -> int:
    n = int(lib().kvq_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads,
                                            head_dim, block_size, max_context_len,
                                            split_tokens))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid workspace arguments")
    return n


def _split_mode(mode) -> int:
    return PREFILL_SPLIT_MODES[mode] if isinstance(mode, str) else int(mode)


def kvq_prefill_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int,
                               head_dim: int, block_size: int, max_context_len: int,
                               max_query_len: int, split_mode="auto") -> int:
    n = int(lib().kvq_prefill_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                             block_size, max_context_len, max_query_len,
                                             _split_mode(split_mode)))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid workspace arguments")
    return n


BLOCK_ID_MASK = 0x3FFFFFFF      # table entry bits 0..29: physical block id
SHARED_HINT_BIT = 1 << 30       # bit 30: shared-block cache hint


def _validate_wanted(validate: Optional[bool]) -> bool:
    if validate is not None:
        return validate
    return os.environ.get("KVQ_VALIDATE", "0") not in ("", "0")


def validate_decode_inputs(block_tables: torch.Tensor, context_lens: torch.Tensor,
                           max_context_len: int, block_size: int, num_blocks: int,
                           query_start: Optional[torch.Tensor] = None) -> None:
    """Check the device metadata of a decode or prefill call on host copies
    (synchronizes; a debugging aid, off by default).  The kernels never read
    outside the pools whatever these hold -- block ids are clamped into the
    pool and lengths into max_context_len -- but wrong metadata gives wrong
    attention; this names the first offending sequence instead.

    Checks: every context length in [1, max_context_len]; every table entry
    a sequence uses (its first ceil(ctx / block_size)) has bit 31 clear and a
    block id below num_blocks (bit 30, the shared-block hint, is allowed);
    max_context_len fits the table width; chunk offsets (prefill) are
    non-decreasing with each chunk no longer than its context."""
    bt = block_tables.detach().to("cpu", torch.int64)
    cl = context_lens.detach().to("cpu", torch.int64).reshape(-1)
    B, width = bt.shape
    if cl.numel() != B:
        raise ValueError("context_lens has %d entries for %d table rows" % (cl.numel(), B))
    if max_context_len > width * block_size:
        raise ValueError("max_context_len %d exceeds the table width (%d blocks of %d)"
                         % (max_context_len, width, block_size))
    bad = ((cl < 1) | (cl > max_context_len)).nonzero()
    if bad.numel():
        b = int(bad[0])
        raise ValueError("sequence %d: context length %d outside [1, %d]"
                         % (b, int(cl[b]), max_context_len))
    used = (torch.arange(width)[None, :] * block_size) < cl[:, None]
    neg = (bt < 0) & used           # int32 entries with bit 31 set
    ids = bt & BLOCK_ID_MASK
    over = (ids >= num_blocks) & used
    for what, m in (("has bit 31 set", neg), ("names a block outside the pool", over)):
        hit = m.nonzero()
        if hit.numel():
            b, i = int(hit[0, 0]), int(hit[0, 1])
            raise ValueError("sequence %d: table entry %d (%#x) %s (%d blocks)"
                             % (b, i, int(bt[b, i]) & 0xFFFFFFFF, what, num_blocks))
    if query_start is not None:
        qs = query_start.detach().to("cpu", torch.int64).reshape(-1)
        if qs.numel() != B + 1:
            raise ValueError("query_start has %d entries for %d sequences" % (qs.numel(), B))
        n = qs[1:] - qs[:-1]
        bad = ((n < 0) | (n > cl)).nonzero()
        if bad.numel():
            b = int(bad[0])
            raise ValueError("sequence %d: chunk of %d tokens for a context of %d"
                             % (b, int(n[b]), int(cl[b])))


def alloc_workspace(nbytes: int, device="cuda") -> Optional[torch.Tensor]:
    """Decode workspace (contents on entry do not matter)."""
    if nbytes == 0:
        return None
    return torch.empty((nbytes + 15) // 16 * 16, dtype=torch.uint8, device=device)


def kvq_paged_decode(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                     k_scale: Optional[torch.Tensor], v_scale: Optional[torch.Tensor],
                     block_tables: torch.Tensor, context_lens: torch.Tensor,
                     max_context_len: int, fmt: str, group_size: int = 0,
                     softmax_scale: float = 0.0, split_tokens: int = 0,
                     out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None,
                     stream=None, validate: Optional[bool] = None) -> torch.Tensor:
    """One decode step of paged attention (see kvq.h).  Returns ``out``.
    ``validate`` (default: the KVQ_VALIDATE environment variable) checks the
    tables and lengths on the host first (validate_decode_inputs)."""
    num_blocks, hkv, bs, d = _pool_geometry(k_pool, fmt)
    B, hq, dq = q.shape
    if q.dtype != torch.float16 or dq != d:
        raise ValueError("q must be float16 [B][Hq][%d]" % d)
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B][max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.numel() != B:
        raise ValueError("context_lens must be int32 [B]")
    if _validate_wanted(validate) and B > 0:
        validate_decode_inputs(block_tables, context_lens, max_context_len, bs, num_blocks)
    if out is None:
        out = torch.empty_like(q)
    for t in (q, k_pool, v_pool, block_tables, context_lens, out):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    ws_need = kvq_decode_workspace_size(B, hq, hkv, d, bs, max(max_context_len, 1),
                                        split_tokens) if B > 0 else 0
    if workspace is None and ws_need:
        workspace = alloc_workspace(ws_need, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().kvq_paged_decode(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
                                _ptr(v_scale), _ptr(block_tables), block_tables.shape[1],
                                _ptr(context_lens), max_context_len, B, hq, hkv, d, bs,
                                num_blocks, _fmt(fmt), group_size, softmax_scale,
                                split_tokens, _ptr(out), _ptr(workspace), ws_bytes,
                                _stream(stream))
    _check(st, "kvq_paged_decode")
    return out


def kvq_paged_decode_noalloc(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                             k_scale: Optional[torch.Tensor], v_scale: Optional[torch.Tensor],
                             block_tables: torch.Tensor, context_lens: torch.Tensor,
                             max_context_len: int, fmt: str, out: torch.Tensor,
                             group_size: int = 0, softmax_scale: float = 0.0,
                             split_tokens: int = 0, stream=None) -> torch.Tensor:
    """kvq_paged_decode without a workspace: the library's static device
    scratch holds the plan and partials (see kvq.h; calls on one GPU must
    not overlap).  ``out`` is required, so nothing is allocated here."""
    num_blocks, hkv, bs, d = _pool_geometry(k_pool, fmt)
    B, hq, dq = q.shape
    if q.dtype != torch.float16 or dq != d:
        raise ValueError("q must be float16 [B][Hq][%d]" % d)
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B][max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.numel() != B:
        raise ValueError("context_lens must be int32 [B]")
    if out.shape != q.shape or out.dtype != torch.float16:
        raise ValueError("out must be float16 shaped like q")
    for t in (q, k_pool, v_pool, block_tables, context_lens, out):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    st = lib().kvq_paged_decode_noalloc(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
                                        _ptr(v_scale), _ptr(block_tables),
                                        block_tables.shape[1], _ptr(context_lens),
                                        max_context_len, B, hq, hkv, d, bs, num_blocks,
                                        _fmt(fmt), group_size, softmax_scale, split_tokens,
                                        _ptr(out), _stream(stream))
    _check(st, "kvq_paged_decode_noalloc")
    return out


def kvq_copy_blocks(block_pairs: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                    k_scale: Optional[torch.Tensor], v_scale: Optional[torch.Tensor],
                    fmt: str, group_size: int = 0, stream=None) -> None:
    """Copy whole blocks src -> dst (block_pairs int32 [n][2] on the device)."""
    num_blocks, hkv, bs, d = _pool_geometry(k_pool, fmt)
    if block_pairs.dtype != torch.int32 or (block_pairs.numel() and block_pairs.shape[-1] != 2):
        raise ValueError("block_pairs must be int32 [n][2]")
    n = block_pairs.numel() // 2
    scale_ok = scale_mode(fmt, group_size) == "group"
    st = lib().kvq_copy_blocks(_ptr(block_pairs), n, hkv, d, bs, num_blocks, _fmt(fmt),
                               group_size, _ptr(k_pool), _ptr(v_pool),
                               _ptr(k_scale) if scale_ok else None,
                               _ptr(v_scale) if scale_ok else None, _stream(stream))
    _check(st, "kvq_copy_blocks")


# ------------------------------------------------------------------ swap
def kvq_swap_block_bytes(num_kv_heads: int, head_dim: int, block_size: int, fmt: str,
                         group_size: int = 0) -> int:
    """Bytes of one swap slot (one block's codes and per-group scales)."""
    n = lib().kvq_swap_block_bytes(num_kv_heads, head_dim, block_size, _fmt(fmt),
                                   group_size)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("unsupported swap arguments")
    return int(n)


def _swap_args(pairs, k_pool, fmt, group_size, buf):
    num_blocks, hkv, bs, d = _pool_geometry(k_pool, fmt)
    if pairs.dtype != torch.int32 or (pairs.numel() and pairs.shape[-1] != 2):
        raise ValueError("block_slot_pairs must be int32 [n][2]")
    if buf.dtype != torch.uint8 or not buf.is_contiguous():
        raise ValueError("swap buffer must be a contiguous uint8 tensor")
    slot = kvq_swap_block_bytes(hkv, d, bs, fmt, group_size)
    return num_blocks, hkv, bs, d, pairs.numel() // 2, buf.numel() // slot


def kvq_swap_out(block_slot_pairs: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                 k_scale: Optional[torch.Tensor], v_scale: Optional[torch.Tensor],
                 fmt: str, group_size: int, dst: torch.Tensor, stream=None) -> None:
    """Copy pool blocks into swap slots of ``dst`` (device or pinned host
    uint8 buffer of whole slots).  ``block_slot_pairs``: int32 [n][2]."""
    nb, hkv, bs, d, n, slots = _swap_args(block_slot_pairs, k_pool, fmt, group_size, dst)
    grp = scale_mode(fmt, group_size) == "group"
    st = lib().kvq_swap_out(_ptr(block_slot_pairs), n, hkv, d, bs, nb, _fmt(fmt), group_size,
                            _ptr(k_pool), _ptr(v_pool), _ptr(k_scale) if grp else None,
                            _ptr(v_scale) if grp else None, _ptr(dst), slots, _stream(stream))
    _check(st, "kvq_swap_out")


def kvq_swap_in(block_slot_pairs: torch.Tensor, src: torch.Tensor, k_pool: torch.Tensor,
                v_pool: torch.Tensor, k_scale: Optional[torch.Tensor],
                v_scale: Optional[torch.Tensor], fmt: str, group_size: int,
                stream=None) -> None:
    """Copy swap slots of ``src`` into pool blocks."""
    nb, hkv, bs, d, n, slots = _swap_args(block_slot_pairs, k_pool, fmt, group_size, src)
    grp = scale_mode(fmt, group_size) == "group"
    st = lib().kvq_swap_in(_ptr(block_slot_pairs), n, hkv, d, bs, nb, _fmt(fmt), group_size,
                           _ptr(src), slots, _ptr(k_pool), _ptr(v_pool),
                           _ptr(k_scale) if grp else None, _ptr(v_scale) if grp else None,
                           _stream(stream))
    _check(st, "kvq_swap_in")


# ------------------------------------------------------------------ prefill
def kvq_paged_prefill(q: torch.Tensor, query_start: torch.Tensor, max_query_len: int,
                      k_pool: torch.Tensor, v_pool: torch.Tensor,
                      k_scale: Optional[torch.Tensor], v_scale: Optional[torch.Tensor],
                      block_tables: torch.Tensor, context_lens: torch.Tensor,
                      max_context_len: int, fmt: str, group_size: int = 0,
                      softmax_scale: float = 0.0, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None,
                      stream=None, validate: Optional[bool] = None,
                      split_mode="auto") -> torch.Tensor:
    """Causal attention of each sequence's chunk (its last n_b tokens, already
    in the pool) over its cached tokens.  q: fp16 [sum n][Hq][D];
    query_start: int32 [B + 1] on the device.  ``split_mode``: "auto",
    "walk" or "split" (see kvq.h); ``workspace`` (allocated here when None)
    is used by the split cut only."""
    num_blocks, hkv, bs, d = _pool_geometry(k_pool, fmt)
    T, hq, dq = q.shape
    B = context_lens.numel()
    if dq != d or q.dtype != torch.float16 or not q.is_contiguous():
        raise ValueError("q must be contiguous fp16 [tokens][Hq][head_dim]")
    if query_start.dtype != torch.int32 or query_start.numel() != B + 1:
        raise ValueError("query_start must be int32 [B + 1]")
    if _validate_wanted(validate) and B > 0:
        validate_decode_inputs(block_tables, context_lens, max_context_len, bs, num_blocks,
                               query_start)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None and B > 0 and max_query_len > 0:
        workspace = alloc_workspace(kvq_prefill_workspace_size(
            B, hq, hkv, d, bs, max_context_len, max_query_len, split_mode), q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().kvq_paged_prefill(_ptr(q), _ptr(query_start), max_query_len, _ptr(k_pool),
                                 _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
                                 _ptr(block_tables), block_tables.shape[1],
                                 _ptr(context_lens), max_context_len, B, hq, hkv, d, bs,
                                 num_blocks, _fmt(fmt), group_size, softmax_scale,
                                 _split_mode(split_mode), _ptr(out), _ptr(workspace), ws_bytes,
                                 _stream(stream))
    _check(st, "kvq_paged_prefill")
    return out


# ------------------------------------------------------------------ head subsets
def kvq_cache_write_heads(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                          kv_head_ids: torch.Tensor, k_pool: torch.Tensor,
                          v_pool: torch.Tensor, k_scale: Optional[torch.Tensor],
                          v_scale: Optional[torch.Tensor], fmt: str, group_size: int = 0,
                          stream=None) -> None:
    """kvq_cache_write into a pool that holds the model's KV heads
    ``kv_head_ids`` (int32 on the device); k, v carry all the model's heads."""
    num_blocks, hkv, bs, d = _pool_geometry(k_pool, fmt)
    T, hsrc, dk = k.shape
    if kv_head_ids.dtype != torch.int32 or kv_head_ids.numel() != hkv:
        raise ValueError("kv_head_ids must be int32 [pool heads]")
    st = lib().kvq_cache_write_heads(_ptr(k), _ptr(v), _ptr(slot_mapping), T, hsrc,
                                     _ptr(kv_head_ids), hkv, d, bs, num_blocks, _fmt(fmt),
                                     group_size, _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
                                     _ptr(v_scale), _stream(stream))
    _check(st, "kvq_cache_write_heads")


def kvq_paged_decode_heads(q: torch.Tensor, num_kv_heads: int, kv_head_ids: torch.Tensor,
                           k_pool: torch.Tensor, v_pool: torch.Tensor,
                           k_scale: Optional[torch.Tensor], v_scale: Optional[torch.Tensor],
                           block_tables: torch.Tensor, context_lens: torch.Tensor,
                           max_context_len: int, fmt: str, group_size: int = 0,
                           out: Optional[torch.Tensor] = None, workspace=None,
                           softmax_scale: float = 0.0, split_tokens: int = 0,
                           stream=None, validate: Optional[bool] = None) -> torch.Tensor:
    """kvq_paged_decode over a pool holding the model KV heads
    ``kv_head_ids``; writes only their query heads' rows of ``out``."""
    num_blocks, hkv, bs, d = _pool_geometry(k_pool, fmt)
    B, hq, _ = q.shape
    if _validate_wanted(validate) and B > 0:
        validate_decode_inputs(block_tables, context_lens, max_context_len, bs, num_blocks)
    if out is None:
        out = torch.zeros_like(q)
    if workspace is None:
        workspace = alloc_workspace(kvq_decode_workspace_size(
            B, hkv * (hq // num_kv_heads), hkv, d, bs, max_context_len, split_tokens),
            device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    st = lib().kvq_paged_decode_heads(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
                                      _ptr(v_scale), _ptr(block_tables), block_tables.shape[1],
                                      _ptr(context_lens), max_context_len, B, hq,
                                      num_kv_heads, _ptr(kv_head_ids), hkv, d, bs, num_blocks,
                                      _fmt(fmt), group_size, softmax_scale, split_tokens,
                                      _ptr(out), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "kvq_paged_decode_heads")
    return out
