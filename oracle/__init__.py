"""CPU oracle for the paged, quantized KV-cache decode path.

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product path
(``paged_quantized_kv_cache_amd``) never does.

The arithmetic lives in plain C (``kvq_oracle.c``); this module only compiles
it with gcc (no fast-math, no FP contraction) and marshals numpy arrays.  It
shares no code with the HIP library.

Sources (web pages, cited by title and section):
  * "KV Cache优化实战：大模型推理显存占用与加速方案详解" (0539edu.com):
    s1.1 decode with a KV cache, s1.2 byte formula, s2.1 GQA, s2.3 INT8
    absmax / per-channel / per-group / FP8 quantization, s3.1 memory
    estimator, s3.3 per_channel / per_group / per_token granularity with
    group 128 or 64.
  * xpshop.cn article 312, s3: FP8 KV cache as ``fp8_e5m2``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    stale = (not os.path.exists(_LIB_PATH)
             or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC))
    if force or stale:
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _L():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            P = ctypes.c_void_p
            i64, i32 = ctypes.c_int64, ctypes.c_int
            lib.orc_f16_to_f64.restype = ctypes.c_double
            lib.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
            lib.orc_f16_to_f64_array.argtypes = [P, i64, P]
            lib.orc_int8_quantize_rows.restype = i32
            lib.orc_int8_quantize_rows.argtypes = [P, i64, i32, i32, P, P]
            lib.orc_int8_dequantize_rows.argtypes = [P, P, i64, i32, i32, P]
            lib.orc_int4_quantize_rows.restype = i32
            lib.orc_int4_quantize_rows.argtypes = [P, i64, i32, i32, P, P]
            lib.orc_e4m3_decode.restype = ctypes.c_double
            lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
            lib.orc_e4m3_encode.restype = ctypes.c_uint8
            lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
            lib.orc_fp8_quantize_rows.restype = i32
            lib.orc_fp8_quantize_rows.argtypes = [P, i64, i32, i32, P, P]
            lib.orc_fp8_dequantize_rows.argtypes = [P, i64, i32, i32, P, P]
            lib.orc_e5m2_decode.restype = ctypes.c_double
            lib.orc_e5m2_decode.argtypes = [ctypes.c_uint8]
            lib.orc_e5m2_encode.restype = ctypes.c_uint8
            lib.orc_e5m2_encode.argtypes = [ctypes.c_float]
            lib.orc_fp8_quantize_rows_fmt.restype = i32
            lib.orc_fp8_quantize_rows_fmt.argtypes = [P, i64, i32, i32, P, i32, P]
            lib.orc_fp8_dequantize_rows_fmt.argtypes = [P, i64, i32, i32, P, i32, P]
            lib.orc_fp8_quantize_groups.restype = i32
            lib.orc_fp8_quantize_groups.argtypes = [P, i64, i32, i32, i32, P, P]
            lib.orc_fp8_dequantize_groups.argtypes = [P, P, i64, i32, i32, i32, P]
            lib.orc_int8_quantize_channels.restype = i32
            lib.orc_int8_quantize_channels.argtypes = [P, i64, i32, i32, P, P]
            lib.orc_int8_dequantize_channels.argtypes = [P, i64, i32, i32, P, P]
            lib.orc_prefill_attention.restype = i32
            lib.orc_prefill_attention.argtypes = [P, P, P, P, P, i32, i32, i32,
                                                  i32, ctypes.c_double, P]
            lib.orc_decode_attention.restype = i32
            lib.orc_decode_attention.argtypes = [P, P, P, P, i32, i32, i32,
                                                 i32, ctypes.c_double, P]
            lib.orc_kv_cache_bytes.restype = i64
            lib.orc_kv_cache_bytes.argtypes = [i64] * 6
            lib.orc_kv_cache_bytes_int8_group.restype = i64
            lib.orc_kv_cache_bytes_int8_group.argtypes = [i64] * 6
            lib.orc_num_threads.restype = i32
            lib.orc_set_num_threads.argtypes = [i32]
            _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _f16_bits(x) -> np.ndarray:
    """Accept fp16 ndarray / torch tensor / uint16 bits; return uint16 bits."""
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().cpu().contiguous().numpy()
    x = np.ascontiguousarray(x)
    if x.dtype == np.float16:
        return x.view(np.uint16)
    if x.dtype == np.uint16:
        return x
    raise TypeError("expected fp16 data, got %s" % x.dtype)


def num_threads() -> int:
    return int(_L().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from now on."""
    _L().orc_set_num_threads(int(n))


# ---------------------------------------------------------------- fp16
def f16_to_f64(x) -> np.ndarray:
    bits = _f16_bits(x)
    out = np.empty(bits.shape, np.float64)
    _L().orc_f16_to_f64_array(_ptr(bits), bits.size, _ptr(out))
    return out


# ---------------------------------------------------------------- INT8
def int8_quantize(x, group_size: int):
    """Per-group absmax INT8 along the last axis.

    Returns ``(codes int8 same shape, scales float32 [..., d/G])``."""
    bits = _f16_bits(x)
    d = bits.shape[-1]
    if d % group_size:
        raise ValueError("group_size must divide the last dimension")
    rows = bits.size // d
    codes = np.empty(bits.shape, np.int8)
    scales = np.empty(bits.shape[:-1] + (d // group_size,), np.float32)
    rc = _L().orc_int8_quantize_rows(_ptr(bits), rows, d, group_size,
                                     _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError("oracle: non-finite input or bad group size (%d)" % rc)
    return codes, scales


def int4_quantize(x, group_size: int):
    """Per-group absmax INT4 along the last axis (codes in [-7, 7]).

    Returns ``(codes int8 same shape, scales float32 [..., d/G])``."""
    bits = _f16_bits(x)
    d = bits.shape[-1]
    if d % group_size:
        raise ValueError("group_size must divide the last dimension")
    rows = bits.size // d
    codes = np.empty(bits.shape, np.int8)
    scales = np.empty(bits.shape[:-1] + (d // group_size,), np.float32)
    rc = _L().orc_int4_quantize_rows(_ptr(bits), rows, d, group_size,
                                     _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError("oracle: non-finite input or bad group size (%d)" % rc)
    return codes, scales


def int8_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.int8)
    scales = np.ascontiguousarray(scales, np.float32)
    d = codes.shape[-1]
    G = d // scales.shape[-1]
    out = np.empty(codes.shape, np.float64)
    _L().orc_int8_dequantize_rows(_ptr(codes), _ptr(scales), codes.size // d,
                                  d, G, _ptr(out))
    return out


# ---------------------------------------------------------------- FP8 E4M3
def e4m3_decode(codes) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    lib = _L()
    return np.array([lib.orc_e4m3_decode(int(c)) for c in codes.ravel()],
                    np.float64).reshape(codes.shape)


def e4m3_encode(y) -> np.ndarray:
    y = np.ascontiguousarray(y, np.float32)
    lib = _L()
    return np.array([lib.orc_e4m3_encode(float(v)) for v in y.ravel()],
                    np.uint8).reshape(y.shape)


FP8_FORMATS = {"e4m3": 0, "e5m2": 1}


def e5m2_decode(codes) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    lib = _L()
    return np.array([lib.orc_e5m2_decode(int(c)) for c in codes.ravel()],
                    np.float64).reshape(codes.shape)


def e5m2_encode(y) -> np.ndarray:
    y = np.ascontiguousarray(y, np.float32)
    lib = _L()
    return np.array([lib.orc_e5m2_encode(float(v)) for v in y.ravel()],
                    np.uint8).reshape(y.shape)


def fp8_quantize(x, scale, fmt: str = "e4m3") -> np.ndarray:
    """x: [T][Hkv][d] fp16; scale: [Hkv] fp32 (static per head).
    code = fp8(fl32(x / S[h]))."""
    bits = _f16_bits(x)
    T, Hkv, d = bits.shape
    S = np.ascontiguousarray(scale, np.float32)
    assert S.shape == (Hkv,)
    codes = np.empty(bits.shape, np.uint8)
    rc = _L().orc_fp8_quantize_rows_fmt(_ptr(bits), T, Hkv, d, _ptr(S),
                                        FP8_FORMATS[fmt], _ptr(codes))
    if rc != 0:
        raise ValueError("oracle: non-finite input")
    return codes


def fp8_dequantize(codes: np.ndarray, scale, fmt: str = "e4m3") -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    T, Hkv, d = codes.shape
    S = np.ascontiguousarray(scale, np.float32)
    out = np.empty(codes.shape, np.float64)
    _L().orc_fp8_dequantize_rows_fmt(_ptr(codes), T, Hkv, d, _ptr(S),
                                     FP8_FORMATS[fmt], _ptr(out))
    return out


def fp8_quantize_groups(x, group_size: int, fmt: str = "e4m3"):
    """Dynamic per-group FP8 along the last axis.

    Returns ``(codes uint8 same shape, scales float32 [..., d/G])``."""
    bits = _f16_bits(x)
    d = bits.shape[-1]
    if group_size <= 0 or d % group_size:
        raise ValueError("group_size must divide the last dimension")
    rows = bits.size // d
    codes = np.empty(bits.shape, np.uint8)
    scales = np.empty(bits.shape[:-1] + (d // group_size,), np.float32)
    rc = _L().orc_fp8_quantize_groups(_ptr(bits), rows, d, group_size,
                                      FP8_FORMATS[fmt], _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError("oracle: non-finite input or bad group size (%d)" % rc)
    return codes, scales


def fp8_dequantize_groups(codes: np.ndarray, scales: np.ndarray,
                          fmt: str = "e4m3") -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.float32)
    d = codes.shape[-1]
    G = d // scales.shape[-1]
    out = np.empty(codes.shape, np.float64)
    _L().orc_fp8_dequantize_groups(_ptr(codes), _ptr(scales), codes.size // d,
                                   d, G, FP8_FORMATS[fmt], _ptr(out))
    return out


def int8_quantize_channels(x, scale) -> np.ndarray:
    """x: [T][Hkv][d] fp16; scale: [Hkv][d] fp32 (static per channel)."""
    bits = _f16_bits(x)
    T, Hkv, d = bits.shape
    S = np.ascontiguousarray(scale, np.float32)
    assert S.shape == (Hkv, d)
    codes = np.empty(bits.shape, np.int8)
    rc = _L().orc_int8_quantize_channels(_ptr(bits), T, Hkv, d, _ptr(S), _ptr(codes))
    if rc != 0:
        raise ValueError("oracle: non-finite input")
    return codes


def int8_dequantize_channels(codes: np.ndarray, scale) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.int8)
    T, Hkv, d = codes.shape
    S = np.ascontiguousarray(scale, np.float32)
    out = np.empty(codes.shape, np.float64)
    _L().orc_int8_dequantize_channels(_ptr(codes), T, Hkv, d, _ptr(S), _ptr(out))
    return out


# ---------------------------------------------------------------- attention
def decode_attention(q, K: np.ndarray, V: np.ndarray, context_lens,
                     softmax_scale: float = 0.0) -> np.ndarray:
    """fp64 decode attention over contiguous K/V.

    q: [B][Hq][d] fp16; K, V: [sum ctx][Hkv][d] fp64 (sequences concatenated
    in batch order); context_lens: [B].  Returns [B][Hq][d] fp64."""
    qb = _f16_bits(q)
    B, Hq, d = qb.shape
    K = np.ascontiguousarray(K, np.float64)
    V = np.ascontiguousarray(V, np.float64)
    Hkv = K.shape[1]
    lens = np.asarray(context_lens, np.int64)
    cu = np.zeros(B + 1, np.int64)
    cu[1:] = np.cumsum(lens)
    assert K.shape == (cu[-1], Hkv, d) and V.shape == K.shape
    sm = float(softmax_scale) if softmax_scale else 1.0 / np.sqrt(d)
    out = np.empty((B, Hq, d), np.float64)
    rc = _L().orc_decode_attention(_ptr(qb), _ptr(K), _ptr(V), _ptr(cu), B, Hq,
                                   Hkv, d, sm, _ptr(out))
    if rc != 0:
        raise ValueError("oracle: invalid attention arguments (%d)" % rc)
    return out


def prefill_attention(q, K: np.ndarray, V: np.ndarray, chunk_lens, context_lens,
                      softmax_scale: float = 0.0) -> np.ndarray:
    """fp64 causal attention of chunk queries over contiguous K/V.

    q: [sum n][Hq][d] fp16 (chunks in batch order); K, V: [sum ctx][Hkv][d]
    fp64; sequence b's chunk is its last n_b tokens.  Returns [sum n][Hq][d]."""
    qb = _f16_bits(q)
    T, Hq, d = qb.shape
    K = np.ascontiguousarray(K, np.float64)
    V = np.ascontiguousarray(V, np.float64)
    Hkv = K.shape[1]
    n = np.asarray(chunk_lens, np.int64)
    c = np.asarray(context_lens, np.int64)
    B = n.size
    cu_q = np.zeros(B + 1, np.int64)
    cu_q[1:] = np.cumsum(n)
    cu_k = np.zeros(B + 1, np.int64)
    cu_k[1:] = np.cumsum(c)
    assert cu_q[-1] == T and K.shape == (cu_k[-1], Hkv, d) and V.shape == K.shape
    sm = float(softmax_scale) if softmax_scale else 1.0 / np.sqrt(d)
    out = np.empty((T, Hq, d), np.float64)
    rc = _L().orc_prefill_attention(_ptr(qb), _ptr(K), _ptr(V), _ptr(cu_q), _ptr(cu_k),
                                    B, Hq, Hkv, d, sm, _ptr(out))
    if rc != 0:
        raise ValueError("oracle: invalid prefill arguments (%d)" % rc)
    return out


# ---------------------------------------------------------------- bytes
def kv_cache_bytes(batch, seq_len, layers, kv_heads, head_dim, elem_bytes) -> int:
    return int(_L().orc_kv_cache_bytes(batch, seq_len, layers, kv_heads,
                                       head_dim, elem_bytes))


def kv_cache_bytes_int8_group(batch, seq_len, layers, kv_heads, head_dim,
                              group_size) -> int:
    return int(_L().orc_kv_cache_bytes_int8_group(batch, seq_len, layers,
                                                  kv_heads, head_dim, group_size))


# ---------------------------------------------------------------- pipeline
def quantize_kv(x, fmt: str, group_size: int = 0, scale=None):
    """Quantize contiguous K or V ``[T][Hkv][d]`` in the given format.

    Returns ``(codes, scales_or_None, dequantized fp64)``."""
    if fmt == "int8":
        codes, sc = int8_quantize(x, group_size)
        return codes, sc, int8_dequantize(codes, sc)
    if fmt in ("fp8", "e5m2"):
        f = "e5m2" if fmt == "e5m2" else "e4m3"
        codes = fp8_quantize(x, scale, f)
        return codes, None, fp8_dequantize(codes, scale, f)
    if fmt == "fp16":
        bits = _f16_bits(x)
        return bits.copy(), None, f16_to_f64(bits)
    raise ValueError(fmt)
