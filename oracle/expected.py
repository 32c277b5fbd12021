"""Expected results of one decode step, from the oracle alone.

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the
benchmark).  Works on contiguous, un-paged arrays: every sequence's cached
tokens are listed in logical order; paging never enters.

``"KV Cache优化实战"`` s1.1: the cache holds each token's K/V once it has been
computed; decode attends with the current query over all of them.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

from . import (decode_attention, prefill_attention, fp8_dequantize, fp8_dequantize_groups,
               fp8_quantize, fp8_quantize_groups, f16_to_f64, int4_quantize,
               int8_dequantize, int8_dequantize_channels, int8_quantize,
               int8_quantize_channels)


@dataclass
class Quantized:
    codes: np.ndarray            # [N][Hkv][D] int8 / uint8 / uint16 (fp16 bits)
    scales: Optional[np.ndarray]  # per-group formats: [N][Hkv][D/G] fp32
    deq: np.ndarray              # [N][Hkv][D] fp64


def quantize(x: np.ndarray, fmt: str, group_size: int = 0,
             static_scale: Optional[np.ndarray] = None) -> Quantized:
    """x: fp16 ``[N][Hkv][D]`` (numpy float16).

    fmt "int8": group_size > 0 per-group absmax; 0 per-channel with
    static_scale [Hkv][D].  fmt "fp8" (E4M3) / "e5m2": group_size 0 static
    per-head static_scale [Hkv]; > 0 dynamic per-group scales."""
    if fmt == "int4":
        c, s = int4_quantize(x, group_size)
        return Quantized(c, s, int8_dequantize(c, s))
    if fmt == "int8":
        if group_size == 0:
            c = int8_quantize_channels(x, static_scale)
            return Quantized(c, None, int8_dequantize_channels(c, static_scale))
        c, s = int8_quantize(x, group_size)
        return Quantized(c, s, int8_dequantize(c, s))
    if fmt in ("fp8", "e5m2"):
        f = "e5m2" if fmt == "e5m2" else "e4m3"
        if group_size:
            c, s = fp8_quantize_groups(x, group_size, f)
            return Quantized(c, s, fp8_dequantize_groups(c, s, f))
        c = fp8_quantize(x, static_scale, f)
        return Quantized(c, None, fp8_dequantize(c, static_scale, f))
    if fmt == "fp16":
        bits = np.ascontiguousarray(x).view(np.uint16)
        return Quantized(bits.copy(), None, f16_to_f64(bits))
    raise ValueError(fmt)


def attention(q: np.ndarray, kq: Quantized, vq: Quantized,
              seq_tokens: Sequence[np.ndarray], softmax_scale: float = 0.0) -> np.ndarray:
    """fp64 decode attention; sequence b reads unique tokens seq_tokens[b]
    in order.  q: fp16 [B][Hq][D].  Returns [B][Hq][D] fp64."""
    idx = np.concatenate([np.asarray(t, np.int64) for t in seq_tokens])
    lens = [len(t) for t in seq_tokens]
    return decode_attention(q, kq.deq[idx], vq.deq[idx], lens, softmax_scale)


def prefill(q: np.ndarray, kq: Quantized, vq: Quantized,
            seq_tokens: Sequence[np.ndarray], chunk_lens: Sequence[int],
            softmax_scale: float = 0.0) -> np.ndarray:
    """fp64 chunked-prefill attention: sequence b reads unique tokens
    seq_tokens[b] in order, the last chunk_lens[b] of which are its chunk.
    q: fp16 [sum chunk][Hq][D].  Returns [sum chunk][Hq][D] fp64."""
    idx = np.concatenate([np.asarray(t, np.int64) for t in seq_tokens])
    lens = [len(t) for t in seq_tokens]
    return prefill_attention(q, kq.deq[idx], vq.deq[idx], chunk_lens, lens, softmax_scale)


def tolerance_ok(got: np.ndarray, ref: np.ndarray, atol: float = 2e-3,
                 rtol: float = 1e-3):
    """Elementwise |got - ref| <= atol + rtol * |ref|.  Returns (ok, max_abs,
    max_rel, worst_excess)."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    ok = bool(np.all(err <= bound)) and not np.isnan(got).any()
    max_abs = float(err.max()) if err.size else 0.0
    max_rel = float((err / np.maximum(np.abs(ref), 1e-30)).max()) if err.size else 0.0
    excess = float((err - bound).max()) if err.size else -1.0
    return ok, max_abs, max_rel, excess
