"""Pins of the oracle's format variants against things other than itself:
FP8 E5M2 (the "fp8_e5m2" cache dtype of xpshop.cn article 312 s3), FP8 with
dynamic per-group / per-token scales, and INT8 with static per-channel scales
("KV Cache优化实战" s2.3, s3.3, s4.2).  CPU only.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import expected as E

ALL_F16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
FMAX = {"e4m3": 448.0, "e5m2": 57344.0}
TORCH_FP8 = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def finite_f16():
    x = ALL_F16.view(np.float16)
    return x[np.isfinite(x)]


# ------------------------------------------------------------------ E5M2
def test_e5m2_decode_is_the_high_byte_of_an_fp16():
    # E5M2 has fp16's sign and exponent fields and the top 2 fraction bits
    codes = np.arange(256, dtype=np.uint16)
    got = oracle.e5m2_decode(codes.astype(np.uint8))
    ref = (codes << 8).astype(np.uint16).view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0]) == {0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF}
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_e5m2_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e5m2_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e5m2).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e5m2_spec_values():
    # OCP 8-bit floating point specification, E5M2 column
    for code, val in [(0x7B, 57344.0), (0x04, 2.0 ** -14), (0x03, 0.75 * 2.0 ** -14),
                      (0x01, 2.0 ** -16), (0x3C, 1.0), (0x7C, math.inf),
                      (0xFC, -math.inf), (0x80, -0.0)]:
        got = oracle.e5m2_decode(np.array([code], np.uint8))[0]
        assert got == val and math.copysign(1, got) == math.copysign(1, val)


def test_e5m2_encode_matches_brute_force_on_all_fp16_values():
    xs = finite_f16().astype(np.float32)
    got = oracle.e5m2_encode(xs)
    pos = np.arange(0x7C)                      # non-negative finite codes
    vals = oracle.e5m2_decode(pos.astype(np.uint8))
    a = np.abs(xs.astype(np.float64))[:, None]
    dist = np.abs(vals[None, :] - a)
    cand = dist == dist.min(1, keepdims=True)
    even = cand & ((pos[None, :] & 1) == 0)
    pick = np.where(even.any(1), np.argmax(even, 1), np.argmax(cand, 1))
    best = pos[pick]
    best[np.abs(xs) >= 57344] = 0x7B
    best = best | np.where(np.signbit(xs), 0x80, 0)
    assert np.array_equal(got.astype(np.int64), best)


def test_e5m2_encode_matches_torch_in_range():
    rng = np.random.default_rng(5)
    y = np.concatenate([rng.standard_normal(20000) * 3000,
                        rng.standard_normal(5000) * 1e-4,
                        np.linspace(-57343.0, 57343.0, 20001)]).astype(np.float32)
    got = oracle.e5m2_encode(y)
    ref = torch.from_numpy(y).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_e5m2_round_trip_and_saturation():
    codes = np.array([c for c in range(256) if (c & 0x7F) < 0x7C], np.uint8)
    vals = oracle.e5m2_decode(codes)
    assert np.array_equal(oracle.e5m2_encode(vals.astype(np.float32)), codes)
    sat = oracle.e5m2_encode(np.array([57344.0, 61440.0, 1e6, -1e38,
                                       np.float32(np.inf)], np.float32))
    assert list(sat) == [0x7B, 0x7B, 0x7B, 0xFB, 0x7B]
    pos = oracle.e5m2_decode(np.arange(0x7C, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)


# ------------------------------------------------------------------ FP8, dynamic group scales
def _fp8_groups_independent(x16, G, fmt):
    """Same definition through numpy fp32 arithmetic (IEEE division) and
    torch's FP8 conversion (round to nearest even) of the saturated value."""
    x = x16.astype(np.float32)
    shp = x.shape[:-1] + (x.shape[-1] // G, G)
    xg = x.reshape(shp)
    a = np.abs(xg).max(-1)
    s = (a / np.float32(FMAX[fmt])).astype(np.float32)
    safe = np.where(s == 0, np.float32(1), s)
    y = (xg / safe[..., None]).astype(np.float32)
    y = np.clip(y, -FMAX[fmt], FMAX[fmt]).astype(np.float32)
    c = torch.from_numpy(np.ascontiguousarray(y)).to(TORCH_FP8[fmt]).view(torch.uint8).numpy()
    c = np.where((s == 0)[..., None], np.uint8(0), c)
    return c.reshape(x.shape), s


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("G", [64, 128])
def test_fp8_group_codec_matches_independent_path(fmt, G):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((300, 2, 128)).astype(np.float32)
    x[:, :, 7] *= 40.0                  # an outlier channel
    x[5, 1, :] = 0.0                    # an all-zero token-head
    x[9, 0, :64] = 0.0                  # an all-zero group
    x[12, 0, 3] = -0.0
    x16 = x.astype(np.float16)
    codes, scales = oracle.fp8_quantize_groups(x16, G, fmt)
    c_ref, s_ref = _fp8_groups_independent(x16, G, fmt)
    assert np.array_equal(scales, s_ref)
    assert np.array_equal(codes, c_ref)
    # the absmax element of every non-zero group codes to the largest finite value
    dec = (oracle.e5m2_decode if fmt == "e5m2" else oracle.e4m3_decode)(codes)
    grp = dec.reshape(300, 2, 128 // G, G)
    nz = scales > 0
    assert np.all(np.abs(grp).max(-1)[nz] == FMAX[fmt])
    # dequantization is code value times the group's scale
    deq = oracle.fp8_dequantize_groups(codes, scales, fmt)
    assert np.array_equal(deq, (grp * scales[..., None].astype(np.float64)).reshape(deq.shape))


# ------------------------------------------------------------------ INT8, static per-channel scales
def test_int8_channel_codec_matches_independent_path():
    rng = np.random.default_rng(12)
    x16 = (rng.standard_normal((200, 3, 64)) * np.linspace(0.1, 8, 64)).astype(np.float16)
    S = (np.abs(x16.astype(np.float32)).max(0) / np.float32(127)).astype(np.float32)
    S[1, 5] = 0.0                                   # a channel with no scale
    S[2, 9] *= np.float32(0.5)                      # a scale too small: clamps
    codes = oracle.int8_quantize_channels(x16, S)
    safe = np.where(S == 0, np.float32(1), S)
    y = (x16.astype(np.float32) / safe[None]).astype(np.float32)
    ref = np.clip(np.rint(y), -127, 127).astype(np.int8)
    ref[:, 1, 5] = 0
    assert np.array_equal(codes, ref)
    assert np.abs(codes[:, 2, 9]).max() == 127
    deq = oracle.int8_dequantize_channels(codes, S)
    assert np.array_equal(deq, codes.astype(np.float64) * S[None].astype(np.float64))
    # within half a step of the input where nothing clamps
    ok = (S > 0)[None] & (np.abs(y) <= 127)
    err = np.abs(deq - x16.astype(np.float64))
    assert np.all(err[ok] <= (S.astype(np.float64)[None] * (0.5 + 2.0 ** -16) + 0 * err)[ok])


# ------------------------------------------------------------------ dispatch
def test_expected_quantize_modes():
    rng = np.random.default_rng(13)
    x16 = rng.standard_normal((20, 2, 128)).astype(np.float16)
    hs = np.array([0.01, 0.02], np.float32)
    cs = np.full((2, 128), 0.03, np.float32)
    q = E.quantize(x16, "e5m2", 0, hs)
    assert q.scales is None and np.array_equal(q.codes, oracle.fp8_quantize(x16, hs, "e5m2"))
    q = E.quantize(x16, "fp8", 128)
    assert q.scales.shape == (20, 2, 1)
    q = E.quantize(x16, "e5m2", 64)
    assert q.scales.shape == (20, 2, 2)
    q = E.quantize(x16, "int8", 0, cs)
    assert q.scales is None and np.array_equal(q.deq, q.codes * np.float64(np.float32(0.03)))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_static_zero_scale_gives_code_zero(fmt):
    x16 = np.random.default_rng(14).standard_normal((5, 2, 64)).astype(np.float16)
    x16[:, 1] = 0                                   # an all-zero head: scale 0
    S = np.array([0.01, 0.0], np.float32)
    codes = oracle.fp8_quantize(x16, S, fmt)
    assert np.all(codes[:, 1] == 0)
    assert np.all(oracle.fp8_dequantize(codes, S, fmt)[:, 1] == 0)


# ------------------------------------------------------------------ INT4, per-group
@pytest.mark.parametrize("G", [64, 128])
def test_int4_codec_matches_independent_path(G):
    rng = np.random.default_rng(15)
    x = rng.standard_normal((300, 2, 128)).astype(np.float32)
    x[:, :, 9] *= 30.0                  # an outlier channel
    x[4, 1, :] = 0.0                    # an all-zero token-head
    x16 = x.astype(np.float16)
    codes, scales = oracle.int4_quantize(x16, G)
    xg = x16.astype(np.float32).reshape(300, 2, 128 // G, G)
    a = np.abs(xg).max(-1)
    s = (a / np.float32(7)).astype(np.float32)          # IEEE fp32 division
    safe = np.where(s == 0, np.float32(1), s)
    y = (xg / safe[..., None]).astype(np.float32)
    ref = np.clip(np.rint(y), -7, 7).astype(np.int8)
    ref = np.where((s == 0)[..., None], np.int8(0), ref).reshape(codes.shape)
    assert np.array_equal(scales, s) and np.array_equal(codes, ref)
    # absmax element codes to +-7; error within half a step
    assert np.all(np.abs(codes.reshape(xg.shape)).max(-1)[s > 0] == 7)
    deq = oracle.int8_dequantize(codes, scales)
    step = np.repeat(scales.astype(np.float64), G, axis=-1).reshape(deq.shape)
    assert np.all(np.abs(deq - x16.astype(np.float64)) <= step * (0.5 + 2.0 ** -16))
    q = E.quantize(x16, "int4", G)
    assert np.array_equal(q.codes, codes) and np.array_equal(q.deq, deq)
