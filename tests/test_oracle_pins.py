"""Pins of the CPU oracle against things other than itself.

Each test ties an oracle function to a library routine, a brute-force
computation, a closed form, an invariant or a value printed on the pages /
in a published format specification.  All run on the CPU (no GPU marker).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ALL_F16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def finite_f16():
    x = ALL_F16.view(np.float16)
    return x[np.isfinite(x)]


# ------------------------------------------------------------------ fp16
def test_f16_decode_matches_numpy_for_every_bit_pattern():
    got = oracle.f16_to_f64(ALL_F16)
    ref = ALL_F16.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ------------------------------------------------------------------ INT8
def _independent_int8(a16, x16):
    """Same definition, different arithmetic path: fp64 division of fp32
    operands rounded once to fp32 equals the correctly rounded fp32 quotient
    (53 >= 2*24 + 2), numpy's rint rounds half to even."""
    a = np.float64(np.float32(a16))
    s = np.float32(a / 127.0)
    if s == 0:
        return s, np.zeros_like(x16, dtype=np.int8)
    y = (x16.astype(np.float32).astype(np.float64) / np.float64(s)).astype(np.float32)
    q = np.clip(np.rint(y), -127, 127).astype(np.int8)
    return s, q


@pytest.mark.parametrize("a", [1.0, 0.1, 3.5, 17.25, 65504.0, 6.1035e-05,
                               5.96e-08, 0.333, 1000.0])
def test_int8_codec_exhaustive_against_independent_rounding(a):
    a16 = np.float16(a)
    xs = finite_f16()
    xs = xs[np.abs(xs.astype(np.float64)) <= float(a16)]
    # groups of two: [a, x] so the absmax of every group is a
    grp = np.stack([np.full_like(xs, a16), xs], axis=1)
    codes, scales = oracle.int8_quantize(grp, 2)
    s_ref, q_ref = _independent_int8(a16, xs)
    assert np.all(scales[:, 0] == s_ref)
    assert np.array_equal(codes[:, 1], q_ref)
    assert np.all(codes[:, 0] == 127)            # the absmax element -> 127


def test_int8_invariants_random_groups():
    rng = np.random.default_rng(1)
    for G in (64, 128):
        x = (rng.standard_normal((512, 256)) *
             np.exp(rng.uniform(-8, 8, (512, 1)))).astype(np.float16)
        x[3] = 0                                  # an all-zero row
        codes, sc = oracle.int8_quantize(x, G)
        xg = x.astype(np.float64).reshape(512, -1, G)
        cg = codes.astype(np.float64).reshape(512, -1, G)
        s = sc.astype(np.float64)[..., None]
        # round-trip error <= s * (1/2 + fp32 rounding of x/s)
        assert np.all(np.abs(xg - cg * s) <= s * (0.5 + 2.0 ** -16) + 0.0)
        # every non-zero group reaches +-127 at its absmax element
        amax = np.abs(xg).max(-1)
        nz = amax > 0
        assert np.all(np.abs(cg).max(-1)[nz] == 127)
        assert np.all(sc[~nz] == 0) and np.all(cg[~nz] == 0)
        assert np.abs(codes.astype(np.int32)).max() <= 127  # -128 never appears
        # odd symmetry
        codes_neg, sc_neg = oracle.int8_quantize(-x, G)
        assert np.array_equal(codes_neg, -codes) and np.array_equal(sc_neg, sc)
        # scale = fl32(absmax / 127)
        assert np.array_equal(sc, (amax / 127.0).astype(np.float32))
        # dequantize = code * scale exactly
        deq = oracle.int8_dequantize(codes, sc)
        assert np.array_equal(deq.reshape(512, -1, G), cg * s)


def test_int8_groups_run_along_head_dim():
    # one huge element only affects the scale of its own group
    x = np.ones((1, 2, 128), np.float16)
    x[0, 1, 70] = 1000.0
    codes, sc = oracle.int8_quantize(x, 64)
    assert sc.shape == (1, 2, 2)
    assert sc[0, 0, 0] == sc[0, 0, 1] == sc[0, 1, 0] == np.float32(1.0 / 127.0)
    assert sc[0, 1, 1] == np.float32(1000.0 / 127.0)
    assert np.all(codes[0, 1, :64] == 127)


def test_int8_rejects_nonfinite():
    x = np.zeros((1, 64), np.float16)
    x[0, 5] = np.inf
    with pytest.raises(ValueError):
        oracle.int8_quantize(x, 64)


# ------------------------------------------------------------------ FP8
def _ocp_table():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_ocp_table.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                c, v = line.split()
                rows.append((int(c, 16), float(v)))
    return rows


def test_e4m3_decode_spec_values():
    for code, val in _ocp_table():
        got = oracle.e4m3_decode(np.array([code], np.uint8))[0]
        assert got == val and math.copysign(1, got) == math.copysign(1, val)


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def _brute_e4m3(y: float) -> int:
    """Nearest finite E4M3 by exhaustive search; ties -> even code; beyond
    the largest finite magnitude -> saturate; sign kept on zero."""
    codes = [c for c in range(128) if c != 0x7F]
    vals = {c: oracle.e4m3_decode(np.array([c], np.uint8))[0] for c in codes}
    a = abs(y)
    if a >= 448.0:
        best = 0x7E
    else:
        best = min(codes, key=lambda c: (abs(vals[c] - a), c & 1))
    return best | (0x80 if math.copysign(1.0, y) < 0 else 0)


def test_e4m3_encode_matches_brute_force_on_all_fp16_values():
    xs = finite_f16().astype(np.float32)
    got = oracle.e4m3_encode(xs)
    # brute force, vectorised over the 127 non-negative finite codes
    pos = np.array([c for c in range(128) if c != 0x7F])
    vals = oracle.e4m3_decode(pos.astype(np.uint8))
    a = np.abs(xs.astype(np.float64))[:, None]
    dist = np.abs(vals[None, :] - a)
    # tie-break: smaller distance, then even code
    key = dist * 4 + (pos[None, :] & 1) * 0  # distances are exact dyadics
    best = np.empty(xs.size, np.int64)
    dmin = dist.min(1, keepdims=True)
    cand = dist == dmin
    even = cand & ((pos[None, :] & 1) == 0)
    pick = np.where(even.any(1), np.argmax(even, 1), np.argmax(cand, 1))
    best = pos[pick]
    best[np.abs(xs) >= 448] = 0x7E
    best = best | np.where(np.signbit(xs), 0x80, 0)
    assert np.array_equal(got.astype(np.int64), best)
    # a few scalars through the slow path too
    for y in (0.0, -0.0, 1e-30, -1e-30, 464.0, 480.0, 1e9, 0.0009765625, 3.0 * 2 ** -10):
        assert oracle.e4m3_encode(np.array([y], np.float32))[0] == _brute_e4m3(y)


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(2)
    y = np.concatenate([rng.standard_normal(20000) * 50,
                        rng.standard_normal(5000) * 0.01,
                        np.linspace(-447.9, 447.9, 20001)]).astype(np.float32)
    got = oracle.e4m3_encode(y)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_e4m3_round_trip_and_saturation():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.e4m3_decode(codes)
    assert np.array_equal(oracle.e4m3_encode(vals.astype(np.float32)), codes)
    sat = oracle.e4m3_encode(np.array([448.0, 449.0, 500.0, 1e38, -1e38,
                                       np.float32(np.inf)], np.float32))
    assert list(sat) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E]
    # monotone over the positive codes
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)


def test_fp8_quantize_uses_per_head_static_scale():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((10, 3, 16)).astype(np.float16)
    S = np.array([0.01, 0.5, 2.0], np.float32)
    codes = oracle.fp8_quantize(x, S)
    for h in range(3):
        y = (x[:, h].astype(np.float32) / S[h]).astype(np.float32)
        ref = torch.from_numpy(np.clip(y, -448, 448)).to(torch.float8_e4m3fn)
        assert np.array_equal(codes[:, h], ref.view(torch.uint8).numpy())
    deq = oracle.fp8_dequantize(codes, S)
    assert np.array_equal(deq, oracle.e4m3_decode(codes) * S[None, :, None].astype(np.float64))


# ------------------------------------------------------------------ attention
def _naive_attention(q, K, V, lens, sm):
    """Textbook softmax without max subtraction, explicit loops."""
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    r = Hq // Hkv
    out = np.zeros((B, Hq, d))
    off = 0
    for b in range(B):
        n = int(lens[b])
        for g in range(Hq):
            h = g // r
            w = [math.exp(sm * sum(float(q[b, g, i]) * K[off + t, h, i] for i in range(d)))
                 for t in range(n)]
            tot = sum(w)
            for i in range(d):
                out[b, g, i] = sum(w[t] * V[off + t, h, i] for t in range(n)) / tot
        off += n
    return out


def _rand_case(rng, B, Hq, Hkv, d, lens, scale=1.0):
    q = (rng.standard_normal((B, Hq, d)) * scale).astype(np.float16)
    n = int(np.sum(lens))
    K = rng.standard_normal((n, Hkv, d))
    V = rng.standard_normal((n, Hkv, d))
    return q, K, V


def test_attention_brute_force_tiny():
    rng = np.random.default_rng(4)
    lens = [1, 3, 4]
    q, K, V = _rand_case(rng, 3, 4, 2, 8, lens)
    got = oracle.decode_attention(q, K, V, lens)
    ref = _naive_attention(q, K, V, lens, 1 / math.sqrt(8))
    assert np.max(np.abs(got - ref)) < 1e-12


def test_attention_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(5)
    lens = [7, 33, 64, 130]
    B, Hq, Hkv, d = 4, 8, 2, 64
    q, K, V = _rand_case(rng, B, Hq, Hkv, d, lens, scale=2.0)
    got = oracle.decode_attention(q, K, V, lens)
    off = 0
    for b in range(B):
        n = lens[b]
        kq = torch.from_numpy(K[off:off + n]).permute(1, 0, 2)   # [Hkv, n, d]
        vq = torch.from_numpy(V[off:off + n]).permute(1, 0, 2)
        kq = kq.repeat_interleave(Hq // Hkv, 0)                  # g -> g // r
        vq = vq.repeat_interleave(Hq // Hkv, 0)
        qq = torch.from_numpy(q[b].astype(np.float64))[:, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kq, vq)[:, 0]
        assert np.max(np.abs(got[b] - ref.numpy())) < 1e-12
        off += n


def test_attention_closed_forms():
    rng = np.random.default_rng(6)
    # ctx = 1: the output is the single value row, exactly
    q, K, V = _rand_case(rng, 2, 4, 2, 16, [1, 1])
    got = oracle.decode_attention(q, K, V, [1, 1])
    for b in range(2):
        for g in range(4):
            assert np.array_equal(got[b, g], V[b, g // 2])
    # identical keys (or q = 0): the mean of the values
    lens = [5, 9]
    q, K, V = _rand_case(rng, 2, 4, 2, 16, lens)
    K[:] = K[0]
    got = oracle.decode_attention(q, K, V, lens)
    qz = np.zeros_like(q)
    K2 = rng.standard_normal(K.shape)
    got0 = oracle.decode_attention(qz, K2, V, lens)
    off = 0
    for b, n in enumerate(lens):
        mean = V[off:off + n].mean(0)
        for g in range(4):
            assert np.allclose(got[b, g], mean[g // 2], atol=1e-14, rtol=0)
            assert np.allclose(got0[b, g], mean[g // 2], atol=1e-14, rtol=0)
        off += n
    # a dominant key: the output follows its value
    lens = [6]
    q = np.zeros((1, 1, 4), np.float16)
    q[0, 0, 0] = 8.0
    K = np.zeros((6, 1, 4))
    K[2, 0, 0] = 100.0
    V = rng.standard_normal((6, 1, 4))
    got = oracle.decode_attention(q, K, V, lens)
    assert np.allclose(got[0, 0], V[2, 0], atol=1e-12)


def test_gqa_equals_mha_on_replicated_heads_and_mqa():
    rng = np.random.default_rng(7)
    lens = [3, 17, 40]
    B, Hq, Hkv, d = 3, 8, 2, 32
    q, K, V = _rand_case(rng, B, Hq, Hkv, d, lens)
    gqa = oracle.decode_attention(q, K, V, lens)
    Kr = np.repeat(K, Hq // Hkv, axis=1)
    Vr = np.repeat(V, Hq // Hkv, axis=1)
    mha = oracle.decode_attention(q, Kr, Vr, lens)
    assert np.array_equal(gqa, mha)
    # MQA: one KV head serves every query head
    K1, V1 = K[:, :1], V[:, :1]
    mqa = oracle.decode_attention(q, K1, V1, lens)
    mha1 = oracle.decode_attention(q, np.repeat(K1, Hq, 1), np.repeat(V1, Hq, 1), lens)
    assert np.array_equal(mqa, mha1)
    # a wrong head mapping (g % Hkv instead of g // r) would differ
    Kp = K[:, [1, 0]]
    assert not np.allclose(oracle.decode_attention(q, Kp, V, lens), gqa)


def test_attention_softmax_scale_and_rejects_empty():
    rng = np.random.default_rng(8)
    q, K, V = _rand_case(rng, 1, 2, 1, 16, [5])
    a = oracle.decode_attention(q, K, V, [5], softmax_scale=0.25)
    b = oracle.decode_attention(q, K * 0.25 * 4.0, V, [5])  # 1/sqrt(16) = 0.25
    assert np.allclose(a, b, atol=1e-14)
    with pytest.raises(ValueError):
        oracle.decode_attention(q, K[:0], V[:0], [0])


# ------------------------------------------------------------------ bytes
def _bytes_rows():
    rows = []
    with open(os.path.join(GOLDEN, "kv_bytes_examples.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                p = line.split()
                rows.append(tuple(int(v) for v in p[:7]) + (float(p[7]), p[8]))
    return rows


def test_byte_formula_against_page_examples():
    for b, L, layers, kvh, d, bits, exp_bytes, exp_gib, note in _bytes_rows():
        got = oracle.kv_cache_bytes(b, L, layers, kvh, d, bits // 8)
        assert got == exp_bytes, note
        if exp_gib:
            assert abs(got / 2.0 ** 30 - exp_gib) < 0.005, note


def test_byte_formula_matches_allocated_arrays():
    B, L, layers, kvh, d = 3, 50, 2, 4, 64
    cache = np.zeros((2, B, L, layers, kvh, d), np.float16)
    assert cache.nbytes == oracle.kv_cache_bytes(B, L, layers, kvh, d, 2)
    rng = np.random.default_rng(9)
    for G in (64, 32):
        x = rng.standard_normal((B * L * layers, kvh, d)).astype(np.float16)
        codes, sc = oracle.int8_quantize(x, G)
        total = 2 * (codes.nbytes + sc.nbytes)
        assert total == oracle.kv_cache_bytes_int8_group(B, L, layers, kvh, d, G)
        ratio = total / oracle.kv_cache_bytes(B, L, layers, kvh, d, 2)
        assert ratio == pytest.approx((1 + 4 / G) / 2)
    # GQA 8 KV heads vs MHA 32: exactly a quarter
    assert 4 * oracle.kv_cache_bytes(100, 2048, 32, 8, 128, 2) == \
        oracle.kv_cache_bytes(100, 2048, 32, 32, 128, 2)
