"""Pins of the oracle's chunked-prefill attention against things other than
itself ("KV Cache优化实战" s1.1: prefill computes every prompt token's K/V and
each token attends to the tokens before it; xpshop.cn article 312 s6: long
prompts are processed in chunks).  CPU only.
"""
import numpy as np
import pytest
import torch

import oracle


def _case(rng, B=3, Hq=8, Hkv=2, d=32, ctx=(5, 40, 17), chunk=(5, 9, 1)):
    ctx = np.asarray(ctx)
    chunk = np.asarray(chunk)
    q = rng.standard_normal((int(chunk.sum()), Hq, d)).astype(np.float16)
    K = rng.standard_normal((int(ctx.sum()), Hkv, d))
    V = rng.standard_normal((int(ctx.sum()), Hkv, d))
    return q, K, V, chunk, ctx


def test_prefill_matches_torch_sdpa_with_offset_causal_mask():
    rng = np.random.default_rng(21)
    q, K, V, n, c = _case(rng)
    got = oracle.prefill_attention(q, K, V, n, c)
    Hq, Hkv = q.shape[1], K.shape[1]
    r = Hq // Hkv
    qo = ko = 0
    for b in range(len(n)):
        qb = torch.from_numpy(q[qo:qo + n[b]].astype(np.float64)).transpose(0, 1)  # [Hq][n][d]
        kb = torch.from_numpy(K[ko:ko + c[b]]).transpose(0, 1).repeat_interleave(r, 0)
        vb = torch.from_numpy(V[ko:ko + c[b]]).transpose(0, 1).repeat_interleave(r, 0)
        pos = torch.arange(c[b] - n[b], c[b])[:, None]
        mask = torch.arange(c[b])[None, :] <= pos                                   # [n][ctx]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qb.contiguous(), kb.contiguous(), vb.contiguous(), attn_mask=mask)
        assert np.allclose(got[qo:qo + n[b]], ref.transpose(0, 1).numpy(), rtol=1e-12, atol=1e-12)
        qo += n[b]
        ko += c[b]


def test_prefill_last_token_equals_decode_over_the_whole_context():
    rng = np.random.default_rng(22)
    q, K, V, n, c = _case(rng, ctx=(12, 33, 7), chunk=(12, 4, 3))
    got = oracle.prefill_attention(q, K, V, n, c)
    last = np.cumsum(n) - 1
    dec = oracle.decode_attention(q[last], K, V, c)
    assert np.allclose(got[last], dec, rtol=1e-13, atol=1e-13)


def test_prefill_first_prompt_token_reads_only_itself():
    rng = np.random.default_rng(23)
    q, K, V, n, c = _case(rng, B=2, ctx=(6, 9), chunk=(6, 9))   # whole prompts
    got = oracle.prefill_attention(q, K, V, n, c)
    Hq, Hkv = q.shape[1], K.shape[1]
    for b, (qo, ko) in enumerate([(0, 0), (6, 6)]):
        for g in range(Hq):
            assert np.array_equal(got[qo, g], V[ko, g // (Hq // Hkv)])


def test_prefill_chunking_is_invisible():
    # one chunk of 10 after 20 cached tokens == the last 10 rows of a 30-token prompt
    rng = np.random.default_rng(24)
    q, K, V, _, _ = _case(rng, B=1, ctx=(30,), chunk=(30,))
    whole = oracle.prefill_attention(q, K, V, [30], [30])
    part = oracle.prefill_attention(q[20:], K, V, [10], [30])
    assert np.allclose(part, whole[20:], rtol=1e-13, atol=1e-13)


def test_prefill_brute_force_tiny():
    rng = np.random.default_rng(25)
    q, K, V, n, c = _case(rng, B=1, Hq=2, Hkv=1, d=4, ctx=(4,), chunk=(3,))
    got = oracle.prefill_attention(q, K, V, n, c)
    sm = 1 / np.sqrt(4)
    for i in range(3):
        pos = 1 + i
        for g in range(2):
            w = np.exp([sm * q[i, g].astype(np.float64) @ K[t, 0] for t in range(pos + 1)])
            o = sum(w[t] * V[t, 0] for t in range(pos + 1)) / w.sum()
            assert np.allclose(got[i, g], o, rtol=1e-12, atol=1e-12)


def test_prefill_rejects_chunk_longer_than_context():
    q = np.zeros((3, 2, 4), np.float16)
    with pytest.raises(ValueError):
        oracle.prefill_attention(q, np.zeros((2, 1, 4)), np.zeros((2, 1, 4)), [3], [2])
