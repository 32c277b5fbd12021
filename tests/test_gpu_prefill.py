"""GPU parity of chunked-prefill attention over the paged pools
(kvq_paged_prefill through the C ABI) against the CPU oracle.

Each sequence's chunk is its last n_b tokens (already written by
kvq_cache_write); chunk token i attends to every token up to its position.
Chunks: whole prompts, a fixed-size tail chunk after cached tokens, one
token (where prefill must agree with decode), and short ragged chunks of at
most 16 / (Hq / Hkv) or 32 / (Hq / Hkv) tokens (empty ones included), which
are walked by the decode partition: runs over every wavefront, one MFMA
column per (chunk token, query head) with its own causal bound (one or two
groups of 16 columns per wavefront), cut units merged.  Tolerance
as for decode: |gpu - oracle| <= 2e-3 + 1e-3 |oracle|.
"""
import numpy as np
import pytest
import torch

from oracle import expected as E
from paged_quantized_kv_cache_amd import kvq
from paged_quantized_kv_cache_amd import workloads as W
from paged_quantized_kv_cache_amd.harness import DecodeCase

from test_gpu_parity import SMALL_CASES

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-3
CASES = ["c1_tiny", "gqa_int8_g64_outliers", "mha_int8_g128", "gqa_fp16", "fp8_bs32",
         "int8_bs32_g128_r8", "int8_d64_bs32_r16", "e5m2_bs16", "fp8_token_g128",
         "int8_channel", "int4_g64_outliers"]


def _quantized(case, layer, seqs):
    s, fmt = case.spec, case.fmt(layer)
    d = case.data[layer]
    sk = sv = None
    if kvq.scale_mode(fmt, s.G) in ("head", "channel"):
        sk = case.pools[layer].k_scale.cpu().numpy()
        sv = case.pools[layer].v_scale.cpu().numpy()
    ids = np.unique(np.concatenate([case.layout.seq_tokens[b] for b in seqs]))
    remap = np.full(case.layout.n_unique, -1, np.int64)
    remap[ids] = np.arange(ids.size)
    idx = torch.from_numpy(ids).to(d.k.device)
    kq = E.quantize(d.k.index_select(0, idx).cpu().numpy(), fmt, s.G, sk)
    vq = E.quantize(d.v.index_select(0, idx).cpu().numpy(), fmt, s.G, sv)
    toks = [remap[case.layout.seq_tokens[b]] for b in seqs]
    return kq, vq, toks


def _chunks(lens, mode, r=1):
    if mode == "whole":
        return lens.copy()
    if mode == "tail":
        return np.minimum(lens, 37)
    if mode in ("short", "short2"):  # at most 16 (32) / r tokens, ragged, one empty
        qpc = (16 if mode == "short" else 32) // r
        pat = [qpc, 1, max(qpc - 1, 1), 0, min(2, qpc)]
        return np.minimum(lens, [pat[b % len(pat)] for b in range(lens.size)])
    return np.ones_like(lens)


@pytest.mark.parametrize("cut", ["walk", "split"])
@pytest.mark.parametrize("mode", ["whole", "tail", "one", "short", "short2"])
@pytest.mark.parametrize("name", CASES)
def test_prefill_within_tolerance(name, mode, cut, gpu):
    """Both cuts of the work on every chunk shape: the per-(sequence, KV head,
    token groups) walk, and the decode partition (chunks longer than 32 / r
    tokens cut into virtual sequences first)."""
    print("case", name, mode, cut, flush=True)
    spec = SMALL_CASES[name]
    case = DecodeCase(spec, device=gpu, gen_device="cpu")
    case.setup_layer(0)
    n = _chunks(case.lens, mode, spec.Hq // spec.Hkv)
    q = case.chunk_queries(n)
    got = case.prefill_attention(0, n, q, split_mode=cut).float().cpu().numpy()
    assert np.isfinite(got).all()
    kq, vq, toks = _quantized(case, 0, range(spec.B))
    ref = E.prefill(q.cpu().numpy(), kq, vq, toks, n)
    ok, mabs, mrel, excess = E.tolerance_ok(got, ref, ATOL, RTOL)
    assert ok, "%s/%s: max_abs %.3g max_rel %.3g excess %.3g" % (name, mode, mabs, mrel, excess)


@pytest.mark.parametrize("name", ["gqa_int8_g64_outliers", "fp8_bs16", "gqa_fp16"])
def test_one_token_chunk_agrees_with_decode(name, gpu):
    spec = SMALL_CASES[name]
    case = DecodeCase(spec, device=gpu, gen_device="cpu")
    case.setup_layer(0)
    q = case.data[0].q.to(gpu).contiguous()
    dec = case.decode(0, q=q, workspace=case.workspace(0)).float().cpu().numpy()
    pre = case.prefill_attention(0, np.ones_like(case.lens), q).float().cpu().numpy()
    kq, vq, toks = _quantized(case, 0, range(spec.B))
    ref = E.attention(q.cpu().numpy(), kq, vq, toks)
    assert np.all(np.abs(dec - pre) <= 2 * (ATOL + RTOL * np.abs(ref)))


def test_full_size_prefill_every_row_of_four_prompts(gpu):
    # the prefill workload: 16 prompts of 2048 tokens, GQA 32/8, INT8 g64,
    # cut as the benchmark times it; every chunk row (all 2048 positions, all
    # 32 query heads) of four prompts against the oracle's causal attention,
    # and every output of the batch finite
    spec = W.spec("p1_prefill_gqa")
    print("workload", spec.name, flush=True)
    case = DecodeCase(spec, device=gpu, poison=True)
    case.setup_layer(0)
    n = case.lens.copy()
    q = case.chunk_queries(n)
    got = case.prefill_attention(0, n, q).float()
    assert torch.isfinite(got).all()
    got = got.cpu().numpy()
    seqs = [0, 5, 10, spec.B - 1]
    starts = np.concatenate([[0], np.cumsum(n)])
    rows = np.concatenate([np.arange(starts[b], starts[b + 1]) for b in seqs])
    kq, vq, toks = _quantized(case, 0, seqs)
    ref = E.prefill(q.cpu().numpy()[rows], kq, vq, toks, n[seqs])
    ok, mabs, mrel, excess = E.tolerance_ok(got[rows], ref, ATOL, RTOL)
    assert ok, "max_abs %.3g max_rel %.3g excess %.3g" % (mabs, mrel, excess)


@pytest.mark.parametrize("chunks", [(4, 3, 4, 1, 4, 2), (8, 5, 8, 1, 6, 2),
                                    (40, 17, 64, 1, 33, 2)])
@pytest.mark.parametrize("name", ["c3_gqa", "c3_gqa_fp16"])
def test_short_chunks_long_context(name, chunks, gpu):
    """A few new tokens per sequence (e.g. draft tokens to verify) over long
    cached contexts: every unit is cut into many pieces.  Lengths one or two
    past a block boundary leave last tiles whose tokens all lie beyond the
    first chunk tokens' causal bounds, so some pieces hold columns with no
    token to attend (they must weigh nothing in the merge)."""
    lens = (16 * 600 + 1, 16 * 900 + 2, 4097, 16 * 1200 + 1, 5000, 16 * 800 + 2)
    spec = W.spec(name, B=len(lens), lens="fixed", lens_args=lens)
    print("workload", spec.name, lens, flush=True)
    case = DecodeCase(spec, device=gpu, gen_device="cpu")
    case.setup_layer(0)
    n = np.array(chunks)
    assert kvq.kvq_prefill_workspace_size(spec.B, spec.Hq, spec.Hkv, spec.D, spec.BS,
                                          case.max_context_len, int(n.max())) > 0
    q = case.chunk_queries(n)
    got = case.prefill_attention(0, n, q).float().cpu().numpy()
    assert np.isfinite(got).all()
    kq, vq, toks = _quantized(case, 0, range(spec.B))
    ref = E.prefill(q.cpu().numpy(), kq, vq, toks, n)
    ok, mabs, mrel, excess = E.tolerance_ok(got, ref, ATOL, RTOL)
    assert ok, "max_abs %.3g max_rel %.3g excess %.3g" % (mabs, mrel, excess)
    # the last chunk token of each sequence is its decode row
    last = np.cumsum(n) - 1
    qd = q[torch.from_numpy(last).to(q.device)].contiguous()
    dec = case.decode(0, q=qd).float().cpu().numpy()
    assert np.all(np.abs(dec - got[last]) <= 2 * (ATOL + RTOL * np.abs(ref[last])))


@pytest.mark.parametrize("name", ["p2_short_chunks", "p3_short_chunks_8", "p4_medium_chunks"])
def test_full_size_chunk_workloads_every_row(name, gpu):
    """The chunk workloads at their benchmark sizes (sequences of 32,768
    cached tokens with 4-, 8- or 32-token chunks), cut as the benchmark
    times them (split mode auto: the short-chunk path, or virtual sequences
    for the 32-token chunks): every chunk row of every sequence against the
    oracle."""
    spec = W.spec(name)
    print("workload", spec.name, flush=True)
    case = DecodeCase(spec, device=gpu, poison=True)
    case.setup_layer(0)
    n = np.minimum(case.lens, spec.chunk)
    q = case.chunk_queries(n)
    got = case.prefill_attention(0, n, q).float()
    assert torch.isfinite(got).all()
    got = got.cpu().numpy()
    qh = q.cpu().numpy()
    starts = np.concatenate([[0], np.cumsum(n)])
    for b0 in range(0, spec.B, 4):
        seqs = list(range(b0, min(b0 + 4, spec.B)))
        rows = np.concatenate([np.arange(starts[b], starts[b + 1]) for b in seqs])
        kq, vq, toks = _quantized(case, 0, seqs)
        ref = E.prefill(qh[rows], kq, vq, toks, n[seqs])
        ok, mabs, mrel, excess = E.tolerance_ok(got[rows], ref, ATOL, RTOL)
        assert ok, "seqs %s: max_abs %.3g max_rel %.3g excess %.3g" % (seqs, mabs, mrel, excess)
