"""Parity at the benchmark's full sizes, in the launch configuration the
benchmark times (automatic split), on every sequence.

For each workload the whole pool is built on the GPU (prefill writes, the
copy-on-write copies, the one-token append) and the decode runs over every
sequence.  Then every sequence is checked against the CPU oracle: its cache
codes and scales, read back through its block table (every slot a table
reaches), bit for bit; its outputs within 2e-3 + 1e-3 * |ref|.  Sequences are
checked in batches of bounded token count, to bound host memory.
"""
import gc

import numpy as np
import pytest
import torch

from oracle import expected as E
from paged_quantized_kv_cache_amd import kvq
from paged_quantized_kv_cache_amd import workloads as W
from paged_quantized_kv_cache_amd.harness import DecodeCase

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-3
BATCH_TOKENS = 160_000      # logical tokens per checked batch of sequences


def _batches(lens):
    out, cur, n = [], [], 0
    for b, c in enumerate(lens):
        if cur and n + int(c) > BATCH_TOKENS:
            out.append(cur)
            cur, n = [], 0
        cur.append(b)
        n += int(c)
    if cur:
        out.append(cur)
    return out


def _check_seqs(case, layer, got_all, seqs):
    s, fmt = case.spec, case.fmt(layer)
    d = case.data[layer]
    ids = np.unique(np.concatenate([case.layout.seq_tokens[b] for b in seqs]))
    remap = np.full(case.layout.n_unique, -1, np.int64)
    remap[ids] = np.arange(ids.size)
    idx = torch.from_numpy(ids).to(d.k.device)
    k16 = d.k.index_select(0, idx).cpu().numpy()
    v16 = d.v.index_select(0, idx).cpu().numpy()
    sk = sv = None
    if kvq.scale_mode(fmt, s.G) in ("head", "channel"):   # static scales
        sk = case.pools[layer].k_scale.cpu().numpy()
        sv = case.pools[layer].v_scale.cpu().numpy()
    kq = E.quantize(k16, fmt, s.G, sk)
    vq = E.quantize(v16, fmt, s.G, sv)
    toks = [remap[case.layout.seq_tokens[b]] for b in seqs]
    codes = case.gather_codes(layer, seqs)
    for i, b in enumerate(seqs):
        t = toks[i]
        gk, gv = codes[i]["k"], codes[i]["v"]
        if fmt == "fp16":
            gk, gv = gk.view(np.uint16), gv.view(np.uint16)
        assert np.array_equal(gk, kq.codes[t]), "K codes (layer %d seq %d)" % (layer, b)
        assert np.array_equal(gv, vq.codes[t]), "V codes (layer %d seq %d)" % (layer, b)
        if kq.scales is not None:
            assert np.array_equal(codes[i]["k_scale"], kq.scales[t]), \
                "K scales (layer %d seq %d)" % (layer, b)
            assert np.array_equal(codes[i]["v_scale"], vq.scales[t]), \
                "V scales (layer %d seq %d)" % (layer, b)
    q = d.q.cpu().numpy()[seqs]
    ref = E.attention(q, kq, vq, toks)
    ok, mabs, mrel, excess = E.tolerance_ok(got_all[seqs], ref, ATOL, RTOL)
    assert ok, "layer %d (%s) seqs %d..%d: max_abs %.3g max_rel %.3g excess %.3g" % (
        layer, fmt, seqs[0], seqs[-1], mabs, mrel, excess)
    err = np.abs(got_all[seqs] - ref) / (ATOL + RTOL * np.abs(ref))
    return float(err.max())


def _check_layer(case, layer, seqs=None):
    out = case.decode(layer).float()
    assert torch.isfinite(out).all(), "non-finite output"
    got = out.cpu().numpy()
    lens = case.lens if seqs is None else case.lens[seqs]
    base = np.arange(case.spec.B) if seqs is None else np.asarray(seqs)
    worst = 0.0
    for bt in _batches(lens):
        worst = max(worst, _check_seqs(case, layer, got, [int(base[i]) for i in bt]))
    return worst


def _run(name, layers=(0,)):
    print("workload", name, flush=True)
    spec = W.spec(name)
    case = DecodeCase(spec, device="cuda:0", poison=True)
    try:
        for layer in layers:
            case.setup_layer(layer)
            worst = _check_layer(case, layer)
            print("  layer %d %s: every sequence, worst err/bound %.3f"
                  % (layer, case.fmt(layer), worst), flush=True)
            case.pools[layer] = None
            case.data[layer] = None
    finally:
        del case
        gc.collect()
        torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["c1_tiny", "c2_mha", "c3_gqa", "c3_gqa_fp16",
                                  "c4_long_bs16", "c4_long_bs32", "c4_long_e5m2",
                                  "c3_fp8_token", "c3_int8_channel", "c3_int4"])
def test_full_size_single_layer(name, gpu):
    _run(name)


def test_full_size_prefix_sharing_mixed_precision(gpu):
    # the 32-layer workload: fp16 layers 0 and 28-31, INT8 g128 layers 1-27,
    # each over the shared-prefix layout with its copy-on-write copies
    _run("c5_prefix_mixed", layers=tuple(range(32)))


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_single_long_sequence_split_over_every_wavefront(fmt, gpu):
    # one 131,072-token sequence: each of its 8 units is cut into ~250
    # pieces (more than a wavefront's 64 lanes), merged by one workgroup each
    spec = W.spec("c4_long_bs16", fmt=fmt, G=0 if fmt == "fp8" else 64, B=1,
                  lens="fixed", lens_args=(131072,))
    print("case", fmt, flush=True)
    case = DecodeCase(spec, device=gpu, poison=True)
    case.setup_layer(0)
    _check_layer(case, 0, [0])
