"""Parity at the benchmark's full sizes, in the launch configuration the
benchmark times (automatic split), on sampled sequences.

For each workload the whole pool is built on the GPU (prefill writes, the
copy-on-write copies, the one-token append), the decode runs over every
sequence, and a seeded sample of sequences -- always including the longest
and the shortest -- is checked against the CPU oracle: cache codes and scales
bit-exact through the block tables, outputs within 2e-3 + 1e-3 * |ref|.
Every output of the batch is also checked to be finite.
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


def _sample(lens, k=4, seed=0):
    rng = np.random.default_rng(seed)
    picks = {int(np.argmax(lens)), int(np.argmin(lens))}
    while len(picks) < min(k, len(lens)):
        picks.add(int(rng.integers(len(lens))))
    return sorted(picks)


def _check_layer(case, layer, seqs):
    s, fmt = case.spec, case.fmt(layer)
    d = case.data[layer]
    out = case.decode(layer).float()
    assert torch.isfinite(out).all(), "non-finite output"
    got = out.cpu().numpy()[seqs]
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
        assert np.array_equal(gk, kq.codes[t]), "K codes (seq %d)" % b
        assert np.array_equal(gv, vq.codes[t]), "V codes (seq %d)" % b
        if kq.scales is not None:
            assert np.array_equal(codes[i]["k_scale"], kq.scales[t]), "K scales (seq %d)" % b
            assert np.array_equal(codes[i]["v_scale"], vq.scales[t]), "V scales (seq %d)" % b
    q = d.q.cpu().numpy()[seqs]
    ref = E.attention(q, kq, vq, toks)
    ok, mabs, mrel, excess = E.tolerance_ok(got, ref, ATOL, RTOL)
    assert ok, "layer %d (%s): max_abs %.3g max_rel %.3g excess %.3g" % (
        layer, fmt, mabs, mrel, excess)


def _run(name, layers=(0,)):
    print("workload", name, flush=True)
    spec = W.spec(name)
    case = DecodeCase(spec, device="cuda:0", poison=True)
    seqs = _sample(case.lens)
    try:
        for layer in layers:
            print("  layer", layer, case.fmt(layer), flush=True)
            case.setup_layer(layer)
            _check_layer(case, layer, seqs)
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
    # the 32-layer workload: an fp16 first layer, INT8 middle layers and an
    # fp16 last layer, each over the shared-prefix layout with COW copies
    _run("c5_prefix_mixed", layers=(0, 1, 15, 31))


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
