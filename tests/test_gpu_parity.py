"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Cache writes must match the oracle bit for bit (INT8 codes and fp32 scales,
E4M3 bytes, fp16 copies), read back through the block tables.  Decode
attention must satisfy |gpu - oracle| <= 2e-3 + 1e-3 * |oracle| elementwise,
the oracle attending in fp64 over contiguous dequantized K/V.

Small cases run the whole batch through the oracle; they span several
16-token tiles, ragged tails and forced splits.  Full-size workloads are
checked on every sequence (test_gpu_fullsize.py).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import expected as E
from paged_quantized_kv_cache_amd import kvq
from paged_quantized_kv_cache_amd import workloads as W
from paged_quantized_kv_cache_amd.harness import DecodeCase, tile_offsets

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-3


def small(name, **kw):
    return W.spec(name, **kw)


SMALL_CASES = {
    "c1_tiny": small("c1_tiny"),
    "mha_int8_g128": small("c2_mha", B=6, Hq=4, Hkv=4, lens="uniform",
                           lens_args=(1, 300)),
    "gqa_int8_g64_outliers": small("c3_gqa", B=5, Hq=8, Hkv=2, lens="fixed",
                                   lens_args=(1, 17, 100, 257, 700)),
    "gqa_fp16": small("c3_gqa_fp16", B=5, Hq=8, Hkv=2, lens="fixed",
                      lens_args=(3, 16, 31, 200, 513)),
    "fp8_bs16": small("c4_long_bs16", B=3, Hq=8, Hkv=2, lens="fixed",
                      lens_args=(1, 150, 1100)),
    "fp8_bs32": small("c4_long_bs32", B=3, Hq=8, Hkv=2, lens="fixed",
                      lens_args=(15, 33, 1100)),
    "int8_bs32_g128_r8": small("c2_mha", B=4, Hq=16, Hkv=2, BS=32, lens="fixed",
                               lens_args=(31, 32, 65, 400)),
    "int8_d64_bs32_r16": small("c1_tiny", B=3, Hq=16, Hkv=1, BS=32, pool_blocks=0,
                               lens="fixed", lens_args=(2, 40, 97)),
    "fp16_d64_mqa": small("c1_tiny", fmt="fp16", G=0, B=3, pool_blocks=0,
                          lens="fixed", lens_args=(7, 64, 90)),
    # format variants: E5M2, FP8 with dynamic per-token / per-group scales,
    # INT8 with static per-channel scales
    "e5m2_bs16": small("c4_long_bs16", fmt="e5m2", B=3, Hq=8, Hkv=2, lens="fixed",
                       lens_args=(1, 150, 1100)),
    "e5m2_d64_bs32": small("c1_tiny", fmt="e5m2", G=0, B=3, Hq=16, Hkv=1, BS=32,
                           pool_blocks=0, lens="fixed", lens_args=(2, 40, 97)),
    "fp8_token_g128": small("c3_gqa", fmt="fp8", G=128, B=5, Hq=8, Hkv=2, lens="fixed",
                            lens_args=(1, 17, 100, 257, 700)),
    "fp8_g64_bs32": small("c3_gqa", fmt="fp8", G=64, BS=32, B=4, Hq=16, Hkv=2,
                          lens="fixed", lens_args=(31, 32, 65, 400)),
    "fp8_d64_token": small("c1_tiny", fmt="fp8", G=64, B=3, pool_blocks=0,
                           lens="fixed", lens_args=(7, 64, 90)),
    "int8_channel": small("c3_gqa", fmt="int8", G=0, B=5, Hq=8, Hkv=2, lens="fixed",
                          lens_args=(1, 17, 100, 257, 700)),
    "int8_channel_d64_bs32": small("c1_tiny", fmt="int8", G=0, B=3, Hq=16, Hkv=1, BS=32,
                                   pool_blocks=0, lens="fixed", lens_args=(2, 40, 97)),
    # INT4 (two codes per byte)
    "int4_g64_outliers": small("c3_gqa", fmt="int4", G=64, B=5, Hq=8, Hkv=2, lens="fixed",
                               lens_args=(1, 17, 100, 257, 700)),
    "int4_g128_bs32_r8": small("c2_mha", fmt="int4", G=128, B=4, Hq=16, Hkv=2, BS=32,
                               lens="fixed", lens_args=(31, 32, 65, 400)),
}


def _host(t):
    return t.detach().cpu().numpy()


def _expected(case: DecodeCase, layer: int, seqs=None):
    """Oracle codes per unique token and attention output per sequence."""
    s, fmt = case.spec, case.fmt(layer)
    d = case.data[layer]
    k16, v16 = _host(d.k), _host(d.v)
    sk = sv = None
    if kvq.scale_mode(fmt, s.G) in ("head", "channel"):   # static scales
        sk = _host(case.pools[layer].k_scale)
        sv = _host(case.pools[layer].v_scale)
    seqs = list(range(s.B)) if seqs is None else list(seqs)
    ids = np.unique(np.concatenate([case.layout.seq_tokens[b] for b in seqs]))
    remap = np.full(case.layout.n_unique, -1, np.int64)
    remap[ids] = np.arange(ids.size)
    kq = E.quantize(k16[ids], fmt, s.G, sk)
    vq = E.quantize(v16[ids], fmt, s.G, sv)
    toks = [remap[case.layout.seq_tokens[b]] for b in seqs]
    q = _host(d.q)[seqs]
    out = E.attention(q, kq, vq, toks)
    return kq, vq, toks, out


def _check_codes(case, layer, kq, vq, toks, seqs):
    fmt = case.fmt(layer)
    got = case.gather_codes(layer, seqs)
    for i, b in enumerate(seqs):
        t = toks[i]
        ek, ev = kq.codes[t], vq.codes[t]
        gk, gv = got[i]["k"], got[i]["v"]
        if fmt == "fp16":
            gk, gv = gk.view(np.uint16), gv.view(np.uint16)
        assert np.array_equal(gk, ek), "K codes differ (seq %d)" % b
        assert np.array_equal(gv, ev), "V codes differ (seq %d)" % b
        if kq.scales is not None:
            assert np.array_equal(got[i]["k_scale"], kq.scales[t]), "K scales (seq %d)" % b
            assert np.array_equal(got[i]["v_scale"], vq.scales[t]), "V scales (seq %d)" % b


def _check_out(got, ref, what):
    ok, mabs, mrel, excess = E.tolerance_ok(got, ref, ATOL, RTOL)
    assert ok, "%s: max_abs %.3g max_rel %.3g excess %.3g" % (what, mabs, mrel, excess)
    return mabs


def _build(spec, gpu, **kw):
    case = DecodeCase(spec, device=gpu, gen_device="cpu", **kw)
    case.setup_layer(0)
    torch.cuda.synchronize()
    return case


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_cache_write_bit_exact(name, gpu):
    spec = SMALL_CASES[name]
    print("case", name, flush=True)
    case = _build(spec, gpu)
    seqs = list(range(spec.B))
    kq, vq, toks, _ = _expected(case, 0, seqs)
    _check_codes(case, 0, kq, vq, toks, seqs)


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_decode_within_tolerance(name, gpu):
    spec = SMALL_CASES[name]
    print("case", name, flush=True)
    case = _build(spec, gpu)
    _, _, _, ref = _expected(case, 0)
    outs = {}
    for split in (0, 16, 64, 1024):
        ws = case.workspace(split)
        got = _host(case.decode(0, split_tokens=split, workspace=ws)).astype(np.float64)
        _check_out(got, ref, "%s split=%d" % (name, split))
        outs[split] = got
    # splitting changes only rounding: the variants agree within twice the bound
    for split in (16, 64, 1024):
        assert np.all(np.abs(outs[0] - outs[split]) <= 2 * (ATOL + RTOL * np.abs(ref)))


def test_decode_repeat_reuses_workspace(gpu):
    spec = SMALL_CASES["gqa_int8_g64_outliers"]
    case = _build(spec, gpu)
    ws = case.workspace(16)
    a = case.decode(0, split_tokens=16, workspace=ws).clone()
    for _ in range(3):
        b = case.decode(0, split_tokens=16, workspace=ws)
        assert torch.equal(a, b)  # deterministic; stale workspace contents unused


def test_results_independent_of_physical_placement(gpu):
    spec = SMALL_CASES["gqa_int8_g64_outliers"]
    outs = []
    for layout_seed in (None, 1, 2):
        case = DecodeCase(spec, device=gpu, gen_device="cpu", layout_seed=layout_seed)
        case.setup_layer(0)
        for split in (0, 32):
            outs.append((split, _host(case.decode(0, split_tokens=split))))
    base = {s: o for s, o in outs[:2]}
    for s, o in outs:
        assert np.array_equal(o.view(np.uint16), base[s].view(np.uint16))


def _prefix_spec(fmt="int8"):
    return W.spec("c5_prefix_mixed", B=6, Hq=8, Hkv=2, layers=1,
                  layer_fmts=(fmt,), fmt=fmt, shared_prefix=64,
                  lens_args=(5, 120), fork_pairs=2)


@pytest.mark.parametrize("fmt", ["int8", "fp16"])
def test_shared_prefix_and_cow(fmt, gpu):
    spec = _prefix_spec(fmt)
    case = _build(spec, gpu)
    L = case.layout
    assert L.cow_pairs.shape[0] == spec.fork_pairs
    seqs = list(range(spec.B))
    kq, vq, toks, ref = _expected(case, 0, seqs)
    _check_codes(case, 0, kq, vq, toks, seqs)          # incl. the forked partners
    got = _host(case.decode(0)).astype(np.float64)
    _check_out(got, ref, "shared prefix %s" % fmt)

    # the same logical data held in private copies decodes bit-identically
    priv_spec = W.spec("c5_prefix_mixed", B=6, Hq=8, Hkv=2, layers=1,
                       layer_fmts=(fmt,), fmt=fmt, shared_prefix=0, fork_pairs=0,
                       lens="fixed", lens_args=tuple(int(x) for x in case.lens))
    priv = DecodeCase(priv_spec, device=gpu, gen_device="cpu")
    d = case.data[0]
    ids = np.concatenate(L.seq_tokens)       # private token j <- shared token ids[j]
    order = np.concatenate(priv.layout.seq_tokens)
    k = torch.empty((ids.size,) + tuple(d.k.shape[1:]), dtype=d.k.dtype)
    v = torch.empty_like(k)
    k[torch.from_numpy(order)] = d.k[torch.from_numpy(ids)]
    v[torch.from_numpy(order)] = d.v[torch.from_numpy(ids)]
    priv.data[0] = W.LayerData(k=k, v=v, q=d.q)
    priv.alloc(0)
    priv.prefill(0)
    priv.append(0)
    got_priv = _host(priv.decode(0))
    got_shared = _host(case.decode(0))
    assert np.array_equal(got_priv.view(np.uint16), got_shared.view(np.uint16))
    # the shared-block hint bit changes only the cache policy of the loads
    assert (case.layout.block_tables_hinted >> 30 == 1).any()
    plain = case.block_tables & 0x3FFFFFFF
    case.block_tables, hinted = plain, case.block_tables
    got_plain = _host(case.decode(0))
    case.block_tables = hinted
    assert np.array_equal(got_plain.view(np.uint16), got_shared.view(np.uint16))


def test_cow_leaves_other_sharer_untouched(gpu):
    """The writer gets a private copy of the shared partial block; the slots
    filled before the append stay unchanged for the other sharer, which then
    appends into the original block in place."""
    spec = _prefix_spec("int8")
    case = DecodeCase(spec, device=gpu, gen_device="cpu")
    case.gen(0)
    case.alloc(0)
    case.prefill(0)
    p = case.pools[0]
    pairs = case.layout.cow_pairs
    koff, voff = tile_offsets(spec.BS, spec.D, 1)

    def slots(pool, blk, offs, fill):
        flat = pool[int(blk)].view(torch.uint8).reshape(spec.Hkv, -1).cpu().numpy()
        return flat[:, offs[:fill].ravel()]

    fills = [(int(case.lens[2 * i]) - 1) % spec.BS for i in range(pairs.shape[0])]
    before = [(slots(p.k_pool, s_, koff, f), slots(p.v_pool, s_, voff, f),
               p.k_scale[int(s_), :, :f].clone(), p.v_scale[int(s_), :, :f].clone())
              for (s_, _), f in zip(pairs, fills)]
    case.cow(0)
    case.append(0)
    torch.cuda.synchronize()
    for (src, dst), f, bef in zip(pairs, fills, before):
        assert f > 0
        for blk in (src, dst):
            assert np.array_equal(slots(p.k_pool, blk, koff, f), bef[0])
            assert np.array_equal(slots(p.v_pool, blk, voff, f), bef[1])
            assert torch.equal(p.k_scale[int(blk), :, :f], bef[2])
            assert torch.equal(p.v_scale[int(blk), :, :f], bef[3])
    # the writers' tables point at the copies, the partners' at the originals
    bt = case.layout.block_tables
    for i in range(pairs.shape[0]):
        last = (int(case.lens[2 * i]) - 1) // spec.BS
        assert bt[2 * i, last] == pairs[i, 1] and bt[2 * i + 1, last] == pairs[i, 0]


def test_constant_keys_give_mean_of_values(gpu):
    # closed form: identical dequantized keys -> softmax is uniform
    spec = W.spec("c3_gqa", B=2, Hq=8, Hkv=2, lens="fixed", lens_args=(37, 300))
    case = DecodeCase(spec, device=gpu, gen_device="cpu")
    d = case.gen(0)
    d.k[:] = d.k[0:1]
    case.alloc(0)
    case.prefill(0)
    case.append(0)
    kq, vq, toks, ref = _expected(case, 0)
    got = _host(case.decode(0, split_tokens=64)).astype(np.float64)
    _check_out(got, ref, "constant keys")
    for b, t in enumerate(toks):
        mean = vq.deq[t].mean(0)                      # [Hkv][D]
        for g in range(spec.Hq):
            assert np.allclose(got[b, g], mean[g // spec.r], atol=ATOL, rtol=RTOL)


@pytest.mark.parametrize("fmt,G", [("int8", 64), ("int4", 64), ("fp8", 128), ("fp16", 0),
                                   ("int8", 0)])
def test_extreme_magnitudes_stay_finite(fmt, G, gpu):
    # K/V near the top of the fp16 range: group scales up to ~330 (INT8) or
    # ~6000 (INT4) multiply P^T entries in fp16, and scores differ by
    # thousands (a hard maximum); the output must still match the oracle
    spec = W.spec("c3_gqa", fmt=fmt, G=G, B=3, Hq=8, Hkv=2, lens="fixed",
                  lens_args=(40, 300, 700))
    print("case", fmt, G, flush=True)
    case = DecodeCase(spec, device=gpu, gen_device="cpu")
    d = case.gen(0)
    for x, f in ((d.k, 3000.0), (d.v, 12000.0)):
        x.copy_((x.float() * f).clamp(-65000, 65000).to(torch.float16))
    case.alloc(0)
    case.prefill(0)
    case.append(0)
    _, _, _, ref = _expected(case, 0)
    for split in (0, 64):
        got = _host(case.decode(0, split_tokens=split)).astype(np.float64)
        assert np.isfinite(got).all()
        _check_out(got, ref, "%s g%d x-large split=%d" % (fmt, G, split))


@pytest.mark.parametrize("B,hi", [(1500, 200), (9000, 40)])
def test_large_batches_planned_by_the_plan_kernel(B, hi, gpu):
    """More than 1024 sequences: the balanced runs come from plan_kernel (one
    workgroup scanning the lengths; past 8192 sequences its prefix sums stay
    in global memory instead of LDS), for decode and for short chunks."""
    # N(0,1) data: the test is about the plan; C1's x8 outlier channels on
    # Q, K and V at this scale put ~1e-5 of the outputs past the bound in
    # every partition (fp16 P operands times |V| up to ~30, see the parity
    # notes of the design), while the four-sequence C1 workload stays within
    spec = small("c2_mha", B=B, Hq=8, Hkv=2, D=64, G=64, lens="uniform",
                 lens_args=(1, hi))
    print("batch", B, flush=True)
    case = _build(spec, gpu)
    _, _, _, ref = _expected(case, 0)
    got = _host(case.decode(0)).astype(np.float64)
    _check_out(got, ref, "B=%d decode" % B)
    # the same batch as short chunks of up to 16 / r = 4 tokens (some empty)
    n = np.minimum(case.lens, np.arange(B) % 5)
    q = case.chunk_queries(n)
    pre = case.prefill_attention(0, n, q).float().cpu().numpy()
    kq, vq, toks, _ = _expected(case, 0)
    ref_p = E.prefill(q.cpu().numpy(), kq, vq, toks, n)
    _check_out(pre, ref_p, "B=%d short chunks" % B)


def test_validation_flag_checks_device_metadata(gpu, monkeypatch):
    """KVQ_VALIDATE=1: the binding checks tables and lengths on host copies
    before the launch; a corrupt entry is named instead of silently clamped."""
    spec = SMALL_CASES["gqa_int8_g64_outliers"]
    case = _build(spec, gpu)
    monkeypatch.setenv("KVQ_VALIDATE", "1")
    _, _, _, ref = _expected(case, 0)
    _check_out(_host(case.decode(0)).astype(np.float64), ref, "validated decode")
    bt = case.block_tables.clone()
    bt[3, 2] = case.layout.num_blocks + 5            # sequence 3 uses 7 blocks
    case.block_tables, good = bt, case.block_tables
    with pytest.raises(ValueError, match="sequence 3: table entry 2"):
        case.decode(0)
    case.block_tables = good


def test_one_workspace_reused_by_calls_of_different_shapes(gpu):
    """A workspace's contents on entry never matter: back-to-back decode
    calls of different batches and head shapes (one through the plan
    kernel, over 1024 sequences) and short-chunk and virtual-sequence
    prefill calls share one workspace, each finding the previous call's
    plan and partials in it; each result equals the same call on a fresh
    workspace bit for bit and stays within tolerance of the oracle."""
    big = small("c2_mha", B=1100, Hq=8, Hkv=2, D=64, G=64, lens="uniform", lens_args=(1, 90))
    names = ["gqa_int8_g64_outliers", "mha_int8_g128", "c1_tiny", "fp8_bs32", "gqa_fp16"]
    cases = [_build(SMALL_CASES[n], gpu) for n in names] + [_build(big, gpu)]
    calls = []
    for case in cases:
        calls.append(("decode", case, None))
    r4 = cases[0]                                   # Hq 8 / Hkv 2: r = 4
    calls.append(("prefill", r4, np.minimum(r4.lens, [4, 1, 3, 0, 2])))      # short chunks
    calls.append(("prefill", r4, np.minimum(r4.lens, [37, 9, 40, 20, 33])))  # virtual sequences
    need = 0
    for kind, case, n in calls:
        s = case.spec
        if kind == "decode":
            need = max(need, kvq.kvq_decode_workspace_size(s.B, s.Hq, s.Hkv, s.D, s.BS,
                                                           case.max_context_len, 0))
        else:
            need = max(need, kvq.kvq_prefill_workspace_size(s.B, s.Hq, s.Hkv, s.D, s.BS,
                                                            case.max_context_len,
                                                            int(n.max()), "split"))
    shared = kvq.alloc_workspace(need, gpu)
    for kind, case, n in calls:
        print(kind, case.spec.name, case.spec.B, flush=True)
        if kind == "decode":
            got = case.decode(0, workspace=shared)
            fresh = case.decode(0, workspace=case.workspace(0))
            _, _, _, ref = _expected(case, 0)
        else:
            q = case.chunk_queries(n)
            got = case.prefill_attention(0, n, q, workspace=shared, split_mode="split")
            fresh = case.prefill_attention(0, n, q, split_mode="split")
            kq, vq, toks, _ = _expected(case, 0)
            ref = E.prefill(q.cpu().numpy(), kq, vq, toks, n)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), fresh.view(torch.int16)), kind
        _check_out(_host(got).astype(np.float64), ref, "%s %s" % (kind, case.spec.name))
