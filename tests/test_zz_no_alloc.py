"""kvq_paged_decode_noalloc: the decode call that allocates nothing.

Its output must equal kvq_paged_decode's (same kernels, same plan, the
library's static scratch instead of a caller workspace) bit for bit, and
both must agree with the oracle, on two calls in a row -- the second over a
smaller batch, so the scratch holds the first call's plan and partials when
the second starts.  A call whose plan needs more than the static scratch is
refused before any launch.
"""
import numpy as np
import pytest
import torch

from oracle import expected as E
from paged_quantized_kv_cache_amd import kvq
from paged_quantized_kv_cache_amd import workloads as W
from paged_quantized_kv_cache_amd.harness import DecodeCase

pytestmark = pytest.mark.gpu


def _case(B, seed, gpu, **kw):
    spec = W.spec("c3_gqa", B=B, seed=seed, **kw)
    case = DecodeCase(spec, device=gpu, gen_device="cpu")
    case.setup_layer(0)
    return case


def _noalloc(case, split=0):
    p, s = case.pools[0], case.spec
    q = case.data[0].q.to(case.device)
    out = torch.full_like(q, float("nan"))
    kvq.kvq_paged_decode_noalloc(q, p.k_pool, p.v_pool, p.k_scale, p.v_scale,
                                 case.block_tables, case.context_lens, case.max_context_len,
                                 p.fmt, out, s.G, split_tokens=split)
    return out


def _oracle(case):
    s, d = case.spec, case.data[0]
    kq = E.quantize(d.k.numpy(), s.fmt, s.G)
    vq = E.quantize(d.v.numpy(), s.fmt, s.G)
    return E.attention(d.q.numpy(), kq, vq, case.layout.seq_tokens)


def test_noalloc_matches_decode_on_two_calls_second_smaller(gpu):
    big = _case(192, 3, gpu)                       # lognormal lengths up to 8192
    small = _case(9, 4, gpu, lens="fixed",
                  lens_args=(1, 15, 16, 17, 300, 1000, 2049, 33, 4000))
    for case, split in ((big, 0), (small, 0), (small, 64)):
        print("noalloc B=%d split=%d" % (case.spec.B, split), flush=True)
        got = _noalloc(case, split)
        ref = case.decode(0, split_tokens=split, workspace=case.workspace(split))
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), \
            "noalloc differs from kvq_paged_decode (B=%d split=%d)" % (case.spec.B, split)
        ok, mabs, mrel, _ = E.tolerance_ok(got.float().cpu().numpy(), _oracle(case))
        assert ok, "max_abs %.3g max_rel %.3g" % (mabs, mrel)


def test_noalloc_refuses_plans_beyond_its_scratch(gpu):
    case = _case(64, 5, gpu)
    # 16-token spans over 64 sequences x 8 KV heads: ~10^5 partials of 2 KiB
    with pytest.raises(kvq.KvqError) as e:
        _noalloc(case, split=16)
    assert e.value.status == -3                      # KVQ_ERR_WORKSPACE
    # the refused call launched nothing; the next one still works
    got = _noalloc(case, 0)
    ref = case.decode(0)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
