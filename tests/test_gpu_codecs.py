"""Exhaustive GPU codec parity: every finite fp16 value through kvq_cache_write.

The device encoders (INT8 / INT4 absmax per group, INT8 with static
per-channel scales, E4M3 and E5M2 with static per-head or dynamic per-group
scales) are bit-level code paths of their own.  Here each one quantizes every
finite fp16 input -- both zeros, subnormals, the largest values -- under
scales that reach its rounding ties, its saturation and its zero-scale case,
and the stored bytes and scales are compared bit for bit with the oracle's
codes for the same inputs ("KV Cache优化实战" s2.3 / s3.3: absmax symmetric
INT8 per group with a stored scale, or per channel; FP8 as in xpshop.cn
article 312 s3).

Per-group formats: every group is [a, x_1 .. x_{G-1}] with |x_i| <= |a|, so
its absmax, and hence its scale, is a, and the x_i run over every finite fp16
value of magnitude at most |a| (as the oracle's own INT8 pin does on the CPU).
"""
import numpy as np
import pytest
import torch

from oracle import expected as E
from paged_quantized_kv_cache_amd import kvq
from paged_quantized_kv_cache_amd.harness import int4_tile_offsets, tile_offsets

pytestmark = pytest.mark.gpu

BS = 16
ANCHORS = [1.0, -0.1, 3.5, -17.25, 65504.0, 6.1035e-05, -5.96e-08, 0.333, 1000.0, 0.0]


def _finite_f16():
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    return x[np.isfinite(x)]


def _anchored_tokens(G, D, hkv, anchors=ANCHORS):
    """fp16 [T][hkv][D]: groups [a, x...] covering every finite |x| <= |a|."""
    xs_all = _finite_f16()
    groups = []
    for a in anchors:
        a16 = np.float16(a)
        xs = xs_all[np.abs(xs_all.astype(np.float64)) <= abs(float(a16))]
        n = -(-xs.size // (G - 1))
        body = np.zeros(n * (G - 1), np.float16)
        body[:xs.size] = xs
        g = np.concatenate([np.full((n, 1), a16, np.float16), body.reshape(n, G - 1)], 1)
        groups.append(g)
    g = np.concatenate(groups, 0)
    per_tok = hkv * (D // G)
    pad = (-g.shape[0]) % per_tok
    if pad:
        g = np.concatenate([g, np.zeros((pad, G), np.float16)], 0)
    return g.reshape(-1, hkv, D)


def _broadcast_tokens(D, hkv):
    """fp16 [T][hkv][D]: token t holds the t-th finite fp16 value everywhere."""
    xs = _finite_f16()
    return np.ascontiguousarray(np.broadcast_to(xs[:, None, None], (xs.size, hkv, D)))


def _write(x, fmt, G, static=None):
    """Write x as both K and V (slots 0..T-1) and read back codes and scales."""
    T, hkv, D = x.shape
    nb = -(-T // BS)
    kp, vp, ks, vs = kvq.alloc_pools(nb, hkv, BS, D, fmt, G, device="cuda")
    kp.fill_(0x5A)
    vp.fill_(0xA5)
    if static is not None:
        ks.copy_(torch.from_numpy(static))
        vs.copy_(torch.from_numpy(static))
    elif ks is not None:
        ks.fill_(float("nan"))
        vs.fill_(float("nan"))
    xt = torch.from_numpy(x).cuda()
    slots = torch.arange(T, dtype=torch.int64, device="cuda")
    kvq.kvq_cache_write(xt, xt.clone(), slots, kp, vp, ks, vs, fmt, G)
    torch.cuda.synchronize()
    blk = np.arange(T) // BS
    off = np.arange(T) % BS
    h = np.arange(hkv)[None, :, None]
    out = {}
    for name, pool in (("k", kp), ("v", vp)):
        flat = pool.view(torch.uint8).reshape(nb, hkv, -1).cpu().numpy()
        if fmt == "int4":
            (koff, khi), (voff, vhi) = int4_tile_offsets(BS, D)
            offs, hi = (koff, khi) if name == "k" else (voff, vhi)
            byte = flat[blk[:, None, None], h, offs[off][:, None, :]]
            sh = np.where(hi[off], 4, 0)[:, None, :]
            out[name] = (((byte >> sh) & 0xF).astype(np.int16) - 8).astype(np.int8)
        else:
            koff, voff = tile_offsets(BS, D, 1)
            offs = (koff if name == "k" else voff)[..., 0]
            byte = flat[blk[:, None, None], h, offs[off][:, None, :]]
            out[name] = (byte ^ np.uint8(0x80)).view(np.int8) if fmt == "int8" else byte
    if kvq.scale_mode(fmt, G) == "group":    # [block][head][slot][group]
        out["k_scale"] = ks.cpu().numpy()[blk, :, off, :]
        out["v_scale"] = vs.cpu().numpy()[blk, :, off, :]
    return out


def _compare(x, fmt, G, static=None):
    got = _write(x, fmt, G, static)
    ref = E.quantize(x, fmt, G, static)
    codes = ref.codes.view(np.uint8) if fmt in ("fp8", "e5m2") else ref.codes
    for name in ("k", "v"):
        bad = np.nonzero(got[name] != codes)
        assert bad[0].size == 0, "%s %s G=%d: %d codes differ, first at %s: x=%r got %r want %r" % (
            fmt, name, G, bad[0].size, tuple(int(b[0]) for b in bad),
            float(x[tuple(b[0] for b in bad)]), got[name][tuple(b[0] for b in bad)],
            codes[tuple(b[0] for b in bad)])
    if ref.scales is not None:
        for name in ("k_scale", "v_scale"):
            assert np.array_equal(got[name].view(np.uint32), ref.scales.view(np.uint32)), \
                "%s %s G=%d: scales differ" % (fmt, name, G)


@pytest.mark.parametrize("fmt,G,D", [("int8", 64, 64), ("int8", 64, 128), ("int8", 128, 128),
                                     ("fp8", 64, 64), ("fp8", 64, 128), ("fp8", 128, 128),
                                     ("int4", 64, 128), ("int4", 128, 128)])
def test_group_codecs_every_fp16_value(fmt, G, D, gpu):
    print("codec", fmt, G, D, flush=True)
    _compare(_anchored_tokens(G, D, 2), fmt, G)


# static per-channel INT8 scales: zero (code 0), tiny (everything saturates),
# powers of two (exact ties of x / s), and ordinary values
CHANNEL_SCALES = np.array([0.0, 1e-30, 2.0 ** -24, 2.0 ** -8, 1.0 / 127, 0.5, 1.0, 3.7,
                           1000.0, 65504.0 / 127, 2.0 ** -14, 0.0123],
                          np.float32)


@pytest.mark.parametrize("D", [64, 128])
def test_int8_channel_codec_every_fp16_value(D, gpu):
    print("codec int8 per channel", D, flush=True)
    s = np.resize(CHANNEL_SCALES, D)[None, :].repeat(2, 0).astype(np.float32)   # [Hkv][D]
    s[1] = s[1][::-1]
    _compare(_broadcast_tokens(D, 2), "int8", 0, s)


# static per-head FP8 scales: 1 (the fp16 value itself), 2^-8, one that
# sends most values into saturation, a non-power-of-two, and zero (code 0)
HEAD_SCALES = {"fp8": [1.0, 2.0 ** -8, 2.0 ** -4, 0.37, 0.0],
               "e5m2": [1.0, 2.0 ** -8, 1e-3, 0.37, 0.0]}


@pytest.mark.parametrize("fmt", ["fp8", "e5m2"])
@pytest.mark.parametrize("D", [64, 128])
def test_fp8_static_codec_every_fp16_value(fmt, D, gpu):
    print("codec", fmt, "per head", D, flush=True)
    s = np.array(HEAD_SCALES[fmt], np.float32)
    _compare(_broadcast_tokens(D, s.size), fmt, 0, s)
