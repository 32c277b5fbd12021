#!/usr/bin/env python3
"""Benchmark of the paged INT8 GQA decode hot path on one MI355X.

One step = the whole hot path for one batch: the quantizing cache write of
one new token per sequence (kvq_cache_write) followed by paged decode
attention over the INT8 pool (kvq_paged_decode), for every layer of the
workload.  Inputs are seeded synthetic data resident in HBM before timing.

Prints one JSON line.  `value` is seq-steps/s (sequences x steps / second).
`roofline` prices the decode kernel (the dominant one) against MI355X HBM
bandwidth using algorithmic bytes (every valid cached K/V code and scale
once, plus q, out, table entries and lengths) over its event-timed duration.
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload
(one step's work: quantize the appended tokens, fp64 attention over the
dequantized cache).  With the default workload the line also carries
`workloads` (the other decode configurations -- the MHA layer, the long
FP8 contexts with 16- and 32-token blocks, the 32-layer prefix-sharing
step -- timed the same way over fewer steps), `cache_write_us` (the
append's event time) and `reconstruction_error` (the format's error
against the fp16 data, from the oracle).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged INT8 GQA decode-attn seq-steps/s + achieved HBM GB/s (% of MI355X peak)"
HBM_PEAK_GBPS = 8000.0
DEFAULT_WORKLOAD = "c3_gqa"


# the kernels of the default workload's decode call (plan, the INT8 g64
# head_dim-128 16-token-block tile walk with one column group, the
# 128-dim merge; substrings of their mangled names): traffic counters taken
# on them stay valid while other kernels and instances change
DECODE_KERNELS = ("plan_kernel", "merge_runs_kernelILi128E",
                  "paged_decode_kernelILi1ELi128ELi16ELi2ELi1E")


def kernel_hash() -> str:
    """Identity of the decode call's device code the counters were taken on."""
    from paged_quantized_kv_cache_amd import build as B
    return B.device_code_hash(kernels=DECODE_KERNELS)


def load_traffic(workload: str):
    """HBM bytes per decode call from committed rocprofv3 counter runs, if
    they were taken on the device code now built; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_hash") != kernel_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(case, spec, max_seqs: int, layer: int = 0, min_seconds: float = 10.0):
    """Time the oracle (as it stands) doing one decode step's work for the
    first `max_seqs` sequences of one layer, like the GPU step: quantize each
    sequence's appended token, then fp64 attention over its cached K/V.  The
    cache itself is state, as the GPU's pool is: every cached token is
    quantized, dequantized and laid out contiguously per sequence (the form
    the oracle reads) once, before timing.  Median over at least three
    passes and about `min_seconds` of work, on all the oracle's threads and,
    for the first 16 sequences, on one (three passes)."""
    import numpy as np
    import torch

    import oracle
    from oracle import expected as E
    from paged_quantized_kv_cache_amd import kvq

    nseq = min(max_seqs, spec.B)
    d = case.data[layer] if case.data[layer] is not None else case.gen(layer)
    fmt = spec.fmt_of_layer(layer)
    sk = sv = None
    if kvq.scale_mode(fmt, spec.G) in ("head", "channel"):   # static scales
        sk = case.pools[layer].k_scale.cpu().numpy()
        sv = case.pools[layer].v_scale.cpu().numpy()
    toks = [np.asarray(case.layout.seq_tokens[b], np.int64) for b in range(nseq)]
    lens = np.array([t.size for t in toks], np.int64)
    idx = np.concatenate(toks)
    ids = np.unique(idx)
    remap = np.full(case.layout.n_unique, -1, np.int64)
    remap[ids] = np.arange(ids.size)
    tdev = torch.from_numpy(ids).to(d.k.device)
    k16 = d.k.index_select(0, tdev).cpu().numpy()
    v16 = d.v.index_select(0, tdev).cpu().numpy()
    q = d.q[:nseq].cpu().numpy()
    # state: the dequantized cache, contiguous per sequence
    K = E.quantize(k16, fmt, spec.G, sk).deq[remap[idx]]
    V = E.quantize(v16, fmt, spec.G, sv).deq[remap[idx]]
    last = np.cumsum(lens) - 1                       # each sequence's appended token
    ka, va = k16[remap[idx[last]]], v16[remap[idx[last]]]

    def step(n):
        kq = E.quantize(ka[:n], fmt, spec.G, sk)     # the appended tokens
        vq = E.quantize(va[:n], fmt, spec.G, sv)
        K[last[:n]] = kq.deq
        V[last[:n]] = vq.deq
        oracle.decode_attention(q[:n], K[:last[n - 1] + 1], V[:last[n - 1] + 1], lens[:n])

    times = []
    while len(times) < 3 or (sum(times) < min_seconds and len(times) < 60):
        t0 = time.perf_counter()
        step(nseq)
        times.append(time.perf_counter() - t0)
    passes = len(times)
    cores = oracle.num_threads()
    n1 = min(16, nseq)
    oracle.set_num_threads(1)
    try:
        t1 = []
        for _ in range(3):
            t0 = time.perf_counter()
            step(n1)
            t1.append(time.perf_counter() - t0)
    finally:
        oracle.set_num_threads(cores)
    med = float(np.median(times))
    return {
        "value": nseq / med,
        "unit": "seq-steps/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "first %d of %d sequences of layer %d (%d cached tokens): quantize the "
                  "appended tokens, fp64 attention over the dequantized cache (built once, "
                  "untimed); median of %d passes, %.2f s each"
                  % (nseq, spec.B, layer, int(lens.sum()), passes, med),
        "single_thread_value": n1 / float(np.median(t1)),
        "cpu_model": cpu_model(),
    }


def recon_error_summary(case, spec, layer: int = 0, ntok: int = 4096, nseq: int = 4) -> dict:
    """Reconstruction error of the layer's format on its own data, from the
    oracle (reported beside the parity check, not gated): K / V max-abs and
    RMSE of x - x_hat over the first `ntok` tokens, and the decode output of
    the first `nseq` sequences over the original fp16 K/V against the output
    over the dequantized K/V (both fp64)."""
    import numpy as np
    import torch

    import oracle
    from oracle import expected as E
    from paged_quantized_kv_cache_amd import kvq

    d = case.data[layer] if case.data[layer] is not None else case.gen(layer)
    fmt = spec.fmt_of_layer(layer)
    st = {}
    if kvq.scale_mode(fmt, spec.G) in ("head", "channel"):
        st = {"k": case.pools[layer].k_scale.cpu().numpy(),
              "v": case.pools[layer].v_scale.cpu().numpy()}
    out = {"format": fmt, "group_size": spec.G, "tokens": ntok}
    for which, x in (("k", d.k), ("v", d.v)):
        x16 = x[:ntok].cpu().numpy()
        err = E.quantize(x16, fmt, spec.G, st.get(which)).deq - oracle.f16_to_f64(x16)
        out[which + "_max_abs"] = float(np.abs(err).max())
        out[which + "_rmse"] = float(np.sqrt(np.mean(err ** 2)))
    toks = [np.asarray(case.layout.seq_tokens[b], np.int64) for b in range(nseq)]
    ids = np.unique(np.concatenate(toks))
    remap = np.full(case.layout.n_unique, -1, np.int64)
    remap[ids] = np.arange(ids.size)
    tdev = torch.from_numpy(ids).to(d.k.device)
    k16 = d.k.index_select(0, tdev).cpu().numpy()
    v16 = d.v.index_select(0, tdev).cpu().numpy()
    q = d.q[:nseq].cpu().numpy()
    lt = [remap[t] for t in toks]
    ref = E.attention(q, E.quantize(k16, "fp16"), E.quantize(v16, "fp16"), lt)
    got = E.attention(q, E.quantize(k16, fmt, spec.G, st.get("k")),
                      E.quantize(v16, fmt, spec.G, st.get("v")), lt)
    out["attn_seqs"] = nseq
    out["attn_max_abs"] = float(np.abs(got - ref).max())
    out["attn_rel"] = float(np.abs(got - ref).max() / np.abs(ref).max())
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def swap_bandwidth(case, spec, reps: int = 3) -> dict:
    """Swap every block layer 0 uses out to a pinned host buffer and back in
    place; bytes of the swap slots over event time, best of ``reps``."""
    import torch
    from paged_quantized_kv_cache_amd import kvq
    p = case.pools[0]
    blocks = sorted(int(b) for b in case.layout.used_blocks)
    slot = kvq.kvq_swap_block_bytes(spec.Hkv, spec.D, spec.BS, p.fmt, spec.G)
    buf = torch.empty(len(blocks) * slot, dtype=torch.uint8, pin_memory=True)
    pairs = torch.tensor([[b, i] for i, b in enumerate(blocks)], dtype=torch.int32,
                         device=p.k_pool.device)
    best = {}
    for name in ("out", "in"):
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if name == "out":
                kvq.kvq_swap_out(pairs, p.k_pool, p.v_pool, p.k_scale, p.v_scale, p.fmt,
                                 spec.G, buf)
            else:
                kvq.kvq_swap_in(pairs, buf, p.k_pool, p.v_pool, p.k_scale, p.v_scale,
                                p.fmt, spec.G)
            e1.record()
            torch.cuda.synchronize()
            best[name] = min(best.get(name, 1e30), e0.elapsed_time(e1))
    nbytes = len(blocks) * slot
    return {"blocks": len(blocks), "bytes": nbytes, "staging": "pinned host",
            "out_ms": round(best["out"], 3), "in_ms": round(best["in"], 3),
            "out_GBps": round(nbytes / (best["out"] * 1e-3) / 1e9, 1),
            "in_GBps": round(nbytes / (best["in"] * 1e-3) / 1e9, 1)}


PREFILL_METRIC = ("paged INT8 GQA prefill attention prompt-tokens/s + achieved TFLOP/s "
                  "(% of MI355X fp16 dense MFMA peak)")
MFMA_FP16_PEAK_TFLOPS = 2500.0


def prefill_cpu_baseline(case, spec, q, chunk, min_seconds: float,
                         unit: str = "prompt-tokens/s") -> dict:
    """The oracle's chunked prefill on the first sequence of the workload,
    repeated to about ``min_seconds``."""
    import numpy as np
    import oracle
    from oracle import expected as E
    from paged_quantized_kv_cache_amd import kvq
    d = case.data[0]
    fmt = spec.fmt_of_layer(0)
    ids = np.asarray(case.layout.seq_tokens[0], np.int64)
    sk = sv = None
    if kvq.scale_mode(fmt, spec.G) in ("head", "channel"):
        sk = case.pools[0].k_scale.cpu().numpy()
        sv = case.pools[0].v_scale.cpu().numpy()
    k16 = d.k.cpu().numpy()[ids]
    v16 = d.v.cpu().numpy()[ids]
    qh = q.cpu().numpy()[:int(chunk[0])]
    total, passes = 0.0, 0
    while total < min_seconds and passes < 20:
        t0 = time.perf_counter()
        kq = E.quantize(k16, fmt, spec.G, sk)
        vq = E.quantize(v16, fmt, spec.G, sv)
        E.prefill(qh, kq, vq, [np.arange(ids.size)], [int(chunk[0])])
        total += time.perf_counter() - t0
        passes += 1
    return {"value": int(chunk[0]) * passes / total, "unit": unit,
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "sequence 0 (%d-token chunk over %d tokens): quantize its K/V, fp64 "
                      "causal attention; %d pass(es), %.1f s"
                      % (int(chunk[0]), ids.size, passes, total)}


SHORT_METRIC = ("paged INT8 GQA short-chunk attention chunk-tokens/s + achieved HBM GB/s "
                "(% of MI355X peak)")


def run_short_chunks(args, spec) -> int:
    """Short chunks over long contexts (a few new tokens per sequence): one
    step writes the chunks' K/V into their slots (kvq_cache_write) and runs
    their causal attention over every cached token (kvq_paged_prefill, whose
    short-chunk path deals the tiles over every wavefront like decode).  Bound
    by HBM: every cached K/V byte is read once per step."""
    import numpy as np
    import torch

    from paged_quantized_kv_cache_amd import kvq
    from paged_quantized_kv_cache_amd import workloads as W
    from paged_quantized_kv_cache_amd.harness import DecodeCase

    kvq.lib()
    dev = torch.device("cuda:0")
    case = DecodeCase(spec, device=dev, poison=False)
    case.setup_layer(0)              # every token written, the chunks' included
    L = case.layout
    chunk = np.minimum(case.lens, spec.chunk)
    if L.cow_pairs.size:
        raise SystemExit("chunk workloads: no shared blocks")
    slot_of = np.full(L.n_unique, -1, np.int64)
    slot_of[L.prefill_ids] = L.prefill_slots
    slot_of[L.append_ids] = L.append_slots
    ids = np.concatenate([L.seq_tokens[b][len(L.seq_tokens[b]) - int(c):]
                          for b, c in enumerate(chunk)])
    d = case.data[0]
    it = torch.from_numpy(ids).to(d.k.device)
    k = d.k.index_select(0, it).to(dev).contiguous()
    v = d.v.index_select(0, it).to(dev).contiguous()
    slots = torch.from_numpy(slot_of[ids]).to(dev)
    q = case.chunk_queries(chunk)
    out = torch.empty_like(q)
    qstart = case.query_start(chunk)
    ws = kvq.alloc_workspace(kvq.kvq_prefill_workspace_size(
        spec.B, spec.Hq, spec.Hkv, spec.D, spec.BS, case.max_context_len,
        int(chunk.max()), args.prefill_split), dev)
    p = case.pools[0]
    nchunk = int(chunk.sum())
    # decode's algorithmic bytes with q / out for every chunk token, plus
    # the chunk offsets
    nbytes = (W.algorithmic_bytes(spec, case.lens, spec.fmt)
              + 2 * (nchunk - spec.B) * spec.Hq * spec.D * 2 + 4 * (spec.B + 1))
    stream = torch.cuda.current_stream()

    def step(ev=None):
        kvq.kvq_cache_write(k, v, slots, p.k_pool, p.v_pool, p.k_scale, p.v_scale, p.fmt,
                            spec.G)
        if ev is not None:
            ev[0].record(stream)
        case.prefill_attention(0, chunk, q, out=out, workspace=ws, query_start=qstart,
                               split_mode=args.prefill_split)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    times = np.array([a.elapsed_time(b) for a, b in ev])
    att_ms = float(times.mean())
    gbps = nbytes / (att_ms * 1e-3) / 1e9
    result = {
        "metric": SHORT_METRIC,
        "value": nchunk / (ms_per_step * 1e-3),
        "unit": "chunk-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": spec.fmt,
        "data": "synthetic (seeded N(0,1) fp16 K/V/Q with outlier channels, shuffled "
                "block pool)",
        "config": {"workload": spec.name, "description": spec.description,
                   "num_seqs": spec.B, "num_q_heads": spec.Hq, "num_kv_heads": spec.Hkv,
                   "head_dim": spec.D, "block_size": spec.BS, "kv_format": spec.fmt,
                   "group_size": spec.G, "chunk_tokens": nchunk,
                   "cached_tokens": int(case.lens.sum()), "prefill_split": args.prefill_split},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "kvq_paged_prefill, short chunks: paged_decode_kernel + "
                               "merge_runs_kernel (%s)" % spec.fmt,
                     "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": round(att_ms, 5)},
        "attention_ms_p10_p50_p90": [round(float(x), 5)
                                     for x in np.percentile(times, [10, 50, 90])],
        "cpu_baseline": (prefill_cpu_baseline(case, spec, q, chunk, args.cpu_min_seconds,
                                              "chunk-tokens/s")
                         if args.cpu_seqs > 0 else None),
    }
    print(json.dumps(result), flush=True)
    return 0


def run_mixed_heads(args, spec) -> int:
    """Per-head mixed precision: the KV heads in spec.fp16_heads live in an
    fp16 pool, the others in a pool of spec.fmt; a step appends one token per
    sequence to both pools and runs one decode call per pool into the same
    output."""
    import dataclasses
    import numpy as np
    import torch

    from paged_quantized_kv_cache_amd import kvq
    from paged_quantized_kv_cache_amd import workloads as W
    from paged_quantized_kv_cache_amd.harness import DecodeCase

    kvq.lib()
    dev = torch.device("cuda:0")
    case = DecodeCase(spec, device=dev, poison=False)
    d = case.gen(0)
    L = case.layout
    sens = list(spec.fp16_heads)
    rest = [h for h in range(spec.Hkv) if h not in sens]
    pools = []
    for fmt, G, ids in ((spec.fmt, spec.G, rest), ("fp16", 0, sens)):
        kp, vp, ks, vs = kvq.alloc_pools(L.num_blocks, len(ids), spec.BS, spec.D, fmt, G,
                                         device=dev)
        if W.static_scales(fmt, G, d.k[:, ids]) is not None:
            ks.copy_(W.static_scales(fmt, G, d.k[:, ids]))
            vs.copy_(W.static_scales(fmt, G, d.v[:, ids]))
        ids_t = torch.tensor(ids, dtype=torch.int32, device=dev)
        k = d.k.index_select(0, case.prefill_ids).to(dev).contiguous()
        v = d.v.index_select(0, case.prefill_ids).to(dev).contiguous()
        kvq.kvq_cache_write_heads(k, v, case.prefill_slots, ids_t, kp, vp, ks, vs, fmt, G)
        ws = kvq.alloc_workspace(kvq.kvq_decode_workspace_size(
            spec.B, len(ids) * spec.r, len(ids), spec.D, spec.BS, case.max_context_len),
            device=dev)
        pools.append((fmt, G, ids_t, kp, vp, ks, vs, ws))
    ka, va = case.append_inputs(0)
    q = d.q.to(dev).contiguous()
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        for fmt, G, ids_t, kp, vp, ks, vs, ws in pools:
            kvq.kvq_cache_write_heads(ka, va, case.append_slots, ids_t, kp, vp, ks, vs, fmt, G)
        if ev is not None:
            ev[0].record(stream)
        for fmt, G, ids_t, kp, vp, ks, vs, ws in pools:
            kvq.kvq_paged_decode_heads(q, spec.Hkv, ids_t, kp, vp, ks, vs, case.block_tables,
                                       case.context_lens, case.max_context_len, fmt, G,
                                       out=out, workspace=ws)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    dec_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    nbytes = 0
    for fmt, G, ids in ((spec.fmt, spec.G, rest), ("fp16", 0, sens)):
        sub = dataclasses.replace(spec, Hkv=len(ids), Hq=len(ids) * spec.r, fmt=fmt, G=G)
        nbytes += W.algorithmic_bytes(sub, case.lens, fmt)
    achieved = nbytes / (dec_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC, "value": spec.B / (ms_per_step * 1e-3), "unit": "seq-steps/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "mixed",
        "data": "synthetic (seeded N(0,1) fp16 K/V/Q with outlier channels, shuffled "
                "block pool)",
        "config": {"workload": spec.name, "description": spec.description,
                   "num_seqs": spec.B, "num_q_heads": spec.Hq, "num_kv_heads": spec.Hkv,
                   "fp16_kv_heads": sens, "head_dim": spec.D, "block_size": spec.BS,
                   "cached_tokens": int(case.lens.sum())},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None,
                     "kernel": "kvq_paged_decode_heads x2 (int8 pool + fp16 pool)",
                     "algorithmic_bytes_per_launch": int(nbytes),
                     "avg_launch_ms": round(dec_ms, 5)},
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)
    return 0


def run_prefill(args, spec) -> int:
    """A prefill workload: one step writes every prompt token's K/V into the
    pool (kvq_cache_write) and runs causal attention of the prompts over it
    (kvq_paged_prefill)."""
    import numpy as np
    import torch

    from paged_quantized_kv_cache_amd import kvq
    from paged_quantized_kv_cache_amd import workloads as W
    from paged_quantized_kv_cache_amd.harness import DecodeCase

    kvq.lib()
    dev = torch.device("cuda:0")
    case = DecodeCase(spec, device=dev, poison=False)
    case.gen(0)
    case.alloc(0)
    chunk = np.minimum(case.lens, spec.chunk)
    if np.any(chunk != case.lens):
        raise SystemExit("prefill workloads here write whole prompts (chunk >= every length)")
    q = case.chunk_queries(chunk)
    out = torch.empty_like(q)
    qstart = case.query_start(chunk)
    flops = W.prefill_flops(spec, case.lens, chunk)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        case.prefill(0)
        case.append(0)
        if ev is not None:
            ev[0].record(stream)
        case.prefill_attention(0, chunk, q, out=out, query_start=qstart)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    att_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    achieved = flops / (att_ms * 1e-3) / 1e12
    result = {
        "metric": PREFILL_METRIC,
        "value": float(chunk.sum()) / (ms_per_step * 1e-3),
        "unit": "prompt-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": spec.fmt,
        "data": "synthetic (seeded N(0,1) fp16 K/V/Q with outlier channels, shuffled "
                "block pool)",
        "config": {"workload": spec.name, "description": spec.description,
                   "num_seqs": spec.B, "num_q_heads": spec.Hq, "num_kv_heads": spec.Hkv,
                   "head_dim": spec.D, "block_size": spec.BS, "kv_format": spec.fmt,
                   "group_size": spec.G, "prompt_tokens": int(chunk.sum())},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1),
                     "peak": MFMA_FP16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_FP16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "kvq_paged_prefill: prefill_kernel (%s)" % spec.fmt,
                     "flops_per_launch": flops, "avg_launch_ms": round(att_ms, 5)},
        "cpu_baseline": (prefill_cpu_baseline(case, spec, q, chunk, args.cpu_min_seconds)
                         if args.cpu_seqs > 0 else None),
    }
    print(json.dumps(result), flush=True)
    return 0


EXTRA_WORKLOADS = ("c2_mha", "c4_long_bs16", "c4_long_bs32", "c5_prefix_mixed")


def decode_bench(spec, steps: int, warmup: int, kv_copies: int = 4, flush_bytes: int = 0,
                 flush_mode: str = "read") -> dict:
    """Build a decode workload in HBM and time `steps` steps after `warmup`
    untimed ones.  A step, for every layer: the one-token append
    (kvq_cache_write) and the decode call (kvq_paged_decode), each between
    HIP events on the stream they run on."""
    import dataclasses

    import numpy as np
    import torch

    from paged_quantized_kv_cache_amd import workloads as W
    from paged_quantized_kv_cache_amd.harness import DecodeCase

    dev = torch.device("cuda:0")
    t_setup = time.perf_counter()
    # A single-layer workload keeps `copies` independent caches of its layer
    # (the per-layer draws of the same recipe) and step i runs on copy
    # i % copies: consecutive steps touch different K/V, as consecutive layers
    # of a model do, so no step reads what the previous one left in the
    # 256 MB last-level cache.  (Back to back on one cache, C3 ran ~3.5 %
    # faster than with a 2 GiB read between steps.)
    copies = max(1, kv_copies) if spec.layers == 1 else 1
    case_spec = dataclasses.replace(spec, layers=copies) if copies > 1 else spec
    case = DecodeCase(case_spec, device=dev, poison=False)
    inputs = []
    for layer in range(case_spec.layers):
        # prefill every cached token of the layer (untimed), keep only what a
        # decode step needs: the appended tokens' K/V and the queries
        case.gen(layer)
        case.alloc(layer)
        case.prefill(layer)
        case.cow(layer)
        k, v = case.append_inputs(layer)
        q = case.data[layer].q.contiguous()
        case.append(layer, (k, v))
        if layer != (1 if spec.layers > 1 else 0):   # keep one layer's data (CPU leg)
            case.data[layer] = None
        inputs.append((k, v, q, torch.empty_like(q)))
    ws = case.workspace(0)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    print("setup %.1fs: %s, %d seqs, %d cached tokens, pool %d blocks" %
          (setup_s, spec.name, spec.B, int(case.lens.sum()), case.layout.num_blocks),
          file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    nl = spec.layers
    # optional: stream flush_bytes through a scratch copy before every step
    # (outside the decode events) so that no K/V can be served from the
    # last-level cache left by the previous step; a check of that effect,
    # not the default (the wall-clock step time then includes the copies)
    flush = None
    if flush_bytes:
        flush = (torch.empty(flush_bytes, dtype=torch.uint8, device=dev),
                 torch.empty(flush_bytes, dtype=torch.uint8, device=dev))
        flush[0].fill_(1)

    def step(i, events=None):
        if flush is not None:
            if flush_mode == "copy":
                flush[1].copy_(flush[0])
            else:  # read only: no dirty lines left behind
                torch.amax(flush[0])
        for li in range(nl):
            layer = i % copies if copies > 1 else li
            k, v, q, out = inputs[layer]
            if events is not None:
                events[li][0].record(stream)
            case.append(layer, (k, v))
            if events is not None:
                events[li][1].record(stream)
            case.decode(layer, q=q, out=out, workspace=ws)
            if events is not None:
                events[li][2].record(stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: exactly `steps` steps, synchronized on both sides
    ev = [[tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(nl)]
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i, ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    dec_ms = np.array([[ev[i][l][1].elapsed_time(ev[i][l][2]) for l in range(nl)]
                       for i in range(steps)])
    wr_ms = np.array([[ev[i][l][0].elapsed_time(ev[i][l][1]) for l in range(nl)]
                      for i in range(steps)])
    per_layer_ms = dec_ms.mean(0)
    fmts = [spec.fmt_of_layer(l) for l in range(nl)]
    uniq = case.layout.n_unique if spec.shared_prefix else None  # shared blocks once
    layer_bytes = [W.algorithmic_bytes(spec, case.lens, f, unique_tokens=uniq) for f in fmts]
    logical_bytes = [W.algorithmic_bytes(spec, case.lens, f) for f in fmts]
    # dominant kernel: the INT8 decode (all layers of that format)
    dom = [l for l in range(nl) if fmts[l] == "int8"] or list(range(nl))
    dom_ms = float(np.mean(per_layer_ms[dom]))
    dom_bytes = float(np.mean([layer_bytes[l] for l in dom]))
    all_layers = None
    if nl > 1 or spec.shared_prefix:
        # whole step, every layer's decode call: unique bytes (shared blocks
        # once) and logical bytes (every sequence's own reads)
        tot = float(per_layer_ms.sum())
        all_layers = {
            "ms": round(tot, 5),
            "unique_bytes": int(sum(layer_bytes)),
            "unique_GBps": round(sum(layer_bytes) / (tot * 1e-3) / 1e9, 1),
            "logical_bytes": int(sum(logical_bytes)),
            "logical_GBps": round(sum(logical_bytes) / (tot * 1e-3) / 1e9, 1),
            "full_model_seq_steps_per_s": round(spec.B / (tot * 1e-3), 1),
        }
    return {
        "case": case, "copies": copies, "fmts": fmts, "setup_s": round(setup_s, 1),
        "ms_per_step": wall * 1e3 / steps, "per_layer_ms": per_layer_ms,
        "dom_ms": dom_ms, "dom_bytes": dom_bytes,
        "achieved": dom_bytes / (dom_ms * 1e-3) / 1e9,
        "p10_p50_p90": [round(float(x), 5) for x in
                        np.percentile(dec_ms[:, dom].ravel(), [10, 50, 90])],
        "write_us": round(float(wr_ms.mean()) * 1e3, 2),
        "all_layers": all_layers,
    }


def summarize(spec, r: dict) -> dict:
    """The figures of one extra workload for the bench line."""
    import numpy as np
    fmt = "int8" if "int8" in r["fmts"] else r["fmts"][0]
    out = {
        "format": fmt if spec.layers == 1 else "mixed (%s dominant)" % fmt,
        "decode_call_ms": round(r["dom_ms"], 5),
        "algorithmic_bytes_per_call": int(r["dom_bytes"]),
        "achieved_GBps": round(r["achieved"], 1),
        "frac_of_peak": round(r["achieved"] / HBM_PEAK_GBPS, 4),
        "decode_ms_p10_p50_p90": r["p10_p50_p90"],
        "cache_write_us": r["write_us"],
        "ms_per_step": round(r["ms_per_step"], 5),
        "seq_steps_per_s": round(spec.B / (r["ms_per_step"] * 1e-3), 1),
    }
    if r["all_layers"] is not None:
        out["decode_all_layers"] = r["all_layers"]
        out["fp16_layer_call_ms"] = (round(float(np.mean([r["per_layer_ms"][l]
                                                          for l, f in enumerate(r["fmts"])
                                                          if f == "fp16"])), 5)
                                     if "fp16" in r["fmts"] else None)
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seqs", type=int, default=256,
                    help="sequences in the CPU-oracle sample (0 = skip)")
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0)
    ap.add_argument("--prefill-split", choices=("auto", "walk", "split"), default="auto",
                    help="chunk workloads: how kvq_paged_prefill cuts the work")
    ap.add_argument("--kv-copies", type=int, default=4,
                    help="single-layer workloads: independent caches the steps rotate "
                         "over (1 = every step on the same cache)")
    ap.add_argument("--flush-bytes", type=int, default=0,
                    help="copy this many bytes between steps, outside the timed decode "
                         "calls (last-level-cache check; off by default)")
    ap.add_argument("--flush-mode", choices=("read", "copy"), default="read",
                    help="read the flush buffer, or copy it (which also leaves dirty lines)")
    ap.add_argument("--copy-calib-bytes", type=int, default=0,
                    help="also run one plain copy of this many bytes (counter calibration)")
    ap.add_argument("--no-extras", dest="extras", action="store_false",
                    help="default workload only: skip the other decode workloads (C2, C4 "
                         "bs16 / bs32, the 32-layer prefix-sharing step), timed after it "
                         "over fewer steps")
    ap.add_argument("--no-recon", dest="recon", action="store_false",
                    help="skip the reconstruction-error summary (oracle, CPU)")
    ap.add_argument("--swap", action="store_true",
                    help="also time swapping layer 0's blocks out to pinned host "
                         "memory and back (kvq_swap_out / kvq_swap_in), outside the "
                         "timed steps")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the decode path has no cross-GPU "
              "stage (--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from paged_quantized_kv_cache_amd import kvq
    from paged_quantized_kv_cache_amd import workloads as W
    from paged_quantized_kv_cache_amd.harness import DecodeCase

    kvq.lib()
    dev = torch.device("cuda:0")
    spec = W.spec(args.workload)
    if spec.chunk > 0:
        if spec.chunk < max(spec.lens_args):   # chunks after cached tokens
            return run_short_chunks(args, spec)
        return run_prefill(args, spec)
    if spec.fp16_heads:
        return run_mixed_heads(args, spec)
    res = decode_bench(spec, args.steps, args.warmup, args.kv_copies, args.flush_bytes,
                       args.flush_mode)
    case = res["case"]
    nl = spec.layers
    fmts = res["fmts"]
    traffic = load_traffic(spec.name)
    swap = swap_bandwidth(case, spec) if args.swap else None
    if args.copy_calib_bytes:
        a = torch.zeros(args.copy_calib_bytes, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    result = {
        "metric": METRIC,
        "value": spec.B / (res["ms_per_step"] * 1e-3),
        "unit": "seq-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8" if "int8" in fmts else fmts[0],
        "data": "synthetic (seeded N(0,1) fp16 K/V/Q with outlier channels, "
                "shuffled block pool)",
        "config": {
            "workload": spec.name,
            "description": spec.description,
            "num_seqs": spec.B, "layers": nl, "num_q_heads": spec.Hq,
            "num_kv_heads": spec.Hkv, "head_dim": spec.D, "block_size": spec.BS,
            "kv_format": fmts[0] if nl == 1 else "mixed",
            "group_size": spec.G, "cached_tokens": int(case.lens.sum()),
            "mean_context": float(case.lens.mean()),
            "max_context": int(case.lens.max()),
            "partition": "balanced runs over the GPU's resident wavefronts",
            "kv_copies": res["copies"],
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(res["achieved"], 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(res["achieved"] / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": "kvq_paged_decode call: paged_decode_kernel + merge_runs_kernel (%s)"
                      % ("int8" if "int8" in fmts else fmts[0]),
            "algorithmic_bytes_per_launch": int(res["dom_bytes"]),
            "avg_launch_ms": round(res["dom_ms"], 5),
        },
        "decode_ms_per_layer": ([round(float(x), 5) for x in res["per_layer_ms"]]
                                if nl > 1 else None),
        "decode_all_layers": res["all_layers"],
        # spread of the timed calls of the dominant format (event times)
        "decode_ms_p10_p50_p90": res["p10_p50_p90"],
        "cache_write_us": res["write_us"],
        "flush_bytes_between_steps": args.flush_bytes,
        "flush_mode": args.flush_mode if args.flush_bytes else None,
        "swap": swap,
        "setup_s": res["setup_s"],
    }
    if args.cpu_seqs > 0:
        result["cpu_baseline"] = cpu_baseline(case, spec, args.cpu_seqs,
                                              layer=1 if nl > 1 else 0,
                                              min_seconds=args.cpu_min_seconds)
    else:
        result["cpu_baseline"] = None
    if args.recon:
        result["reconstruction_error"] = recon_error_summary(case, spec,
                                                             layer=1 if nl > 1 else 0)
    del case, res
    import gc
    gc.collect()
    torch.cuda.empty_cache()
    # the other decode workloads, timed the same way over fewer steps
    if args.extras and spec.name == DEFAULT_WORKLOAD:
        extra = {}
        for name in EXTRA_WORKLOADS:
            r = decode_bench(W.spec(name), max(1, min(args.steps, 10)),
                             max(1, min(args.warmup, 3)), args.kv_copies)
            extra[name] = summarize(W.spec(name), r)
            del r
            gc.collect()
            torch.cuda.empty_cache()
        result["workloads"] = extra
    print(json.dumps(result), flush=True)
    return 0

if __name__ == "__main__":
    sys.exit(main())
