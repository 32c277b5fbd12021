"""Seeded synthetic workloads: shapes, lengths, block layouts and fp16 data.

This module holds inputs only -- none of the method's arithmetic (no
quantization, no attention).  Both the HIP path and the CPU oracle are fed
from what it produces, so neither side depends on the other.

Workload shapes follow the pages' study cases:
  * "KV Cache优化实战" (0539edu.com) s1.2 / s3 / s3.4: a 7B model with 32
    layers, head_dim 128, 32 KV heads (MHA) or 8 KV heads (GQA 4:1), about
    100 concurrent sequences at ~2K context; s3.2: 16-token blocks; s4.2:
    some channels carry much larger values than others (outlier channels).
  * xpshop.cn article 312, s3: 16- or 32-token blocks, FP8 KV cache.
The pages publish no dataset for this path; these seeded draws stand in for
their workloads.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

from .block_manager import BlockManager

FORMATS = ("fp16", "int8", "fp8", "e5m2", "int4")   # fp8 = E4M3


@dataclass
class Outliers:
    """``n`` persistent channels per KV head multiplied by ``factor``."""
    n: int = 0
    factor: float = 1.0


@dataclass
class Spec:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    BS: int
    fmt: str                      # format of single-layer workloads
    G: int = 0                    # scale group size (0: static / none)
    lens: str = "fixed"           # fixed | uniform | lognormal
    lens_args: tuple = ()
    pool_blocks: int = 0          # 0: ceil(slack * needed)
    pool_slack: float = 1.1
    q_out: Outliers = field(default_factory=Outliers)
    k_out: Outliers = field(default_factory=Outliers)
    v_out: Outliers = field(default_factory=Outliers)
    seed: int = 0
    layers: int = 1
    layer_fmts: Optional[Tuple[str, ...]] = None   # per-layer format
    shared_prefix: int = 0        # tokens shared by all sequences
    fork_pairs: int = 0           # pairs (2k, 2k+1) also sharing a partial tail
    chunk: int = 0                # > 0: a prefill workload, chunks of min(chunk, ctx)
    fp16_heads: Tuple[int, ...] = ()   # KV heads kept in an fp16 pool of their own
    description: str = ""

    @property
    def r(self) -> int:
        return self.Hq // self.Hkv

    def fmt_of_layer(self, layer: int) -> str:
        return self.layer_fmts[layer] if self.layer_fmts else self.fmt


# sigma of the lognormal length draw: the 8192 clip sits at the 99th
# percentile of a median-2048 lognormal (ln 4 / z_0.99).
LOGNORMAL_SIGMA = math.log(4.0) / 2.3263478740408408


def _c5_layer_fmts(layers: int = 32) -> Tuple[str, ...]:
    keep = {0, layers - 4, layers - 3, layers - 2, layers - 1}
    return tuple("fp16" if i in keep else "int8" for i in range(layers))


SPECS: Dict[str, Spec] = {
    "c1_tiny": Spec(
        "c1_tiny", B=4, Hq=4, Hkv=1, D=64, BS=16, fmt="int8", G=64,
        lens="fixed", lens_args=(5, 16, 17, 33), pool_blocks=16,
        q_out=Outliers(2, 8.0), k_out=Outliers(2, 8.0), v_out=Outliers(2, 8.0),
        seed=0, description="tiny MQA, INT8 g64, 16-block permuted pool"),
    "c2_mha": Spec(
        "c2_mha", B=100, Hq=32, Hkv=32, D=128, BS=16, fmt="int8", G=128,
        lens="uniform", lens_args=(1024, 3072), seed=0,
        description="7B-MHA-like layer, INT8 g128, shuffled pool"),
    "c3_gqa": Spec(
        "c3_gqa", B=256, Hq=32, Hkv=8, D=128, BS=16, fmt="int8", G=64,
        lens="lognormal", lens_args=(2048, 16, 8192), seed=0,
        k_out=Outliers(5, 10.0),
        description="GQA 4:1 layer, INT8 g64, lognormal lengths, K outliers"),
    "c3_gqa_fp16": Spec(
        "c3_gqa_fp16", B=256, Hq=32, Hkv=8, D=128, BS=16, fmt="fp16",
        lens="lognormal", lens_args=(2048, 16, 8192), seed=0,
        k_out=Outliers(5, 10.0),
        description="the GQA layer with an fp16 cache (baseline format)"),
    "c4_long_bs16": Spec(
        "c4_long_bs16", B=16, Hq=32, Hkv=8, D=128, BS=16, fmt="fp8",
        lens="fixed", lens_args=(32768,) * 16, seed=0,
        description="16 x 32768 tokens, FP8 e4m3, 16-token blocks"),
    "c4_long_bs32": Spec(
        "c4_long_bs32", B=16, Hq=32, Hkv=8, D=128, BS=32, fmt="fp8",
        lens="fixed", lens_args=(32768,) * 16, seed=0,
        description="16 x 32768 tokens, FP8 e4m3, 32-token blocks"),
    "c4_long_e5m2": Spec(
        "c4_long_e5m2", B=16, Hq=32, Hkv=8, D=128, BS=16, fmt="e5m2",
        lens="fixed", lens_args=(32768,) * 16, seed=0,
        description="16 x 32768 tokens, FP8 e5m2 (static per-head scales)"),
    "c3_fp8_token": Spec(
        "c3_fp8_token", B=256, Hq=32, Hkv=8, D=128, BS=16, fmt="fp8", G=128,
        lens="lognormal", lens_args=(2048, 16, 8192), seed=0,
        k_out=Outliers(5, 10.0),
        description="the GQA layer, FP8 e4m3 with a dynamic scale per "
                    "(token, head)"),
    "c3_int8_channel": Spec(
        "c3_int8_channel", B=256, Hq=32, Hkv=8, D=128, BS=16, fmt="int8", G=0,
        lens="lognormal", lens_args=(2048, 16, 8192), seed=0,
        k_out=Outliers(5, 10.0),
        description="the GQA layer, INT8 with static per-channel scales"),
    "c3_int4": Spec(
        "c3_int4", B=256, Hq=32, Hkv=8, D=128, BS=16, fmt="int4", G=64,
        lens="lognormal", lens_args=(2048, 16, 8192), seed=0,
        k_out=Outliers(5, 10.0),
        description="the GQA layer with an INT4 g64 cache"),
    "c3_mixed_heads": Spec(
        "c3_mixed_heads", B=256, Hq=32, Hkv=8, D=128, BS=16, fmt="int8", G=64,
        lens="lognormal", lens_args=(2048, 16, 8192), seed=0,
        k_out=Outliers(5, 10.0), fp16_heads=(2, 5),
        description="the GQA layer with KV heads 2 and 5 in fp16 and the other six "
                    "in INT8 g64 (per-head mixed precision)"),
    "p1_prefill_gqa": Spec(
        "p1_prefill_gqa", B=16, Hq=32, Hkv=8, D=128, BS=16, fmt="int8", G=64,
        lens="fixed", lens_args=(2048,) * 16, seed=0, k_out=Outliers(5, 10.0),
        chunk=2048,
        description="prefill of 16 prompts of 2048 tokens into the GQA INT8 g64 "
                    "pool, causal attention over the quantized cache"),
    "p2_short_chunks": Spec(
        "p2_short_chunks", B=16, Hq=32, Hkv=8, D=128, BS=16, fmt="int8", G=64,
        lens="fixed", lens_args=(32768,) * 16, seed=0, k_out=Outliers(5, 10.0),
        chunk=4,
        description="4 new tokens per sequence (e.g. draft tokens to verify) "
                    "attending over 16 contexts of 32,768 tokens, GQA INT8 g64"),
    "p3_short_chunks_8": Spec(
        "p3_short_chunks_8", B=16, Hq=32, Hkv=8, D=128, BS=16, fmt="int8", G=64,
        lens="fixed", lens_args=(32768,) * 16, seed=0, k_out=Outliers(5, 10.0),
        chunk=8,
        description="8 new tokens per sequence (two groups of 16 MFMA columns) "
                    "attending over 16 contexts of 32,768 tokens, GQA INT8 g64"),
    "p4_medium_chunks": Spec(
        "p4_medium_chunks", B=4, Hq=32, Hkv=8, D=128, BS=16, fmt="int8", G=64,
        lens="fixed", lens_args=(32768,) * 4, seed=0, k_out=Outliers(5, 10.0),
        chunk=32,
        description="32-token chunks of 4 sequences (e.g. draft tokens to verify) "
                    "attending over 32,768 cached tokens each (virtual sequences of "
                    "8 tokens), GQA INT8 g64"),
    "c5_prefix_mixed": Spec(
        "c5_prefix_mixed", B=128, Hq=32, Hkv=8, D=128, BS=16, fmt="int8",
        G=128, lens="prefix_tails", lens_args=(64, 4096), seed=0, layers=32,
        layer_fmts=_c5_layer_fmts(32), shared_prefix=1024, fork_pairs=4,
        description="32 layers, shared 1024-token prefix, fp16 layers "
                    "0 and 28-31, INT8 g128 elsewhere, copy-on-write"),
}


def spec(name: str, **overrides) -> Spec:
    s = SPECS[name]
    return dataclasses.replace(s, **overrides) if overrides else s


# ----------------------------------------------------------------- lengths
def draw_lengths(s: Spec, rng: np.random.Generator) -> np.ndarray:
    """Context length of every sequence *as decode sees it* (the appended
    token included)."""
    if s.lens == "fixed":
        lens = np.asarray(s.lens_args, np.int64)
        if lens.size == 1:
            lens = np.full(s.B, int(lens[0]), np.int64)
        assert lens.size == s.B
        return lens
    if s.lens == "uniform":
        lo, hi = s.lens_args
        return rng.integers(lo, hi + 1, size=s.B).astype(np.int64)
    if s.lens == "lognormal":
        median, lo, hi = s.lens_args
        z = rng.standard_normal(s.B)
        lens = np.rint(np.exp(math.log(median) + LOGNORMAL_SIGMA * z))
        return np.clip(lens, lo, hi).astype(np.int64)
    if s.lens == "prefix_tails":
        lo, hi = s.lens_args
        lens = s.shared_prefix + rng.integers(lo, hi + 1, size=s.B).astype(np.int64)
        # forked pairs share their tail; its last block must be partial so
        # that the append copies it (copy-on-write)
        for k in range(s.fork_pairs):
            n = int(lens[2 * k])
            if (n - s.shared_prefix - 1) % s.BS == 0:
                n += 1
            lens[2 * k] = lens[2 * k + 1] = n
        return lens
    raise ValueError(s.lens)


# ----------------------------------------------------------------- layout
@dataclass
class Layout:
    """Where every logical token of every sequence lives.

    ``seq_tokens[b]`` lists, for positions 0..ctx_b-1, the id of the unique
    token stored there (shared-prefix positions of different sequences map to
    the same id).  ``slot[u]`` is the pool slot (block * BS + offset) that
    holds unique token ``u`` *before* the append step; the appended tokens
    (the last position of every sequence) have ids ``append_ids`` and slots
    ``append_slots``, decided after copy-on-write.
    """
    context_lens: np.ndarray          # [B] int64
    block_tables: np.ndarray          # [B][max_blocks] int32 (after append)
    block_tables_hinted: np.ndarray   # same, shared blocks carry the hint bit
    num_blocks: int
    seq_tokens: List[np.ndarray]      # per sequence, unique token ids
    n_unique: int
    prefill_ids: np.ndarray           # unique ids written before the append
    prefill_slots: np.ndarray         # their slots
    append_ids: np.ndarray            # [B]
    append_slots: np.ndarray          # [B]
    cow_pairs: np.ndarray             # [n][2] (src, dst) blocks to copy first
    block_tables_before: np.ndarray   # tables before the append (for COW tests)
    used_blocks: np.ndarray           # physical ids holding data


def build_layout(s: Spec, lens: np.ndarray, rng: np.random.Generator) -> Layout:
    """Allocate blocks for every sequence through the host block manager.

    Physical ids are drawn from a shuffled free list, so logical neighbours
    are scattered across the pool."""
    B, BS = s.B, s.BS
    lens = np.asarray(lens, np.int64)
    assert lens.shape == (B,) and (lens >= 1).all()
    prefix = s.shared_prefix
    # number of blocks needed (shared blocks counted once)
    if prefix:
        assert prefix % BS == 0 and (lens > prefix).all()
    needed = 0
    if prefix:
        needed += prefix // BS
        for b in range(B):
            needed += -(-(int(lens[b]) - prefix) // BS)
    else:
        needed = int(sum(-(-int(n) // BS) for n in lens))
    needed += 2 * s.fork_pairs            # COW copies
    nblocks = s.pool_blocks or int(math.ceil(s.pool_slack * needed)) + 1
    assert nblocks >= needed, "pool too small for the workload"
    bm = BlockManager(nblocks, BS, rng=rng)

    uid = 0
    seq_tokens: List[Optional[np.ndarray]] = [None] * B
    prefill_ids: List[np.ndarray] = []
    prefill_slots: List[np.ndarray] = []

    def fill(seq: int, n: int):
        nonlocal uid
        ids = np.arange(uid, uid + n, dtype=np.int64)
        slots = np.array([bm.append_slot(seq)[0] for _ in range(n)], np.int64)
        uid += n
        return ids, slots

    # 1) the shared prefix (written once, through sequence 0)
    pre_ids = np.zeros(0, np.int64)
    if prefix:
        bm.add_sequence(0)
        pre_ids, pre_slots = fill(0, prefix)
        prefill_ids.append(pre_ids)
        prefill_slots.append(pre_slots)
        for b in range(1, B):
            bm.fork(0, b)
    else:
        for b in range(B):
            bm.add_sequence(b)

    # 2) the tails, minus the appended token
    fork_tail: Dict[int, np.ndarray] = {}
    for b in range(B):
        n_tail = int(lens[b]) - prefix - 1
        if s.fork_pairs and b < 2 * s.fork_pairs:
            if b % 2 == 1:
                continue                      # filled through its partner
            # pair (b, b+1) shares a tail whose last block is partial
            ids, slots = fill(b, n_tail)
            prefill_ids.append(ids)
            prefill_slots.append(slots)
            bm.drop_sequence(b + 1)
            bm.fork(b, b + 1)
            fork_tail[b] = ids
            fork_tail[b + 1] = ids
            continue
        ids, slots = fill(b, n_tail)
        prefill_ids.append(ids)
        prefill_slots.append(slots)
        seq_tokens[b] = np.concatenate([pre_ids, ids])
    for b, ids in fork_tail.items():
        seq_tokens[b] = np.concatenate([pre_ids, ids])
        assert seq_tokens[b].size == int(lens[b]) - 1

    tables_before = bm.tables(B)

    # 3) the append: one new token per sequence, copy-on-write if shared
    append_ids = np.arange(uid, uid + B, dtype=np.int64)
    uid += B
    append_slots = np.empty(B, np.int64)
    cow: List[Tuple[int, int]] = []
    for b in range(B):
        slot, copy = bm.append_slot(b)
        append_slots[b] = slot
        if copy is not None:
            cow.append(copy)
        seq_tokens[b] = np.concatenate([seq_tokens[b], append_ids[b:b + 1]])

    tables = bm.tables(B)
    hinted = bm.tables(B, mark_shared=True)
    return Layout(
        context_lens=lens.copy(),
        block_tables=tables,
        block_tables_hinted=hinted,
        num_blocks=nblocks,
        seq_tokens=seq_tokens,
        n_unique=uid,
        prefill_ids=np.concatenate(prefill_ids) if prefill_ids else np.zeros(0, np.int64),
        prefill_slots=np.concatenate(prefill_slots) if prefill_slots else np.zeros(0, np.int64),
        append_ids=append_ids,
        append_slots=append_slots,
        cow_pairs=np.array(cow, np.int32).reshape(-1, 2),
        block_tables_before=tables_before,
        used_blocks=np.array(sorted(bm.used_blocks()), np.int64),
    )


# ----------------------------------------------------------------- data
def _outlier_channels(rng: np.random.Generator, Hkv: int, D: int, n: int):
    return [rng.choice(D, size=n, replace=False) for _ in range(Hkv)] if n else None


def _gen(shape, gen: torch.Generator, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


@dataclass
class LayerData:
    """fp16 inputs of one layer: K, V of every unique token and Q."""
    k: torch.Tensor        # [n_unique][Hkv][D] fp16
    v: torch.Tensor        # [n_unique][Hkv][D] fp16
    q: torch.Tensor        # [B][Hq][D] fp16


def gen_layer(s: Spec, n_unique: int, layer: int = 0, device="cpu",
              seed: Optional[int] = None) -> LayerData:
    """N(0,1) fp16 K/V/Q with persistent outlier channels.

    Outlier channels are fixed per (layer, KV head) and shared by the query
    heads of that KV head.  Values are drawn in fp32 and rounded to fp16."""
    seed = s.seed if seed is None else seed
    base = (seed * 1000003 + layer * 7919) & 0x7FFFFFFF
    crng = np.random.default_rng([seed, layer, 0xC4A7])
    chans_q = _outlier_channels(crng, s.Hkv, s.D, s.q_out.n)
    chans_k = _outlier_channels(crng, s.Hkv, s.D, s.k_out.n)
    chans_v = _outlier_channels(crng, s.Hkv, s.D, s.v_out.n)
    if s.q_out.n and s.k_out.n and s.q_out.n == s.k_out.n:
        chans_q = chans_k                     # query outliers align with keys
    if s.v_out.n and s.k_out.n and s.v_out.n == s.k_out.n:
        chans_v = chans_k
    out = []
    for i, (shape, chans, o, per_kv) in enumerate([
            ((n_unique, s.Hkv, s.D), chans_k, s.k_out, 1),
            ((n_unique, s.Hkv, s.D), chans_v, s.v_out, 1),
            ((s.B, s.Hq, s.D), chans_q, s.q_out, s.r)]):
        g = torch.Generator(device=device)
        g.manual_seed(base + 101 * (i + 1))
        x = _gen(shape, g, device)
        if chans is not None:
            mult = torch.ones(shape[1], s.D, device=device)
            for h, cs in enumerate(chans):
                mult[h * per_kv:(h + 1) * per_kv, torch.as_tensor(cs, device=device)] = o.factor
            x.mul_(mult)
        out.append(x.to(torch.float16))
    return LayerData(k=out[0], v=out[1], q=out[2])


FP8_MAX = {"fp8": 448.0, "e5m2": 57344.0}


def fp8_static_scales(x: torch.Tensor, fmt: str = "fp8") -> torch.Tensor:
    """Calibrated static FP8 scale per KV head: absmax over all tokens and
    dims of that head, divided by the format's largest value (E4M3 448,
    E5M2 57344), in fp32, so that no calibrated value saturates."""
    a = x.float().abs().amax(dim=(0, 2))
    return (a / FP8_MAX[fmt]).to(torch.float32)


def int8_channel_scales(x: torch.Tensor) -> torch.Tensor:
    """Calibrated static INT8 scale per (KV head, channel): absmax over all
    tokens of that channel / 127, in fp32.  ``x``: [N][Hkv][D]."""
    a = x.float().abs().amax(dim=0)
    return (a / 127.0).to(torch.float32)


def static_scales(fmt: str, group_size: int, x: torch.Tensor) -> Optional[torch.Tensor]:
    """The static scale array a format needs (None if it has none)."""
    if group_size > 0 or fmt == "fp16":
        return None
    return int8_channel_scales(x) if fmt == "int8" else fp8_static_scales(x, fmt)


def prefill_flops(s: Spec, lens: np.ndarray, chunk_lens: np.ndarray) -> int:
    """Multiply-add flops of causal chunk attention: query at position p
    reads p + 1 tokens, 2 * D flops each for q.k and again for p.v, for
    every query head."""
    lens = np.asarray(lens, np.int64)
    n = np.asarray(chunk_lens, np.int64)
    c = lens - n
    # sum over i < n of (c + i + 1)
    keys = int(np.sum(n * c + n * (n + 1) // 2))
    return 4 * s.Hq * s.D * keys


# ----------------------------------------------------------------- bytes
def algorithmic_bytes(s: Spec, lens: np.ndarray, fmt: str,
                      unique_tokens: Optional[int] = None) -> int:
    """Bytes a decode step must move at least once: every valid cached token's
    K and V codes (+ their scales), Q in, O out, the block-table entries read
    and the context lengths.  ``unique_tokens`` counts shared blocks once."""
    ntok = int(unique_tokens if unique_tokens is not None else lens.sum())
    code_bytes = {"fp16": 2 * s.D, "int4": s.D // 2}.get(fmt, s.D)   # per token and head
    per_tok = s.Hkv * 2 * code_bytes
    G = s.G if fmt != "fp16" else 0
    if G > 0:                                              # per token-group scales
        per_tok += s.Hkv * 2 * (s.D // G) * 4
    total = ntok * per_tok
    if fmt in ("fp8", "e5m2") and G == 0:                  # static per-head scales
        total += 2 * s.Hkv * 4
    if fmt == "int8" and G == 0:                           # static per-channel scales
        total += 2 * s.Hkv * s.D * 4
    total += 2 * s.B * s.Hq * s.D * 2                     # q in, out
    total += int(sum(-(-int(n) // s.BS) for n in lens)) * 4   # table entries
    total += 4 * s.B                                       # context_lens
    return total
