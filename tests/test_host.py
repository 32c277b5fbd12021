"""Host-side logic on the CPU: block manager, layouts, and the C-ABI library
(loads, exports every declared symbol, rejects bad arguments before touching
any device)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import torch
import pytest

from paged_quantized_kv_cache_amd import workloads as W
from paged_quantized_kv_cache_amd.block_manager import BlockManager, PoolExhausted

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# ------------------------------------------------------------------ blocks
def test_block_manager_alloc_fork_cow():
    bm = BlockManager(8, 4, rng=np.random.default_rng(0))
    bm.add_sequence(0)
    slots = [bm.append_slot(0)[0] for _ in range(6)]     # 2 blocks
    b0, b1 = bm.blocks(0)
    assert slots[:4] == [b0 * 4 + i for i in range(4)]
    assert slots[4:] == [b1 * 4, b1 * 4 + 1]
    bm.fork(0, 1)
    assert bm.refcount[b0] == 2 and bm.refcount[b1] == 2
    slot, copy = bm.append_slot(1)                      # shared, partial -> COW
    assert copy is not None and copy[0] == b1
    nb = copy[1]
    assert slot == nb * 4 + 2 and bm.blocks(1) == [b0, nb]
    assert bm.refcount[b1] == 1
    slot, copy = bm.append_slot(0)                      # now private: in place
    assert copy is None and slot == b1 * 4 + 2
    bm.drop_sequence(1)
    assert bm.refcount[nb] == 0 and bm.refcount[b0] == 1
    t = bm.tables(2)
    assert list(t[0, :2]) == [b0, b1] and (t[1] == -1).all()


def test_block_manager_exhaustion():
    bm = BlockManager(2, 16)
    bm.add_sequence(0)
    for _ in range(32):
        bm.append_slot(0)
    with pytest.raises(PoolExhausted):
        bm.append_slot(0)


@pytest.mark.parametrize("name,over", [
    ("c1_tiny", {}),
    ("c3_gqa", dict(B=7, lens="fixed", lens_args=(1, 15, 16, 17, 100, 300, 31))),
    ("c4_long_bs32", dict(B=3, lens="fixed", lens_args=(1, 33, 95))),
    ("c5_prefix_mixed", dict(B=10, shared_prefix=64, lens_args=(3, 90), fork_pairs=3)),
])
def test_layout_gather_reproduces_contiguous(name, over):
    """Writing every unique token into its slot (prefill, COW copies, append)
    and gathering through the tables gives each sequence's tokens in order."""
    s = W.spec(name, **over)
    rng = np.random.default_rng(s.seed)
    lens = W.draw_lengths(s, rng)
    L = W.build_layout(s, lens, rng)
    pool = np.full(L.num_blocks * s.BS, -1, np.int64)   # slot -> unique id
    pool[L.prefill_slots] = L.prefill_ids
    for src, dst in L.cow_pairs:
        pool[dst * s.BS:(dst + 1) * s.BS] = pool[src * s.BS:(src + 1) * s.BS]
    pool[L.append_slots] = L.append_ids
    for b in range(s.B):
        n = int(lens[b])
        t = np.arange(n)
        slots = L.block_tables[b, t // s.BS] * s.BS + t % s.BS
        assert np.array_equal(pool[slots], L.seq_tokens[b])
        assert L.seq_tokens[b][-1] == L.append_ids[b]
    # every sequence's table is contiguous in logical order and has no gaps
    assert (L.block_tables[L.block_tables >= 0] < L.num_blocks).all()
    if s.shared_prefix:
        pre = s.shared_prefix // s.BS
        assert (L.block_tables[:, :pre] == L.block_tables[0, :pre]).all()
        assert L.cow_pairs.shape == (s.fork_pairs, 2)
    # appended slots are distinct
    assert np.unique(L.append_slots).size == s.B


def test_lengths_recipes():
    s = W.spec("c3_gqa")
    lens = W.draw_lengths(s, np.random.default_rng(0))
    assert lens.min() >= 16 and lens.max() <= 8192
    assert 1800 < np.median(lens) < 2300
    s2 = W.spec("c2_mha")
    l2 = W.draw_lengths(s2, np.random.default_rng(0))
    assert l2.min() >= 1024 and l2.max() <= 3072
    s5 = W.spec("c5_prefix_mixed")
    l5 = W.draw_lengths(s5, np.random.default_rng(0))
    assert (l5 >= 1024 + 64).all() and (l5 <= 1024 + 4097).all()
    for k in range(s5.fork_pairs):
        assert l5[2 * k] == l5[2 * k + 1] and (l5[2 * k] - 1024 - 1) % 16 != 0
    assert s5.layer_fmts.count("fp16") == 5 and s5.layer_fmts[0] == "fp16"
    assert s5.layer_fmts[28:] == ("fp16",) * 4


def test_generated_inputs_have_outlier_channels():
    s = W.spec("c3_gqa", B=2)
    d = W.gen_layer(s, 4000, 0, device="cpu")
    a = d.k.float().abs().mean(0)                        # [Hkv][D]
    for h in range(s.Hkv):
        big = (a[h] > 4).sum().item()
        assert big == 5                                  # 4% of 128 -> 5 channels
    assert d.v.float().abs().mean().item() < 1.0


def test_generated_inputs_are_reproducible():
    # both sides are fed from these draws: the same seed and layer give the
    # same bytes, another layer other bytes
    s = W.spec("c1_tiny")
    a = W.gen_layer(s, 71, 0, device="cpu")
    b = W.gen_layer(s, 71, 0, device="cpu")
    c = W.gen_layer(s, 71, 1, device="cpu")
    for x, y in ((a.k, b.k), (a.v, b.v), (a.q, b.q)):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert not torch.equal(a.k, c.k)
    l1 = W.draw_lengths(W.spec("c3_gqa"), np.random.default_rng(0))
    l2 = W.draw_lengths(W.spec("c3_gqa"), np.random.default_rng(0))
    assert np.array_equal(l1, l2)


def test_host_validation_of_decode_metadata():
    from paged_quantized_kv_cache_amd import kvq
    bt = torch.tensor([[3, 5, 7, 0], [1 | kvq.SHARED_HINT_BIT, 2, 99, -1]], dtype=torch.int32)
    cl = torch.tensor([40, 20], dtype=torch.int32)   # 3 and 2 blocks of 16 in use
    kvq.validate_decode_inputs(bt, cl, 64, 16, 8)      # unused entries are not read
    with pytest.raises(ValueError, match="sequence 1: context length 0"):
        kvq.validate_decode_inputs(bt, torch.tensor([40, 0], dtype=torch.int32), 64, 16, 8)
    with pytest.raises(ValueError, match=r"context length 70 outside \[1, 64\]"):
        kvq.validate_decode_inputs(bt, torch.tensor([70, 20], dtype=torch.int32), 64, 16, 8)
    with pytest.raises(ValueError, match="outside the pool"):
        kvq.validate_decode_inputs(bt, torch.tensor([40, 33], dtype=torch.int32), 64, 16, 8)
    with pytest.raises(ValueError, match="bit 31"):
        kvq.validate_decode_inputs(bt, torch.tensor([40, 64], dtype=torch.int32), 64, 16, 8)
    with pytest.raises(ValueError, match="table width"):
        kvq.validate_decode_inputs(bt, cl, 65, 16, 8)
    qs = torch.tensor([0, 4, 4], dtype=torch.int32)
    kvq.validate_decode_inputs(bt, cl, 64, 16, 8, qs)
    with pytest.raises(ValueError, match="chunk of 25 tokens"):
        kvq.validate_decode_inputs(bt, cl, 64, 16, 8, torch.tensor([0, 4, 29], dtype=torch.int32))
    # the workloads' own tables pass
    s = W.spec("c5_prefix_mixed", B=10, shared_prefix=64, lens_args=(3, 90), fork_pairs=3)
    rng = np.random.default_rng(0)
    lens = W.draw_lengths(s, rng)
    L = W.build_layout(s, lens, rng)
    t = torch.from_numpy(np.where(L.block_tables_hinted < 0, 0, L.block_tables_hinted))
    kvq.validate_decode_inputs(t, torch.from_numpy(lens.astype(np.int32)), int(lens.max()),
                               s.BS, L.num_blocks)


# ------------------------------------------------------------------ library
@pytest.fixture(scope="module")
def lib():
    from paged_quantized_kv_cache_amd import build as B
    from paged_quantized_kv_cache_amd import kvq
    if B.stale():
        B.build()
    return kvq.lib()


def _declared_symbols():
    with open(os.path.join(ROOT, "include", "kvq.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"KVQ_API\s+[\w\s\*]+?\b(kvq_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol(lib):
    from paged_quantized_kv_cache_amd import kvq
    names = _declared_symbols()
    assert set(names) == set(kvq.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", kvq.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (kvq_\w+)", out))
    assert exported == set(names)


def test_status_strings_and_version(lib):
    assert lib.kvq_version() >= 100
    for code in (0, -1, -2, -3, -4, 7):
        assert lib.kvq_status_string(code)


def test_workspace_size(lib):
    from paged_quantized_kv_cache_amd import kvq
    # always holds the run plan; grows with the partial slots of the runs
    small = kvq.kvq_decode_workspace_size(4, 4, 1, 64, 16, 33)
    assert small > 0
    big = kvq.kvq_decode_workspace_size(16, 32, 8, 128, 16, 32768)
    assert big > small
    # fixed spans: one run per span of every (sequence, KV head) unit
    fixed = kvq.kvq_decode_workspace_size(16, 32, 8, 128, 16, 32768, 1024)
    runs = 16 * 8 * 32
    assert fixed >= runs * 2 * 4 * (128 + 2) * 4
    with pytest.raises(ValueError):
        kvq.kvq_decode_workspace_size(2, 4, 2, 64, 16, 0)
    with pytest.raises(ValueError):
        kvq.kvq_decode_workspace_size(2, 4, 2, 64, 16, 100, 24)
    with pytest.raises(ValueError):
        kvq.kvq_decode_workspace_size(2, 6, 4, 64, 16, 100)


def test_prefill_workspace_size(lib):
    from paged_quantized_kv_cache_amd import kvq
    # short chunks (chunk x Hq/Hkv <= 32) take the decode partition: partial
    # slots of chunk x r columns per run
    r4 = kvq.kvq_prefill_workspace_size(16, 32, 8, 128, 16, 32768, 4)
    assert r4 > 0
    assert r4 > kvq.kvq_prefill_workspace_size(16, 32, 8, 128, 16, 32768, 1)
    assert kvq.kvq_prefill_workspace_size(16, 32, 8, 128, 16, 32768, 1) == \
        kvq.kvq_decode_workspace_size(16, 32, 8, 128, 16, 32768)
    # longer chunks walk per (sequence, KV head, group): no workspace
    assert kvq.kvq_prefill_workspace_size(16, 32, 8, 128, 16, 32768, 8) > r4
    # longer chunks: the walk needs nothing; split cuts them into virtual
    # sequences of 32 / r tokens (their lengths, then the decode workspace)
    assert kvq.kvq_prefill_workspace_size(16, 32, 8, 128, 16, 32768, 9, "walk") == 0
    v9 = kvq.kvq_prefill_workspace_size(16, 32, 8, 128, 16, 32768, 9, "split")
    assert v9 > kvq.kvq_prefill_workspace_size(16, 32, 8, 128, 16, 32768, 8)
    # auto: few sequences and chunk tokens -> split; whole prompts -> walk
    assert kvq.kvq_prefill_workspace_size(16, 32, 8, 128, 16, 32768, 9) == v9
    assert kvq.kvq_prefill_workspace_size(16, 32, 8, 128, 16, 2048, 2048) == 0
    assert kvq.kvq_prefill_workspace_size(16, 32, 8, 128, 16, 2048, 2048, "split") > 0
    assert kvq.kvq_prefill_workspace_size(4, 8, 8, 64, 16, 100, 33, "walk") == 0
    assert kvq.kvq_prefill_workspace_size(4, 8, 8, 64, 16, 100, 32) > 0
    assert kvq.kvq_prefill_workspace_size(4, 8, 8, 64, 16, 100, 32, "walk") == 0
    assert kvq.kvq_prefill_workspace_size(4, 8, 8, 64, 16, 100, 0) == 0
    with pytest.raises(ValueError):
        kvq.kvq_prefill_workspace_size(4, 8, 8, 64, 16, 10, 11)   # chunk > context bound
    with pytest.raises(ValueError):
        kvq.kvq_prefill_workspace_size(4, 6, 4, 64, 16, 100, 2)   # Hq % Hkv != 0
    with pytest.raises(ValueError):
        kvq.kvq_prefill_workspace_size(4, 8, 2, 64, 16, 100, 2, 7)  # no such mode


def test_prefill_arguments_rejected_before_any_device_work(lib):
    dummy = ctypes.c_void_p(16)

    def pre(mq=4, ws=None, mcl=60, Hq=8, Hkv=2, D=64, mode=0):
        return lib.kvq_paged_prefill(dummy, dummy, mq, dummy, dummy, dummy, dummy, dummy, 4,
                                     dummy, mcl, 2, Hq, Hkv, D, 16, 8, 1, 64, 0.0, mode,
                                     dummy, ws, 0, None)
    assert pre(mq=4) == -3                       # short chunks need a workspace
    assert pre(mq=20, mode=2) == -3              # so does a forced split of longer ones
    assert pre(mq=4, mode=5) == -1               # no such split mode
    assert pre(mq=0) == 0                        # nothing to do
    assert pre(mq=61) == -1                      # chunk longer than the context bound
    assert pre(Hq=6, Hkv=4) == -1
    assert pre(D=96) == -2


def test_bad_arguments_rejected_before_any_device_work(lib):
    P = ctypes.c_void_p
    dummy = P(16)
    # unsupported formats / shapes
    assert lib.kvq_cache_write(dummy, dummy, dummy, 1, 1, 96, 16, 4, 1, 32,
                               dummy, dummy, dummy, dummy, None) == -2
    assert lib.kvq_cache_write(dummy, dummy, dummy, 1, 1, 128, 8, 4, 1, 64,
                               dummy, dummy, dummy, dummy, None) == -2
    assert lib.kvq_cache_write(dummy, dummy, dummy, 1, 1, 64, 16, 4, 1, 128,
                               dummy, dummy, dummy, dummy, None) == -2
    assert lib.kvq_cache_write(dummy, dummy, dummy, 1, 1, 64, 16, 4, 7, 64,
                               dummy, dummy, dummy, dummy, None) == -2
    # E5M2 has static per-head scales only; group sizes are 0, 64 or 128
    assert lib.kvq_cache_write(dummy, dummy, dummy, 1, 1, 128, 16, 4, 3, 64,
                               dummy, dummy, dummy, dummy, None) == -2
    assert lib.kvq_cache_write(dummy, dummy, dummy, 1, 1, 128, 16, 4, 1, 32,
                               dummy, dummy, dummy, dummy, None) == -2
    assert lib.kvq_cache_write(dummy, dummy, dummy, 1, 1, 128, 16, 4, 2, 96,
                               dummy, dummy, dummy, dummy, None) == -2
    # null pointers
    assert lib.kvq_cache_write(None, dummy, dummy, 1, 1, 64, 16, 4, 1, 64,
                               dummy, dummy, dummy, dummy, None) == -1
    # nothing to do
    assert lib.kvq_cache_write(None, None, None, 0, 1, 64, 16, 4, 1, 64,
                               None, None, None, None, None) == 0
    args = dict(q=dummy, kp=dummy, vp=dummy, ks=dummy, vs=dummy, bt=dummy, mb=4,
                cl=dummy, mcl=60, B=2, Hq=8, Hkv=2, D=64, BS=16, nb=8, dt=1, G=64,
                sm=0.0, split=0, out=dummy, ws=None, wsb=0)

    def dec(**kw):
        a = dict(args, **kw)
        return lib.kvq_paged_decode(a["q"], a["kp"], a["vp"], a["ks"], a["vs"], a["bt"],
                                    a["mb"], a["cl"], a["mcl"], a["B"], a["Hq"], a["Hkv"],
                                    a["D"], a["BS"], a["nb"], a["dt"], a["G"], a["sm"],
                                    a["split"], a["out"], a["ws"], a["wsb"], None)
    assert dec(Hq=6, Hkv=4) == -1                 # Hq % Hkv != 0
    assert dec(Hq=68, Hkv=2) == -2                # more than 16 heads per KV head
    assert dec(mcl=65) == -1                      # tables too short for the bound
    assert dec(split=24) == -1                    # not a multiple of 16
    assert dec(sm=-1.0) == -1
    assert dec(q=None) == -1
    assert dec(split=16) == -3                    # needs a workspace
    assert dec() == -3
    assert dec(D=96) == -2
    assert dec(dt=3, G=64) == -2                  # E5M2: static scales only
    assert dec(dt=3, G=0) == -3                   # E5M2 per head: valid, needs a workspace
    assert dec(dt=1, G=0) == -3                   # INT8 per channel: valid
    assert dec(dt=2, G=64) == -3                  # E4M3 per group: valid
    # head subsets: a head list is required; the pool cannot hold more heads
    # than the model has
    a = dict(args)
    assert lib.kvq_paged_decode_heads(a["q"], a["kp"], a["vp"], a["ks"], a["vs"], a["bt"],
                                      a["mb"], a["cl"], a["mcl"], a["B"], a["Hq"], a["Hkv"],
                                      None, 1, a["D"], a["BS"], a["nb"], a["dt"], a["G"],
                                      a["sm"], 0, a["out"], None, 0, None) == -1
    assert lib.kvq_paged_decode_heads(a["q"], a["kp"], a["vp"], a["ks"], a["vs"], a["bt"],
                                      a["mb"], a["cl"], a["mcl"], a["B"], a["Hq"], a["Hkv"],
                                      dummy, 3, a["D"], a["BS"], a["nb"], a["dt"], a["G"],
                                      a["sm"], 0, a["out"], None, 0, None) == -1
    assert lib.kvq_paged_decode_heads(a["q"], a["kp"], a["vp"], a["ks"], a["vs"], a["bt"],
                                      a["mb"], a["cl"], a["mcl"], a["B"], a["Hq"], a["Hkv"],
                                      dummy, 1, a["D"], a["BS"], a["nb"], a["dt"], a["G"],
                                      a["sm"], 0, a["out"], None, 0, None) == -3
    assert lib.kvq_cache_write_heads(dummy, dummy, dummy, 1, 2, None, 1, 64, 16, 4, 1, 64,
                                     dummy, dummy, dummy, dummy, None) == -1
    assert dec(B=0) == 0
    assert dec(dt=1, ks=None) == -1
    assert lib.kvq_copy_blocks(dummy, 1, 1, 64, 16, 4, 1, 64, dummy, dummy, None, None,
                               None) == -1
    assert lib.kvq_copy_blocks(None, 0, 1, 64, 16, 4, 1, 64, None, None, None, None,
                               None) == 0


# ------------------------------------------------------------------ LRU, preemption, swap
def test_block_lru_order_and_preemption():
    from paged_quantized_kv_cache_amd.block_manager import (BlockManager, PoolExhausted,
                                                            SwapSpace)
    bm, space = BlockManager(16, 16), SwapSpace(8)
    for s in (0, 2, 3):
        bm.add_sequence(s)
    for _ in range(40):
        bm.append_slot(0)                           # 3 blocks
    bm.fork(0, 1)                                   # shares them
    for _ in range(20):
        bm.append_slot(2)                           # 2 blocks
    for _ in range(5):
        bm.append_slot(3)                           # 1 block
    bm.touch([2])
    bm.touch([0, 1, 3])
    order = bm.lru_blocks()
    assert order[:2] == sorted(bm.blocks(2))        # read least recently
    # seq 3 has the lowest priority; seq 2 is the least recently read of the rest
    free0 = bm.num_free()
    out = bm.preempt(free0 + 3, {0: 9, 1: 9, 2: 5, 3: 1}, space)
    assert [s for s, _ in out] == [3, 2]
    assert bm.num_free() == free0 + 3 and not bm.resident(2) and not bm.resident(3)
    # swapping seq 1 out copies and frees nothing: its blocks are shared
    # with seq 0, and it keeps its reference to them
    shared = bm.blocks(1)
    slots0 = space.num_free()
    assert bm.swap_out(1, space) == [] and bm.num_free() == free0 + 3
    assert all(bm.refcount[b] == 2 for b in shared) and space.num_free() == slots0
    # a preemption that runs out of swap slots leaves its victim resident
    # with its blocks and reference counts unchanged
    bm.add_sequence(4)
    for _ in range(16 * 4):
        bm.append_slot(4)                           # 4 private blocks
    space.alloc(space.num_free() - 2)               # only 2 slots left
    before = (bm.blocks(4), bm.refcount.copy(), bm.num_free(), space.num_free())
    with pytest.raises(PoolExhausted):
        bm.preempt(100, {0: 9, 4: 0}, space)
    assert bm.resident(4) and bm.blocks(4) == before[0]
    assert np.array_equal(bm.refcount, before[1])
    assert bm.num_free() == before[2] and space.num_free() == before[3]


def test_swap_keeps_prefix_sharing():
    from paged_quantized_kv_cache_amd.block_manager import BlockManager, SwapSpace
    bm, space = BlockManager(32, 16, rng=np.random.default_rng(5)), SwapSpace(16)
    bm.add_sequence(0)
    for _ in range(64):
        bm.append_slot(0)                           # a 4-block prefix
    for s in (1, 2):
        bm.fork(0, s)
        for _ in range(20 + 10 * s):
            bm.append_slot(s)                       # private tails
    prefix, tail = bm.blocks(1)[:4], bm.blocks(1)[4:]
    pairs = bm.swap_out(1, space)
    assert [b for b, _ in pairs] == tail            # only the private blocks move
    assert all(bm.refcount[b] == 3 for b in prefix)
    bm.drop_sequence(0)                             # another sharer leaves
    for _ in range(40):
        bm.append_slot(2)                           # and the pool is reused
    back = bm.swap_in(1, space)
    assert bm.blocks(1)[:4] == prefix               # the same shared blocks again
    assert [b for b, _ in back] == bm.blocks(1)[4:]
    assert [s for _, s in back] == [s for _, s in pairs]
    assert all(bm.refcount[b] == 2 for b in prefix) and space.num_free() == 16
    shared = bm.tables(3, mark_shared=True)[1, :4]
    assert all((x >> 30) & 1 for x in shared)
    # a swapped-out sequence that is dropped gives its slots and references back
    bm.swap_out(1, space)
    bm.drop_sequence(1, space)
    assert all(bm.refcount[b] == 1 for b in prefix) and space.num_free() == 16


def test_swap_round_trip_bookkeeping():
    from paged_quantized_kv_cache_amd.block_manager import BlockManager, SwapSpace
    bm, space = BlockManager(12, 16, rng=np.random.default_rng(3)), SwapSpace(6)
    bm.add_sequence(0)
    bm.add_sequence(1)
    for _ in range(37):
        bm.append_slot(0)
    for _ in range(3):
        bm.append_slot(1)
    old = bm.blocks(0)
    pairs = bm.swap_out(0, space)
    assert [b for b, _ in pairs] == old and space.num_free() == 3
    slots = [s for _, s in pairs]
    for _ in range(20):                             # someone else takes the blocks
        bm.append_slot(1)
    back = bm.swap_in(0, space)
    assert [s for _, s in back] == slots and space.num_free() == 6
    assert bm.length(0) == 37 and len(bm.blocks(0)) == 3
    assert set(bm.blocks(0)).isdisjoint(bm.blocks(1))
    slot, copy = bm.append_slot(0)                  # continues in its last block
    assert copy is None and slot == bm.blocks(0)[-1] * 16 + 37 % 16
    pairs = bm.swap_out(1, space)
    bm.drop_sequence(1, space)                      # dropping a swapped sequence frees its slots
    assert space.num_free() == 6


def test_swap_block_bytes_and_arguments(lib):
    from paged_quantized_kv_cache_amd import kvq
    P = ctypes.c_void_p
    sb = kvq.kvq_swap_block_bytes
    assert sb(8, 128, 16, "int8", 64) == 2 * 8 * 16 * 128 + 2 * 8 * 16 * 2 * 4
    assert sb(8, 128, 16, "fp16") == 2 * 8 * 16 * 128 * 2
    assert sb(8, 128, 16, "fp8", 0) == 2 * 8 * 16 * 128
    assert sb(8, 128, 32, "fp8", 128) == 2 * 8 * 32 * 128 + 2 * 8 * 32 * 4
    assert sb(1, 64, 16, "int8", 0) == 2 * 16 * 64            # static scales stay put
    assert sb(3, 64, 16, "e5m2") % 256 == 0
    with pytest.raises(ValueError):
        sb(8, 128, 16, "e5m2", 64)
    dummy = P(16)
    # null buffer / pairs; nothing to do
    assert lib.kvq_swap_out(dummy, 1, 1, 64, 16, 4, 1, 64, dummy, dummy, dummy, dummy,
                            None, 1, None) == -1
    assert lib.kvq_swap_in(None, 1, 1, 64, 16, 4, 1, 64, dummy, 1, dummy, dummy, dummy,
                           dummy, None) == -1
    assert lib.kvq_swap_out(None, 0, 1, 64, 16, 4, 1, 64, None, None, None, None,
                            None, 0, None) == 0
    assert lib.kvq_swap_out(dummy, 1, 1, 96, 16, 4, 1, 64, dummy, dummy, dummy, dummy,
                            dummy, 1, None) == -2


def test_int4_tile_layouts_are_bijections():
    from paged_quantized_kv_cache_amd.harness import int4_tile_offsets
    for bs in (16, 32):
        (k, kh), (v, vh) = int4_tile_offsets(bs, 128)
        for off, hi in ((k, kh), (v, vh)):
            key = off * 2 + hi
            assert len(np.unique(key)) == key.size == bs * 128
            assert key.min() == 0 and key.max() == bs * 128 - 1
        # a V byte never holds two tokens; a K byte never holds two tokens
        for off in (k, v):
            tok = np.broadcast_to(np.arange(bs)[:, None], off.shape)
            byte_tok = {}
            for b, t in zip(off.ravel(), tok.ravel()):
                assert byte_tok.setdefault(int(b), int(t)) == int(t)


def test_int4_arguments(lib):
    P = ctypes.c_void_p
    dummy = P(16)
    # INT4: head_dim 128 and a group size of 64 or 128 only
    assert lib.kvq_cache_write(dummy, dummy, dummy, 1, 1, 64, 16, 4, 4, 64,
                               dummy, dummy, dummy, dummy, None) == -2
    assert lib.kvq_cache_write(dummy, dummy, dummy, 1, 1, 128, 16, 4, 4, 0,
                               dummy, dummy, dummy, dummy, None) == -2
    assert lib.kvq_cache_write(None, dummy, dummy, 1, 1, 128, 16, 4, 4, 64,
                               dummy, dummy, dummy, dummy, None) == -1
    from paged_quantized_kv_cache_amd import kvq
    assert kvq.kvq_swap_block_bytes(8, 128, 16, "int4", 64) == 2 * 8 * 16 * 64 + 2 * 8 * 16 * 2 * 4


def test_bench_refuses_more_than_one_gpu(capsys):
    # one GPU only: --gpus N > 1 exits with a message before touching a GPU
    import bench
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_generated_inputs_match_their_fingerprints():
    """The seeded inputs of every workload (lengths, block tables, the first
    4,096 tokens' K / V and the queries of layer 0, drawn on the CPU) hash
    to the values stored in tests/golden/input_fingerprints.txt: a change of
    the recipe or of the random streams it uses fails here."""
    import importlib.util
    path = os.path.join(ROOT, "tests", "golden", "make_input_fingerprints.py")
    spec = importlib.util.spec_from_file_location("make_input_fingerprints", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    stored = {}
    with open(os.path.join(ROOT, "tests", "golden", "input_fingerprints.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                p = line.split()
                stored[p[0]] = dict(zip(("lens", "tables", "k", "v", "q"), p[1:]))
    assert set(stored) == set(W.SPECS)
    for name in sorted(W.SPECS):
        assert mod.fingerprints(name) == stored[name], name
