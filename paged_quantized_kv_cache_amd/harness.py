"""Drive the decode hot path on the GPU for a seeded workload.

Builds the block layout on the host (``workloads.build_layout``), allocates one
layer's pools with torch, and runs the library calls in the order a decode
step uses them: prefill writes (all cached tokens), copy-on-write of shared
partial blocks, the one-token append, then paged decode.  Only the library's
kernels touch the pools.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from . import kvq
from . import workloads as W


@dataclass
class LayerPools:
    fmt: str
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    k_scale: Optional[torch.Tensor]
    v_scale: Optional[torch.Tensor]


def poison_(pools: LayerPools) -> None:
    """Fill pools with values that would corrupt any result that read them:
    NaN fp16 / NaN and inf per-group scales; INT8 bytes at the extremes
    (excess-128 bytes 0x00 and 0xFF, codes -128 and +127); FP8 NaN bytes."""
    if pools.fmt == "fp16":
        pools.k_pool.fill_(float("nan"))
        pools.v_pool.fill_(float("nan"))
    elif pools.fmt == "int8":
        pools.k_pool.fill_(0x00)
        pools.v_pool.fill_(0xFF)
    else:
        pools.k_pool.fill_(0x7F)
        pools.v_pool.fill_(0xFF)
    if pools.k_scale is not None and pools.k_scale.dim() == 4:  # per-group scales
        pools.k_scale.fill_(float("nan"))
        pools.v_scale.fill_(float("inf"))


class DecodeCase:
    """One workload on one device: layout, per-layer data and pools."""

    def __init__(self, spec: W.Spec, device="cuda", gen_device=None,
                 poison: bool = True, lens: Optional[np.ndarray] = None,
                 layout_seed: Optional[int] = None):
        self.spec = spec
        self.device = torch.device(device)
        self.gen_device = torch.device(gen_device) if gen_device else self.device
        rng = np.random.default_rng(spec.seed)
        self.lens = W.draw_lengths(spec, rng) if lens is None else np.asarray(lens, np.int64)
        if layout_seed is not None:
            rng = np.random.default_rng([spec.seed, layout_seed])
        self.layout = W.build_layout(spec, self.lens, rng)
        L = self.layout
        # Table entries past a sequence's end point at a poisoned block that
        # holds no data, never at an address outside the pool.
        unused = sorted(set(range(L.num_blocks)) - set(int(x) for x in L.used_blocks))
        self.pad_block = unused[0] if unused else 0
        # decode reads the tables with the shared-block cache hints
        bt = L.block_tables_hinted.copy()
        bt[bt < 0] = self.pad_block
        dev = self.device
        self.block_tables = torch.from_numpy(bt).to(dev)
        self.context_lens = torch.from_numpy(self.lens.astype(np.int32)).to(dev)
        self.max_context_len = int(self.lens.max())
        self.prefill_slots = torch.from_numpy(L.prefill_slots).to(dev)
        self.append_slots = torch.from_numpy(L.append_slots).to(dev)
        self.prefill_ids = torch.from_numpy(L.prefill_ids).to(self.gen_device)
        self.append_ids = torch.from_numpy(L.append_ids).to(self.gen_device)
        self.cow_pairs = torch.from_numpy(L.cow_pairs.astype(np.int32)).to(dev)
        self.poison = poison
        self.pools: List[Optional[LayerPools]] = [None] * spec.layers
        self.data: List[Optional[W.LayerData]] = [None] * spec.layers

    # ------------------------------------------------------------ setup
    def fmt(self, layer: int) -> str:
        return self.spec.fmt_of_layer(layer)

    def gen(self, layer: int) -> W.LayerData:
        d = W.gen_layer(self.spec, self.layout.n_unique, layer, device=self.gen_device)
        self.data[layer] = d
        return d

    def alloc(self, layer: int) -> LayerPools:
        s, fmt = self.spec, self.fmt(layer)
        kp, vp, ks, vs = kvq.alloc_pools(self.layout.num_blocks, s.Hkv, s.BS, s.D, fmt,
                                         s.G, device=self.device)
        pools = LayerPools(fmt, kp, vp, ks, vs)
        if self.poison:
            poison_(pools)
        d = self.data[layer]
        for scale, x in ((pools.k_scale, d.k), (pools.v_scale, d.v)):
            st = W.static_scales(fmt, s.G, x)
            if st is not None:
                scale.copy_(st)
        self.pools[layer] = pools
        return pools

    def prefill(self, layer: int) -> None:
        d, p, s = self.data[layer], self.pools[layer], self.spec
        k = d.k.index_select(0, self.prefill_ids).to(self.device)
        v = d.v.index_select(0, self.prefill_ids).to(self.device)
        kvq.kvq_cache_write(k, v, self.prefill_slots, p.k_pool, p.v_pool, p.k_scale,
                            p.v_scale, p.fmt, s.G)

    def cow(self, layer: int) -> None:
        p = self.pools[layer]
        if self.cow_pairs.numel():
            kvq.kvq_copy_blocks(self.cow_pairs, p.k_pool, p.v_pool, p.k_scale, p.v_scale,
                                p.fmt, self.spec.G)

    def append_inputs(self, layer: int):
        d = self.data[layer]
        return (d.k.index_select(0, self.append_ids).to(self.device).contiguous(),
                d.v.index_select(0, self.append_ids).to(self.device).contiguous())

    def append(self, layer: int, kv=None) -> None:
        p, s = self.pools[layer], self.spec
        k, v = kv if kv is not None else self.append_inputs(layer)
        kvq.kvq_cache_write(k, v, self.append_slots, p.k_pool, p.v_pool, p.k_scale,
                            p.v_scale, p.fmt, s.G)

    def setup_layer(self, layer: int, keep_data: bool = True) -> None:
        self.gen(layer)
        self.alloc(layer)
        self.prefill(layer)
        self.cow(layer)
        self.append(layer)
        if not keep_data:
            self.data[layer] = None

    def workspace(self, split_tokens: int = 0) -> Optional[torch.Tensor]:
        s = self.spec
        n = kvq.kvq_decode_workspace_size(s.B, s.Hq, s.Hkv, s.D, s.BS,
                                          self.max_context_len, split_tokens)
        return kvq.alloc_workspace(n, self.device)

    def decode(self, layer: int, q: Optional[torch.Tensor] = None, split_tokens: int = 0,
               out=None, workspace=None, softmax_scale: float = 0.0) -> torch.Tensor:
        p, s = self.pools[layer], self.spec
        if q is None:
            q = self.data[layer].q.to(self.device)
        return kvq.kvq_paged_decode(q, p.k_pool, p.v_pool, p.k_scale, p.v_scale,
                                    self.block_tables, self.context_lens,
                                    self.max_context_len, p.fmt, s.G,
                                    softmax_scale=softmax_scale, split_tokens=split_tokens,
                                    out=out, workspace=workspace)

    def chunk_queries(self, chunk_lens, seed: int = 7) -> torch.Tensor:
        """Seeded fp16 queries ``[sum chunk][Hq][D]`` for a prefill chunk."""
        s = self.spec
        g = torch.Generator(device="cpu")
        g.manual_seed(seed)
        n = int(np.asarray(chunk_lens).sum())
        q = torch.randn((n, s.Hq, s.D), generator=g, dtype=torch.float32)
        return q.to(torch.float16).to(self.device)

    def query_start(self, chunk_lens) -> torch.Tensor:
        """Chunk offsets ``int32 [B + 1]`` on the device."""
        n = np.asarray(chunk_lens, np.int64)
        qs = np.zeros(n.size + 1, np.int32)
        qs[1:] = np.cumsum(n)
        return torch.from_numpy(qs).to(self.device)

    def prefill_attention(self, layer: int, chunk_lens, q: torch.Tensor,
                          out=None, workspace=None, query_start=None,
                          split_mode="auto") -> torch.Tensor:
        """Chunked prefill: sequence b's last chunk_lens[b] tokens attend
        causally (their K/V are already in the pool).  ``query_start``: the
        offsets from query_start(chunk_lens), made here when None."""
        p, s = self.pools[layer], self.spec
        n = np.asarray(chunk_lens, np.int64)
        if query_start is None:
            query_start = self.query_start(n)
        return kvq.kvq_paged_prefill(q, query_start, int(n.max()) if n.size else 0,
                                     p.k_pool, p.v_pool, p.k_scale, p.v_scale,
                                     self.block_tables, self.context_lens,
                                     self.max_context_len, p.fmt, s.G, out=out,
                                     workspace=workspace, split_mode=split_mode)

    # ------------------------------------------------------------ readback
    def gather_codes(self, layer: int, seqs=None):
        """Read the pools back through the block tables: per sequence,
        contiguous ``[ctx][Hkv][D]`` codes and ``[ctx][Hkv][D/G]`` scales
        (host numpy), in logical token order.  Tile element orders follow the
        layout documented in include/kvq.h."""
        p, s = self.pools[layer], self.spec
        eb = 2 if p.fmt == "fp16" else 1
        if p.fmt == "int4":
            (koff, khi), (voff, vhi) = int4_tile_offsets(s.BS, s.D)
            koff, voff = koff[..., None], voff[..., None]
            shift = {"k": torch.from_numpy(khi.astype(np.int64) * 4).to(self.device),
                     "v": torch.from_numpy(vhi.astype(np.int64) * 4).to(self.device)}
        else:
            koff, voff = tile_offsets(s.BS, s.D, eb)
        kflat = p.k_pool.view(torch.uint8).reshape(p.k_pool.shape[0], s.Hkv, -1)
        vflat = p.v_pool.view(torch.uint8).reshape(p.v_pool.shape[0], s.Hkv, -1)
        bt = self.layout.block_tables
        out = []
        for b in (range(s.B) if seqs is None else seqs):
            n = int(self.lens[b])
            t = np.arange(n)
            blk = torch.from_numpy(bt[b, t // s.BS].astype(np.int64)).to(self.device)
            off = torch.from_numpy((t % s.BS).astype(np.int64)).to(self.device)
            item = {}
            for name, flat, offs in (("k", kflat, koff), ("v", vflat, voff)):
                o = torch.from_numpy(offs).to(self.device)[off]       # [n][D][eb]
                rows = flat[blk]                                        # [n][Hkv][bytes]
                g = torch.gather(rows, 2, o.reshape(n, 1, -1).expand(n, s.Hkv, -1))
                if p.fmt == "int4":     # nibble code + 8 -> signed code
                    sh = shift[name][off].reshape(n, 1, s.D)
                    g = ((g.to(torch.int64) >> sh) & 0xF) - 8
                    item[name] = g.to(torch.int8).cpu().numpy()
                    continue
                g = g.reshape(n, s.Hkv, s.D, eb).contiguous().cpu().numpy()
                if eb == 2:
                    g = g.view(np.float16).reshape(n, s.Hkv, s.D)
                elif p.fmt == "int8":   # excess-128 bytes -> signed codes
                    g = (g.reshape(n, s.Hkv, s.D) ^ np.uint8(0x80)).view(np.int8)
                else:
                    g = g.reshape(n, s.Hkv, s.D).view(np.uint8)
                item[name] = g
            if kvq.scale_mode(p.fmt, s.G) == "group":
                item["k_scale"] = p.k_scale[blk, :, off, :].cpu().numpy()
                item["v_scale"] = p.v_scale[blk, :, off, :].cpu().numpy()
            out.append(item)
        return out


def int4_tile_offsets(BS: int, D: int):
    """INT4 tiles (head_dim 128): ``(byte [BS][D], high-nibble flag [BS][D])``
    of every element of a K and a V tile."""
    t = np.arange(BS)[:, None]
    d = np.arange(D)[None, :]
    k = t * 64 + 16 * ((d % 64) // 16) + 4 * (2 * (d // 64) + (d % 16) // 8) + d % 4
    khi = np.broadcast_to((d % 8) >= 4, k.shape)
    v = ((t // 16) * 1024 + ((((d % 64) // 4) * 4 + (t % 16) // 4) * 4 + 2 * (d // 64)
                             + (d % 4) // 2) * 4 + t % 4)
    vhi = np.broadcast_to((d % 2) == 1, v.shape)
    return (k.astype(np.int64), khi), (v.astype(np.int64), vhi)


def tile_offsets(BS: int, D: int, eb: int):
    """Byte offsets ``[BS][D][eb]`` of every element of a K and a V tile."""
    t = np.arange(BS)[:, None]
    d = np.arange(D)[None, :]
    k = ((d * eb) // 64 * BS + t) * 64 + (d * eb) % 64
    per = 4 // eb                                   # dims per V micro-tile
    e = (d % 4) // per
    v = (((((t // 16) * eb + e) * (D // 4) + d // 4) * 4 + (t % 16) // 4) * 16
         + ((d % 4) % per) * 4 * eb + (t % 4) * eb)
    byte = np.arange(eb)[None, None, :]
    return ((k[..., None] + byte).astype(np.int64), (v[..., None] + byte).astype(np.int64))
