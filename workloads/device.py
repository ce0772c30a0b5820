"""Stage a seeded workload in device memory and describe it to the C ABI.

Input staging only: draws the workload's blocks (threaded), copies them to HBM,
allocates sentinel-filled destinations (dense rows or a paged pool), and builds
the kamera_chunk descriptors. It performs none of the operator's arithmetic.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

from position_free_kv_amd import abi
from .configs import BF16, BF16_SENTINEL, F32_SENTINEL, GQA, POSITIONS, ChunkSpec, Workload


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _sentinel_fill(t: torch.Tensor, dtype: int) -> torch.Tensor:
    """Fill with the sentinel bit pattern; returns `t` itself (not a view)."""
    if dtype == BF16:
        t.fill_(int(np.uint16(BF16_SENTINEL).view(np.int16)))
    else:
        t.view(torch.int32).fill_(int(np.uint32(F32_SENTINEL).view(np.int32)))
    return t


class DeviceWorkload:
    def __init__(self, wl: Workload, device: str = "cuda"):
        self.wl = wl
        self.device = torch.device(device)
        lay = wl.layout
        self.lay = lay
        self.L, self.F, self.P = lay.num_layers, lay.row_width, lay.page_size
        self.tdtype = torch.int16 if lay.dtype == BF16 else torch.float32
        self.es = lay.elem_bytes
        nt = lay.num_tensors

        # ---- which blocks to draw
        canon_ids = sorted({c.canon_id for c in wl.chunks if not c.in_place})
        fac_keys: Dict[Tuple[int, int], Tuple[ChunkSpec, int]] = {}
        for c in wl.chunks:
            if c.patched:
                for fi, f in enumerate(c.factors):
                    fac_keys.setdefault((f.key, f.slot), (c, fi))

        self.canon: Dict[int, List[torch.Tensor]] = {
            cid: [torch.empty((self.L, wl.canon_tokens[cid], self.F), dtype=self.tdtype, device=self.device)
                  for _ in range(nt)] for cid in canon_ids}
        self.factors: Dict[Tuple[int, int], Tuple[torch.Tensor, torch.Tensor]] = {}
        bases: Dict[Tuple[int, int, int, int, int], torch.Tensor] = {}
        for key, (c, fi) in fac_keys.items():
            f = c.factors[fi]
            nl = self.L - f.layer0
            vshape = (nl, f.width, f.rank)
            if f.basis >= 0:   # one V buffer per shared basis, aliased by every chunk that names it
                bk = (f.basis, f.slot, f.layer0, f.width, f.rank)
                if bk not in bases:
                    bases[bk] = torch.empty(vshape, dtype=self.tdtype, device=self.device)
                v = bases[bk]
            else:
                v = torch.empty(vshape, dtype=self.tdtype, device=self.device)
            self.factors[key] = (torch.empty((nl, c.num_tokens, f.rank), dtype=self.tdtype, device=self.device), v)
        # dense destinations and pool, sentinel filled
        self.dense = [[_sentinel_fill(torch.empty((self.L, rows, self.F), dtype=self.tdtype, device=self.device),
                                      lay.dtype) for _ in range(nt)] for rows in wl.dense_rows]
        self.pool: Optional[List[torch.Tensor]] = None
        if wl.num_pages:
            self.pool = [_sentinel_fill(torch.empty((self.L, wl.num_pages, self.P, self.F), dtype=self.tdtype,
                                                    device=self.device), lay.dtype) for _ in range(nt)]

        jobs = []
        for cid in canon_ids:
            for layer in range(self.L):
                for t in range(nt):
                    jobs.append(("canon", cid, layer, t))
        for key, (c, fi) in fac_keys.items():
            for layer in range(c.factors[fi].layer0, self.L):
                jobs.append(("factor", key, layer, None))
        for c in wl.chunks:
            if c.in_place:
                for layer in range(self.L):
                    for t in range(nt):
                        jobs.append(("pool", c.index, layer, t))
        self._stage(jobs, fac_keys)
        torch.cuda.synchronize(self.device)

        # per-token (t, h, w) offsets of re-anchored chunks, [T][3] int32 on the device
        self.positions = {c.index: torch.from_numpy(np.ascontiguousarray(c.positions, dtype=np.int32)).to(self.device)
                          for c in wl.chunks if c.positions is not None}
        self.descs = [self._desc(c) for c in wl.chunks]
        self.pool_desc = None
        if self.pool is not None:
            self.pool_desc = abi.make_pool(self.pool[0], self.pool[1] if nt == 2 else None, wl.num_pages)
        self.layout = abi.make_layout(lay.family, lay.dtype, self.L, num_kv_heads=lay.num_kv_heads,
                                      head_dim=lay.head_dim, latent_dim=lay.latent_dim, rope_dim=lay.rope_dim,
                                      pairing=lay.pairing, rope_base=lay.rope_base, page_size=self.P,
                                      mrope_section=lay.mrope_section)
        self.ws_bytes = abi.batch_workspace_bytes(self.layout, self.descs)
        self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=self.device)

    # ------------------------------------------------------------------ staging
    def _draw(self, job, fac_keys):
        kind, a, layer, t = job
        if kind == "canon":
            return self.wl.canonical(a, layer, t)
        if kind == "pool":
            return self.wl.pool_rows(self.wl.chunks[a], layer, t)
        c, fi = fac_keys[a]
        return self.wl.factor(c, fi, layer)

    def _put(self, job, arr, fac_keys):
        kind, a, layer, t = job
        def dev(x):
            x = np.ascontiguousarray(x)
            if self.lay.dtype == BF16:
                x = x.view(np.int16)
            return torch.from_numpy(x).to(self.device, non_blocking=False)
        if kind == "canon":
            self.canon[a][t][layer].copy_(dev(arr))
        elif kind == "factor":
            c, fi = fac_keys[a]
            lrel = layer - c.factors[fi].layer0
            self.factors[a][0][lrel].copy_(dev(arr[0]))
            self.factors[a][1][lrel].copy_(dev(arr[1]))
        else:
            ch = self.wl.chunks[a]
            idx = self.slot_rows(ch)
            self.pool[t][layer].view(-1, self.F)[idx] = dev(arr)

    def _stage(self, jobs, fac_keys):
        batch = 4 * _threads()
        with ThreadPoolExecutor(_threads()) as ex:
            for i in range(0, len(jobs), batch):
                part = jobs[i:i + batch]
                for job, arr in zip(part, ex.map(lambda j: self._draw(j, fac_keys), part)):
                    self._put(job, arr, fac_keys)

    # ------------------------------------------------------------------ descriptors
    def slot_rows(self, ch: ChunkSpec) -> torch.Tensor:
        """Flat pool row (page * P + offset) of every token of a paged chunk."""
        s = ch.slot0 + np.arange(ch.num_tokens)
        rows = ch.block_table[s // self.P].astype(np.int64) * self.P + s % self.P
        return torch.from_numpy(rows).to(self.device)

    def _desc(self, c: ChunkSpec) -> abi.ChunkDesc:
        nt = self.lay.num_tensors
        kw = dict(num_tokens=c.num_tokens, delta=c.delta, flags=c.flags, slot0=c.slot0,
                  positions=self.positions.get(c.index))
        if c.block_table is not None:
            kw["block_table"] = c.block_table
        elif c.dst_buffer >= 0:
            buf = self.dense[c.dst_buffer]
            rows = buf[0].shape[1]
            off = c.dst_row0 * self.F * self.es
            kw.update(k_dst=buf[0].data_ptr() + off, v_dst=(buf[1].data_ptr() + off) if nt == 2 else None,
                      dst_layer_stride=rows * self.F)
        if not c.in_place:
            src = self.canon[c.canon_id]
            kw.update(k_src=src[0], v_src=src[1] if nt == 2 else None)
        if c.patched:
            fl = []
            for f in c.factors:
                u, v = self.factors[(f.key, f.slot)]
                fl.append(dict(u=u, v=v, tensor=f.tensor, col0=f.col0, width=f.width, rank=f.rank,
                               layer0=f.layer0))
            kw["factors"] = fl
        return abi.ChunkDesc(**kw)

    def copy_descs(self) -> list:
        """The same chunks with delta 0 and no patch: the operator then copies each
        out-of-place chunk through its own access pattern (in-place chunks do nothing)."""
        out = []
        for c in self.wl.chunks:
            d = self._desc(c)
            d.c.delta = 0
            d.c.flags = d.c.flags & ~(abi.PATCH | abi.POSITIONS)
            d.c.num_factors = 0
            out.append(d)
        return out

    def copy_bytes(self) -> int:
        """Bytes moved by copy_descs(): each out-of-place row read once and written once."""
        return sum(self.L * self.lay.num_tensors * 2 * c.num_tokens * self.F * self.es
                   for c in self.wl.chunks if not c.in_place)

    # ------------------------------------------------------------------ running
    def run(self, stream=None, chunks: Optional[Sequence[int]] = None) -> None:
        descs = self.descs if chunks is None else [self.descs[i] for i in chunks]
        abi.rehydrate_batched(self.layout, descs, self.pool_desc, self.workspace, stream)

    def prepared(self, stream=None) -> abi.PreparedBatch:
        """The whole batch marshalled once; .call() issues it again."""
        return abi.PreparedBatch(self.layout, self.descs, self.pool_desc, self.workspace, stream)

    def plan(self, stream=None) -> abi.Plan:
        return abi.plan_upload(self.layout, self.descs, self.pool_desc, self.workspace, stream)

    # ------------------------------------------------------------------ reading back
    def out_rows(self, c: ChunkSpec, layer: int, tensor: int, rows: Optional[Sequence[int]] = None) -> np.ndarray:
        """Destination rows of chunk c (all tokens, or `rows`), as stored (uint16 codes or float32)."""
        r = np.arange(c.num_tokens) if rows is None else np.asarray(rows)
        if c.block_table is not None:
            s = c.slot0 + r
            flat = c.block_table[s // self.P].astype(np.int64) * self.P + s % self.P
            t = self.pool[tensor][layer].view(-1, self.F)[torch.from_numpy(flat).to(self.device)]
        else:
            t = self.dense[c.dst_buffer][tensor][layer][torch.from_numpy(c.dst_row0 + r).to(self.device)]
        a = t.cpu().numpy()
        return a.view(np.uint16) if self.lay.dtype == BF16 else a

    def algorithmic_bytes(self) -> int:
        """Bytes the operator must move: each source byte read once, each output byte
        written once, factors read once per chunk-layer (survivors move K only)."""
        es, F, L = self.es, self.F, self.L
        total = 0
        seen_v = set()
        for c in self.wl.chunks:
            T = c.num_tokens
            if c.in_place and not c.patched:
                cols = F if self.lay.family == GQA else self.lay.rope_dim
                total += L * 2 * T * cols * es
                continue
            total += L * self.lay.num_tensors * 2 * T * F * es
            if c.positions is not None and c.flags & POSITIONS:   # the (t, h, w) offsets, read once per chunk
                total += T * 3 * 4
            if c.patched:
                for f in c.factors:
                    total += (L - f.layer0) * T * f.rank * es
                    vkey = (f.basis, f.slot, f.layer0, f.width, f.rank) if f.basis >= 0 else (id(c), id(f))
                    if vkey not in seen_v:   # a shared basis is read once per layer
                        seen_v.add(vkey)
                        total += (L - f.layer0) * f.rank * f.width * es
        return total
