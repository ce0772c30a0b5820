"""Helpers shared by the GPU parity tests: run a workload, compare with the oracle."""
from __future__ import annotations

import sys
from typing import List, Optional, Sequence

import numpy as np
import torch

from oracle import tolerance as tol
from tests.expect import expect_block
from workloads.configs import (BF16, BF16_SENTINEL, F32_SENTINEL, GQA, IN_PLACE, MLA, NEOX, PATCH, ChunkSpec,
                               FactorSpec, LayoutSpec, Workload)


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def touched_tensors(wl: Workload, ch: ChunkSpec) -> List[int]:
    if wl.layout.family == MLA:
        return [0]
    if ch.in_place and not (ch.patched and any(f.tensor == 1 for f in ch.factors)):
        return [0]
    return [0, 1]


def compare(dw, ch: ChunkSpec, layer: int, tensor: int, rows: Optional[Sequence[int]] = None) -> dict:
    e = expect_block(dw.wl, ch, layer, tensor, rows)
    g = dw.out_rows(ch, layer, tensor, rows)
    if dw.lay.dtype == BF16:
        res = tol.check_bf16(g, e.y, e.r, e.S, e.n, e.A)
    else:
        res = tol.check_f32(g, e.y, e.S, e.n, e.A)
    res["where"] = (ch.index, layer, tensor)
    if res["fail"]:
        bad = np.argwhere(res["mask"])[:5]
        res["examples"] = [(tuple(int(v) for v in b), float(e.y[tuple(b)]), int(np.asarray(g)[tuple(b)].view(
            np.uint16 if dw.lay.dtype == BF16 else np.uint32))) for b in bad]
    return res


def check_all(dw, layers: Optional[Sequence[int]] = None, rows_per_chunk: Optional[int] = None,
              seed: int = 0) -> dict:
    """Compare every (chunk, layer, tensor) block (or sampled rows) with the oracle."""
    rng = np.random.default_rng(seed)
    tot = {"n": 0, "fail": 0, "p2_only": 0, "exact": 0, "bad": []}
    for ch in dw.wl.chunks:
        if ch.num_tokens == 0:
            continue
        for layer in (range(dw.L) if layers is None else layers):
            for t in touched_tensors(dw.wl, ch):
                rows = None
                if rows_per_chunk is not None and ch.num_tokens > rows_per_chunk:
                    rows = np.unique(np.concatenate([[0, ch.num_tokens - 1],
                                                     rng.choice(ch.num_tokens, rows_per_chunk, replace=False)]))
                r = compare(dw, ch, layer, t, rows)
                for k in ("n", "fail", "p2_only", "exact"):
                    tot[k] += r[k]
                if r["fail"]:
                    tot["bad"].append((r["where"], r.get("examples")))
    return tot


def sentinel_code(dtype: int) -> int:
    return BF16_SENTINEL if dtype == BF16 else F32_SENTINEL


def pool_untouched_ok(dw) -> bool:
    """Every pool slot that no chunk owns still holds the sentinel (bit-exact)."""
    if dw.pool is None:
        return True
    P, F = dw.P, dw.F
    used = np.zeros(dw.wl.num_pages * P, dtype=bool)
    for ch in dw.wl.chunks:
        if ch.block_table is None or ch.num_tokens == 0:
            continue
        s = ch.slot0 + np.arange(ch.num_tokens)
        used[ch.block_table[s // P].astype(np.int64) * P + s % P] = True
    free = torch.from_numpy(np.nonzero(~used)[0]).to(dw.device)
    code = sentinel_code(dw.lay.dtype)
    for t in dw.pool:
        flat = t.view(dw.L, -1, F)
        vals = flat[:, free, :]
        if dw.lay.dtype == BF16:
            ok = bool((vals.view(torch.int16) == np.uint16(code).view(np.int16).item()).all())
        else:
            ok = bool((vals.view(torch.int32) == int(np.uint32(code).view(np.int32))).all())
        if not ok:
            return False
    return True


def factor(key, slot, tensor, col0, width, rank, sigma0=0.3, layer0=0) -> FactorSpec:
    return FactorSpec(tensor=tensor, col0=col0, width=width, rank=rank,
                      sigma=sigma0 * 0.9 ** np.arange(rank), key=key, slot=slot, layer0=layer0)


def custom_workload(layout: LayoutSpec, chunks: List[ChunkSpec], *, dense_rows=None, num_pages=0,
                    root=4242) -> Workload:
    canon = {c.canon_id: c.num_tokens for c in chunks}
    if dense_rows is None:
        nb = max([c.dst_buffer for c in chunks] + [-1]) + 1
        dense_rows = [0] * nb
        for c in chunks:
            if c.dst_buffer >= 0:
                dense_rows[c.dst_buffer] = max(dense_rows[c.dst_buffer], c.dst_row0 + c.num_tokens, 1)
    return Workload("custom", root, layout, chunks, canon, dense_rows, num_pages=num_pages)


def gqa_chunks(n, T, delta, H, hd, rank, patch=True, flags=None):
    F = H * hd
    return [ChunkSpec(index=i, num_tokens=T if isinstance(T, int) else T[i],
                      delta=delta if isinstance(delta, int) else delta[i],
                      flags=(PATCH if patch else 0) if flags is None else flags, canon_id=i,
                      factors=[factor(i, 0, 0, 0, F, rank), factor(i, 1, 1, 0, F, rank)] if rank else [],
                      dst_buffer=i) for i in range(n)]
