"""Oracle expectations for workload blocks (test infrastructure).

Joins the seeded inputs (workloads/) with the fp64 oracle (oracle/): for one
chunk, layer and tensor, and an optional subset of token rows, returns the
exact fp64 result y, its once-rounded storage code r and the absolute-term sum
S used by the rounding-error bound.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

import oracle.kamera_oracle as O
from workloads.configs import BF16, GQA, POSITIONS, ChunkSpec, Workload


@dataclass
class Expect:
    y: np.ndarray       # fp64 exact result [rows][F]
    r: np.ndarray       # rounded to storage dtype (uint16 codes or float32)
    S: np.ndarray       # sum of |terms|
    n: int              # number of fp32 roundings allowed by the bound
    src: np.ndarray     # the stored input rows (storage dtype)
    A: np.ndarray = None  # angle term of the bound (oracle.kamera_oracle.angle_terms)


def source_rows(wl: Workload, ch: ChunkSpec, layer: int, tensor: int) -> np.ndarray:
    """Stored rows the operator reads: the canonical, or the pool rows of a survivor."""
    if ch.in_place:
        return wl.pool_rows(ch, layer, tensor)
    return wl.canonical(ch.canon_id, layer, tensor)


def oracle_factors(wl: Workload, ch: ChunkSpec, layer: int, rows: Optional[Sequence[int]] = None):
    out = []
    for fi, f in enumerate(ch.factors):
        if layer < f.layer0:
            continue
        u, v = wl.factor(ch, fi, layer)
        u64 = O.upcast(u, wl.layout.dtype)
        if rows is not None:
            u64 = u64[np.asarray(rows)]
        # the oracle takes the right factor as V^T [m][width]
        out.append(O.Factor(f.tensor, f.col0, u64, O.upcast(v, wl.layout.dtype).T))
    return out


def expect_block(wl: Workload, ch: ChunkSpec, layer: int, tensor: int,
                 rows: Optional[Sequence[int]] = None) -> Expect:
    lay = wl.layout
    src = source_rows(wl, ch, layer, tensor)
    if rows is not None:
        src = src[np.asarray(rows)]
    x = O.upcast(src, lay.dtype)
    facs = oracle_factors(wl, ch, layer, rows)
    bands = O.band_offsets(lay.family, lay.num_kv_heads, lay.head_dim, lay.latent_dim)
    d_rot = O.rotary_width(lay.family, lay.head_dim, lay.rope_dim)
    rotate_this = tensor == 0          # K for GQA/MHA, the whole row for MLA
    pos = None
    if ch.positions is not None and ch.flags & POSITIONS:   # offsets without the flag are ignored
        pos = ch.positions if rows is None else ch.positions[np.asarray(rows)]
    kw = dict(tensor=tensor, delta=ch.delta, rotate_this=rotate_this, bands=bands, d_rot=d_rot,
              base=lay.rope_base, pairing=lay.pairing, factors=facs, patch=ch.patched, positions=pos,
              sections=lay.mrope_section)
    y = O.rehydrate_tensor(x, family=lay.family, **kw)
    S = O.abs_terms(x, **kw)
    A = O.angle_terms(x, **kw)
    m_total = sum(f.u.shape[1] for f in facs if f.tensor == tensor) if ch.patched else 0
    return Expect(y=y, r=O.round_to(y, lay.dtype), S=S, n=m_total + 4, src=src, A=A)
