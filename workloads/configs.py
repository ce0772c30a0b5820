"""The five synthetic workloads of the Kamera reuse operator, as seeded generators.

Shapes follow the backbones and workloads the Kamera preprint names
("Kamera: Unified Position-Invariant Multimodal KV Cache for Training-Free
Reuse", Fig. 2 panels b-c and §5-§6):

  C1  single-layer GQA, 2 KV heads x 64, fp32, 1 chunk of 256 tokens, rank-8 patch
  C2  GQA like Qwen2.5-VL-7B (28 layers, K,V in R^512 = 4 heads x 128), bf16,
      8 video segments of 1024 tokens (16 frames x 64 tokens), rank-32 patch
  C3  MLA like DeepSeek-V2-Lite / Kimi-VL (27 layers, c_KV 512 + k_rope 64),
      16 chunks of 1024 tokens, rank-32 patches on the 576-wide row and the rope band
  C4  MHA 7B (32 layers, 32 heads x 128), 4 two-page-document chunks of 2048
      tokens; all 6 orderings of the first three, one stored patch per chunk
  C5  sliding-window deque like Qwen3-VL (36 layers, 8 heads x 128), 64 ragged
      screenshot/frame chunks in [256, 2048]: 48 survivors relocated in place by
      -(evicted length), 16 recalled chunks rehydrated with a fresh rank-32 patch,
      all into a 16-token paged pool through a seeded random block table

Every block of random numbers is addressable: it is drawn from its own
``numpy.random.default_rng([root, purpose, ...])`` stream, so any single
(chunk, layer, tensor) block can be regenerated on its own, for example to
check sampled rows of a large run without materialising all of it.

Values are drawn in float32, then stored in the layout's dtype (bfloat16 as raw
uint16 bit patterns, converted by torch's round-to-nearest-even cast). The
stored values are the inputs; nothing downstream relies on how they were drawn.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

# ---- enums shared with the C-ABI by value (plain integers) -------------------
GQA, MLA = 0, 1
F32, BF16 = 0, 1
NEOX, GPTJ = 0, 1
PATCH, IN_PLACE, POSITIONS = 1, 2, 4

CONFIG_NAMES = ("C1", "C2", "C3", "C4", "C5")
_ROOT = {"C1": 1001, "C2": 1002, "C3": 1003, "C4": 1004, "C5": 1005}

# draw purposes (second entry of every seed key)
_P_CANON, _P_OUTLIER, _P_DELTA, _P_LEN, _P_ROLE, _P_FACTOR, _P_TABLE, _P_POOL, _P_BASIS = range(1, 10)

BF16_SENTINEL = 0x7FA5  # a quiet-NaN bit pattern no real output produces
F32_SENTINEL = 0x7FC0DEAD


@dataclass(frozen=True)
class LayoutSpec:
    family: int
    dtype: int
    num_layers: int
    num_kv_heads: int = 0
    head_dim: int = 0
    latent_dim: int = 0
    rope_dim: int = 0
    pairing: int = NEOX
    rope_base: float = 10000.0
    page_size: int = 16
    mrope_section: tuple = (0, 0, 0)   # rotary pairs following the t, h, w offsets (all 0: 1-D)

    @property
    def d_rot(self) -> int:
        return self.head_dim if self.family == GQA else self.rope_dim

    @property
    def row_width(self) -> int:
        if self.family == GQA:
            return self.num_kv_heads * self.head_dim
        return self.latent_dim + self.rope_dim

    @property
    def num_tensors(self) -> int:
        return 2 if self.family == GQA else 1

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == BF16 else 4

    @property
    def np_storage(self):
        return np.uint16 if self.dtype == BF16 else np.float32


@dataclass
class FactorSpec:
    """One low-rank patch U.Vt added to columns [col0, col0+width) of a tensor."""
    tensor: int
    col0: int
    width: int
    rank: int
    sigma: np.ndarray
    key: int          # identifies the factor draw: default_rng([root, FACTOR, key, layer, slot])
    slot: int         # factor slot (0..3), part of the draw key
    layer0: int = 0   # first patched layer (layers below it carry no factor)
    basis: int = -1   # >= 0: V is the shared per-layer basis default_rng([root, BASIS, basis, layer, slot])


@dataclass
class ChunkSpec:
    index: int
    num_tokens: int
    delta: int
    flags: int
    canon_id: int                     # which canonical block set feeds this chunk
    factors: List[FactorSpec] = field(default_factory=list)
    # destination: either a dense buffer (rows [dst_row0, dst_row0+T)) or pool pages
    dst_buffer: int = -1
    dst_row0: int = 0
    block_table: Optional[np.ndarray] = None
    slot0: int = 0
    role: str = "rehydrate"          # "rehydrate" | "survivor"
    positions: Optional[np.ndarray] = None   # [T][3] int32 (t, h, w) offsets, with the POSITIONS flag

    @property
    def patched(self) -> bool:
        return bool(self.flags & PATCH)

    @property
    def in_place(self) -> bool:
        return bool(self.flags & IN_PLACE)


@dataclass
class Workload:
    name: str
    root: int
    layout: LayoutSpec
    chunks: List[ChunkSpec]
    canon_tokens: dict                 # canon_id -> T
    dense_rows: List[int]              # rows of each dense output buffer
    num_pages: int = 0                 # pool pages (0: no pool)
    outlier_scale: float = 1.0
    outliers_per_head: int = 0
    description: str = ""

    # -------------------------------------------------------------- helpers
    def _to_storage(self, x32: np.ndarray) -> np.ndarray:
        if self.layout.dtype == F32:
            return np.ascontiguousarray(x32, dtype=np.float32)
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    def outlier_columns(self, layer: int) -> np.ndarray:
        """Key columns scaled up in this layer (4 distinct channels per KV head)."""
        if self.outliers_per_head == 0:
            return np.zeros(0, dtype=np.int64)
        rng = np.random.default_rng([self.root, _P_OUTLIER, layer])
        hd = self.layout.head_dim
        cols = [h * hd + rng.choice(hd, size=self.outliers_per_head, replace=False)
                for h in range(self.layout.num_kv_heads)]
        return np.sort(np.concatenate(cols))

    def canonical(self, canon_id: int, layer: int, tensor: int) -> np.ndarray:
        """Position-free stored rows KV(B|empty) of one chunk/layer/tensor: [T][F]."""
        T = self.canon_tokens[canon_id]
        F = self.layout.row_width
        rng = np.random.default_rng([self.root, _P_CANON, canon_id, layer, tensor])
        x = rng.standard_normal((T, F), dtype=np.float32)
        if tensor == 0 and self.outliers_per_head:
            x[:, self.outlier_columns(layer)] *= np.float32(self.outlier_scale)
        return self._to_storage(x)

    def pool_rows(self, chunk: ChunkSpec, layer: int, tensor: int) -> np.ndarray:
        """Rows a survivor chunk holds in the pool before the window slides: [T][F]."""
        F = self.layout.row_width
        rng = np.random.default_rng([self.root, _P_POOL, chunk.index, layer, tensor])
        x = rng.standard_normal((chunk.num_tokens, F), dtype=np.float32)
        return self._to_storage(x)

    def _factor_fp64(self, f: FactorSpec, T: int, layer: int):
        rng = np.random.default_rng([self.root, _P_FACTOR, f.key, layer, f.slot])
        def orth(n, m):
            g = rng.standard_normal((n, m))
            if n < m:   # no n x m matrix has orthonormal columns: keep the scaled Gaussian
                return g / np.sqrt(n)
            q, r = np.linalg.qr(g)
            return q * np.sign(np.diag(r))[None, :]
        q1 = orth(T, f.rank)
        if f.basis >= 0:   # a basis shared by every chunk whose factor names it
            rng = np.random.default_rng([self.root, _P_BASIS, f.basis, layer, f.slot])
        q2 = orth(f.width, f.rank)
        return q1 * f.sigma[None, :], q2

    def factor(self, chunk: ChunkSpec, fi: int, layer: int):
        """(U.Sigma [T][m], V [width][m]) of factor fi at `layer`, in storage dtype;
        the patch they encode is U V^T."""
        f = chunk.factors[fi]
        u, v = self._factor_fp64(f, chunk.num_tokens, layer)
        return (self._to_storage(u.astype(np.float32)),
                self._to_storage(v.astype(np.float32)))

    @property
    def total_tokens(self) -> int:
        return sum(c.num_tokens for c in self.chunks)


def _sigma(first: float, ratio: float, m: int) -> np.ndarray:
    return first * ratio ** np.arange(m, dtype=np.float64)


def _gqa_factors(key, F, m, sigma, layer0=0):
    return [FactorSpec(tensor=0, col0=0, width=F, rank=m, sigma=sigma, key=key, slot=0, layer0=layer0),
            FactorSpec(tensor=1, col0=0, width=F, rank=m, sigma=sigma, key=key, slot=1, layer0=layer0)]


FRAME_TOKENS, FRAME_GRID = 64, 8   # a video frame / screenshot tile: 8 x 8 merged patches


def grid_positions(num_tokens: int, start: int, frame_tokens: int = FRAME_TOKENS,
                   grid_w: int = FRAME_GRID) -> np.ndarray:
    """(t, h, w) position ids of a run of visual tokens placed at `start`: token k is
    patch (k % frame_tokens) of frame k // frame_tokens, in row-major order on a grid
    grid_w wide; each component is offset by `start` (three-section M-RoPE ids of
    Qwen2-VL-style backbones). [T][3] int32."""
    k = np.arange(num_tokens, dtype=np.int64)
    patch_ = k % frame_tokens
    pos = np.stack([k // frame_tokens, patch_ // grid_w, patch_ % grid_w], axis=1) + int(start)
    return pos.astype(np.int32)


def mrope_sections(d_rot: int) -> tuple:
    """Blocked t/h/w split of the d_rot/2 rotary pairs in the 1 : 1.5 : 1.5 proportion of
    Qwen2-VL's (16, 24, 24) for 128-wide heads."""
    n = d_rot // 2
    t = n // 4
    h = (n - t) // 2
    return (t, h, n - t - h)


def make_workload(name: str, *, num_layers: Optional[int] = None, num_chunks: Optional[int] = None,
                  tokens: Optional[int] = None, rank: Optional[int] = None,
                  patch: bool = True, max_tokens: Optional[int] = None,
                  patch_layer0: Optional[int] = None, shared_basis: bool = False,
                  positions: bool = False, page_order: str = "random") -> Workload:
    """Build config `name` (C1..C5). Keyword overrides shrink it for fast tests;
    patch_layer0 makes every factor start at that layer (e.g. L // 2: the deep-half
    patches of the preprint's Table 2, layers below it carry no patch); shared_basis
    gives every chunk the same per-layer V for a factor slot (the preprint's §4: the
    deficit's directions are shared across items, only the coefficients U differ);
    positions re-anchors every rehydrated chunk token by token with three-section
    (t, h, w) ids of 64-token frames placed at the chunk's start (QV-PIC Eq. 2: keys
    stored unrotated, M-RoPE applied with the request positions); survivors keep delta.
    page_order "physical" gives a paged workload consecutive page ids, chunk after chunk,
    instead of its seeded random block table (same chunks, same pool size)."""
    if page_order not in ("random", "physical"):
        raise ValueError(page_order)
    wl = _make_workload(name, num_layers=num_layers, num_chunks=num_chunks, tokens=tokens, rank=rank,
                        patch=patch, max_tokens=max_tokens, page_order=page_order)
    if positions:
        import dataclasses
        wl.layout = dataclasses.replace(wl.layout, mrope_section=mrope_sections(wl.layout.d_rot))
        for c in wl.chunks:
            if not c.in_place:
                c.positions = grid_positions(c.num_tokens, c.delta)
                c.flags |= POSITIONS
        wl.description += "; per-token (t, h, w) re-anchoring"
    if patch_layer0 is not None:
        if not 0 <= patch_layer0 < wl.layout.num_layers:
            raise ValueError("patch_layer0 outside [0, L)")
        for c in wl.chunks:
            for f in c.factors:
                f.layer0 = patch_layer0
    if shared_basis:
        for c in wl.chunks:
            for f in c.factors:
                f.basis = f.slot
    return wl


def _make_workload(name: str, *, num_layers: Optional[int], num_chunks: Optional[int], tokens: Optional[int],
                   rank: Optional[int], patch: bool, max_tokens: Optional[int], page_order: str) -> Workload:
    root = _ROOT[name]
    if name == "C1":
        lay = LayoutSpec(GQA, F32, num_layers or 1, num_kv_heads=2, head_dim=64, rope_base=10000.0)
        n = num_chunks or 1
        T = tokens or 256
        m = 8 if rank is None else rank
        deltas = np.random.default_rng([root, _P_DELTA]).integers(0, 4096, size=n, endpoint=True)
        F = lay.row_width
        chunks = [ChunkSpec(index=i, num_tokens=T, delta=int(deltas[i]), flags=PATCH if patch else 0,
                            canon_id=i, factors=_gqa_factors(i, F, m, _sigma(0.5, 0.8, m)) if m else [],
                            dst_buffer=i, dst_row0=0) for i in range(n)]
        return Workload(name, root, lay, chunks, {i: T for i in range(n)}, [T] * n,
                        description="single-layer GQA, 2x64, fp32, rank-8 patch")

    if name == "C2":
        lay = LayoutSpec(GQA, BF16, num_layers or 28, num_kv_heads=4, head_dim=128, rope_base=1e6)
        n = num_chunks or 8
        T = tokens or 1024
        m = 32 if rank is None else rank
        deltas = np.random.default_rng([root, _P_DELTA]).integers(0, 32768, size=n, endpoint=True)
        F = lay.row_width
        chunks = [ChunkSpec(index=i, num_tokens=T, delta=int(deltas[i]), flags=PATCH if patch else 0,
                            canon_id=i, factors=_gqa_factors(i, F, m, _sigma(0.3, 0.9, m)) if m else [],
                            dst_buffer=i, dst_row0=0) for i in range(n)]
        return Workload(name, root, lay, chunks, {i: T for i in range(n)}, [T] * n,
                        outlier_scale=8.0, outliers_per_head=4,
                        description="GQA VL-7B-like, 8 video segments x 1024 tokens")

    if name == "C3":
        lay = LayoutSpec(MLA, BF16, num_layers or 27, latent_dim=512, rope_dim=64, rope_base=10000.0)
        n = num_chunks or 16
        T = tokens or 1024
        m = 32 if rank is None else rank
        deltas = np.random.default_rng([root, _P_DELTA]).integers(0, 65536, size=n, endpoint=True)
        sig = _sigma(0.3, 0.9, m)
        chunks = []
        for i in range(n):
            fac = [FactorSpec(tensor=0, col0=0, width=576, rank=m, sigma=sig, key=i, slot=0),
                   FactorSpec(tensor=0, col0=512, width=64, rank=m, sigma=sig, key=i, slot=1)] if m else []
            chunks.append(ChunkSpec(index=i, num_tokens=T, delta=int(deltas[i]),
                                    flags=PATCH if patch else 0, canon_id=i, factors=fac,
                                    dst_buffer=i, dst_row0=0))
        return Workload(name, root, lay, chunks, {i: T for i in range(n)}, [T] * n,
                        description="MLA V2-Lite-like, 16 chunks x 1024 tokens")

    if name == "C4":
        lay = LayoutSpec(GQA, BF16, num_layers or 32, num_kv_heads=32, head_dim=128, rope_base=10000.0)
        T = tokens or 2048
        m = 32 if rank is None else rank
        F = lay.row_width
        import itertools
        orders = list(itertools.permutations(range(3)))
        chunks = []
        for o, perm in enumerate(orders):
            seq = list(perm) + [3]
            for slot, cid in enumerate(seq):
                chunks.append(ChunkSpec(index=len(chunks), num_tokens=T, delta=slot * T,
                                        flags=PATCH if patch else 0, canon_id=cid,
                                        factors=_gqa_factors(cid, F, m, _sigma(0.3, 0.9, m)) if m else [],
                                        dst_buffer=o, dst_row0=slot * T))
        if num_chunks is not None:
            chunks = chunks[:num_chunks]
        nbuf = max(c.dst_buffer for c in chunks) + 1
        return Workload(name, root, lay, chunks, {i: T for i in range(4)}, [4 * T] * nbuf,
                        description="MHA 7B reorder: 6 orderings x 4 chunks x 2048 tokens")

    if name == "C5":
        lay = LayoutSpec(GQA, BF16, num_layers or 36, num_kv_heads=8, head_dim=128, rope_base=1e6,
                         page_size=16)
        n = num_chunks or 64
        m = 32 if rank is None else rank
        lo, hi = 256, (max_tokens or 2048)
        lens = np.random.default_rng([root, _P_LEN]).integers(lo, hi, size=n + 4, endpoint=True)
        if tokens is not None:
            lens = np.minimum(lens, tokens)
        evicted, lens = lens[:4], lens[4:]
        E = int(evicted.sum())
        n_recall = n // 4
        role_perm = np.random.default_rng([root, _P_ROLE]).permutation(n)
        recalled = set(int(i) for i in role_perm[:n_recall])
        P = lay.page_size
        pages_needed = [int(-(-int(L_) // P)) for L_ in lens]
        num_pages = int(np.ceil(1.25 * sum(pages_needed)))
        table = np.random.default_rng([root, _P_TABLE]).permutation(num_pages).astype(np.int32)
        if page_order == "physical":
            table = np.arange(num_pages, dtype=np.int32)
        F = lay.row_width
        chunks, cursor, pos = [], 0, 0
        for i in range(n):
            T = int(lens[i])
            bt = table[cursor:cursor + pages_needed[i]].copy()
            cursor += pages_needed[i]
            if i in recalled:
                chunks.append(ChunkSpec(index=i, num_tokens=T, delta=pos, flags=PATCH if patch else 0,
                                        canon_id=i,
                                        factors=_gqa_factors(i, F, m, _sigma(0.3, 0.9, m)) if m else [],
                                        block_table=bt, slot0=0, role="rehydrate"))
            else:
                chunks.append(ChunkSpec(index=i, num_tokens=T, delta=-E, flags=IN_PLACE, canon_id=i,
                                        block_table=bt, slot0=0, role="survivor"))
            pos += T
        return Workload(name, root, lay, chunks, {c.index: c.num_tokens for c in chunks}, [],
                        num_pages=num_pages,
                        description=f"GQA deque: {n} ragged chunks, {n - n_recall} survivors "
                                    f"(delta=-{E}), {n_recall} recalled, 16-token pages")
    raise KeyError(name)
