"""Plain fp64 CPU oracle of the Kamera reuse operator.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or call this module. The product path
(the HIP library and its Python binding) never imports it, and this module
imports nothing from the product path.

What it computes, and where the pages say so (page titles as cited):
  "Kamera: Unified Position-Invariant Multimodal KV Cache for Training-Free Reuse"
  (the preprint, abbreviated KAMERA below) and its Dutch summary page on
  gist.science (abbreviated SUMMARY).

  Eq. 1 (KAMERA §1; stated cleanly in SUMMARY §2):
      KV^(B|A) = R(delta) . KV(B|empty) + U_m V_m^T
  KAMERA §3: R(delta) re-rotates the stored keys' RoPE phase by
      delta = p1 - p0; it composes exactly, R(delta)R(p0) = R(p1); V is untouched.
      GQA/MHA relocate the full key; MLA rotates only the 64-d decoupled k_rope
      (k_pe) while the latent c_KV is reused as stored. The patch touches both
      channels (K and V; or c_KV and the k_rope band).
  KAMERA App. A (serve listing): rotate the rope band first, then add the
      rank-m product U @ V^T to K and to V; factors are stored as (U*Sigma, V^T).
  KAMERA §5: sliding-window survivors need the rotation only.
  KAMERA §6: the rebuilt KV lands in a paged KV pool.

Readings where the pages are silent:
  * frequencies: textbook RoPE, theta_i = base^(-2i/d_rot), i < d_rot/2;
  * pairing: NeoX half split (i, i + d_rot/2) unless GPT-J (2i, 2i+1) is asked;
  * sign: a' = a cos(phi) - b sin(phi), b' = a sin(phi) + b cos(phi), phi = delta*theta_i,
    i.e. multiplication of (a + i b) by exp(+i phi), as RoFormer defines RoPE;
  * order: rotate, then add the (unrotated) patch;
  * output rounding: the exact fp64 value is rounded once to the output dtype,
    round-to-nearest-even.

All arithmetic is fp64 on the exact fp64 upcast of the stored inputs. There is
no blocking, fusion or reordering beyond the definition: the patch is a plain
loop of rank-1 updates (no BLAS), so a BLAS product stays an independent check.
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

GQA, MLA = 0, 1
F32, BF16 = 0, 1
NEOX, GPTJ = 0, 1


# ----------------------------------------------------------------------------
# storage <-> fp64
# ----------------------------------------------------------------------------
def upcast(x: np.ndarray, dtype: int) -> np.ndarray:
    """Exact fp64 value of stored elements (bf16 given as uint16 bit patterns)."""
    if dtype == BF16:
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        with np.errstate(invalid="ignore"):
            return bits.view(np.float32).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def round_bf16(y: np.ndarray) -> np.ndarray:
    """Round fp64 values once to bfloat16, round-to-nearest, ties to even.

    bfloat16 keeps 8 significant bits and fp32's exponent range. For y = f * 2^e
    with 0.5 <= |f| < 1 the bf16 grid spacing is 2^(e-8) (2^-133 below the
    normal range); y divided by that spacing is an exact fp64 operation (a power
    of two), so rint() on it is exactly the ties-to-even decision. The rounded
    value is a bf16 number, hence exact in fp32, whose top 16 bits are the code.
    """
    y = np.asarray(y, dtype=np.float64)
    _, e = np.frexp(y)
    e = np.maximum(e, -125)                     # subnormal bf16 spacing is 2^-133
    spacing = np.ldexp(1.0, e - 8)
    r = np.rint(y / spacing) * spacing          # exact: only a power-of-two scaling
    with np.errstate(over="ignore", invalid="ignore"):
        r32 = r.astype(np.float32)              # exact unless |r| >= 2^128 (-> inf)
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.isnan(y), np.uint16(0x7FC0), bits)
    return bits


def round_f32(y: np.ndarray) -> np.ndarray:
    """Round fp64 values once to fp32 (IEEE cast, round-to-nearest-even)."""
    return np.asarray(y, dtype=np.float64).astype(np.float32)


def round_to(y: np.ndarray, dtype: int) -> np.ndarray:
    return round_bf16(y) if dtype == BF16 else round_f32(y)


# ----------------------------------------------------------------------------
# R(delta): RoPE phase re-rotation (KAMERA §1 Eq. 1, §3 "Relocate")
# ----------------------------------------------------------------------------
def inv_freq(d_rot: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/d_rot) for i = 0 .. d_rot/2 - 1 (textbook RoPE), fp64."""
    i = np.arange(d_rot // 2, dtype=np.float64)
    return np.float64(base) ** (-2.0 * i / d_rot)


def pair_columns(d_rot: int, pairing: int) -> Tuple[np.ndarray, np.ndarray]:
    """Column offsets (p_i, q_i) inside one rotary band that rotate together."""
    i = np.arange(d_rot // 2)
    if pairing == NEOX:
        return i, i + d_rot // 2
    if pairing == GPTJ:
        return 2 * i, 2 * i + 1
    raise ValueError(pairing)


def phases(delta: int, d_rot: int, base: float) -> Tuple[np.ndarray, np.ndarray]:
    """cos and sin of phi_i = delta * theta_i, all in fp64 (delta is an exact integer)."""
    phi = np.float64(delta) * inv_freq(d_rot, base)
    return np.cos(phi), np.sin(phi)


def rotate(x: np.ndarray, delta: int, band_offsets: Sequence[int], d_rot: int, base: float,
           pairing: int) -> np.ndarray:
    """R(delta) applied to every rotary band of the rows x ([T][F], fp64).

    Bands start at `band_offsets` and are d_rot wide; every other column is
    copied unchanged (KAMERA §3: V and c_KV are never rotated).
    """
    y = np.array(x, dtype=np.float64, copy=True)
    c, s = phases(delta, d_rot, base)
    p, q = pair_columns(d_rot, pairing)
    for o in band_offsets:
        a = x[:, o + p]
        b = x[:, o + q]
        y[:, o + p] = a * c - b * s
        y[:, o + q] = a * s + b * c
    return y


# ----------------------------------------------------------------------------
# Per-token re-anchoring (QV-PIC Eq. 2: the backbone's own M-RoPE applied at the request
# positions; KAMERA §4: a uniform shift of (t, h, w) is the 1-D rotation R(delta))
# ----------------------------------------------------------------------------
def pair_sections(d_rot: int, sections: Sequence[int]) -> np.ndarray:
    """Position component (0 = t, 1 = h, 2 = w) that drives each rotary pair i.

    Sections are blocked: the first sections[0] pairs follow t, the next sections[1]
    follow h, the rest follow w. All zero means a 1-D rotation (every pair follows
    component 0)."""
    n = d_rot // 2
    sec = np.zeros(n, dtype=np.int64)
    if any(sections):
        if sum(sections) != n:
            raise ValueError("sections must add up to d_rot / 2")
        sec[sections[0]:sections[0] + sections[1]] = 1
        sec[sections[0] + sections[1]:] = 2
    return sec


def token_phases(positions: np.ndarray, d_rot: int, base: float, sections: Sequence[int]):
    """cos and sin of phi[t, i] = positions[t, sec(i)] * theta_i, fp64 ([T][d_rot/2])."""
    pos = np.asarray(positions, dtype=np.int64).reshape(len(positions), -1)
    comp = pos[:, pair_sections(d_rot, sections)].astype(np.float64)      # [T][pairs]
    phi = comp * inv_freq(d_rot, base)[None, :]
    return np.cos(phi), np.sin(phi)


def rotate_positions(x: np.ndarray, positions: np.ndarray, sections: Sequence[int], band_offsets: Sequence[int],
                     d_rot: int, base: float, pairing: int) -> np.ndarray:
    """Every rotary band of token t rotated by its own position offsets (t, h, w)."""
    y = np.array(x, dtype=np.float64, copy=True)
    c, s = token_phases(positions, d_rot, base, sections)
    p, q = pair_columns(d_rot, pairing)
    for o in band_offsets:
        a = x[:, o + p]
        b = x[:, o + q]
        y[:, o + p] = a * c - b * s
        y[:, o + q] = a * s + b * c
    return y


# ----------------------------------------------------------------------------
# U_m V_m^T: the rank-m conditioning patch (KAMERA Eq. 1; App. A serve listing)
# ----------------------------------------------------------------------------
def add_patch(y: np.ndarray, u: np.ndarray, vt: np.ndarray, col0: int) -> np.ndarray:
    """y[:, col0:col0+w] += sum_j u[:, j] (outer) vt[j, :], one rank-1 update at a time."""
    w = vt.shape[1]
    for j in range(u.shape[1]):
        y[:, col0:col0 + w] += np.outer(u[:, j], vt[j, :])
    return y


# ----------------------------------------------------------------------------
# Layout helpers: which columns form rotary bands (KAMERA §3; Fig. 2 b-c)
# ----------------------------------------------------------------------------
def band_offsets(family: int, num_kv_heads: int = 0, head_dim: int = 0, latent_dim: int = 0) -> List[int]:
    """GQA/MHA: every key head is one rotary band; MLA: the k_rope band after c_KV."""
    if family == GQA:
        return [h * head_dim for h in range(num_kv_heads)]
    return [latent_dim]


def rotary_width(family: int, head_dim: int = 0, rope_dim: int = 0) -> int:
    return head_dim if family == GQA else rope_dim


class Factor:
    """One stored patch factor pair, fp64: u = U*Sigma [T][m], vt = V^T [m][width]."""

    def __init__(self, tensor: int, col0: int, u: np.ndarray, vt: np.ndarray):
        self.tensor, self.col0 = tensor, col0
        self.u = np.asarray(u, dtype=np.float64)
        self.vt = np.asarray(vt, dtype=np.float64)


def rehydrate_tensor(x: np.ndarray, *, tensor: int, family: int, delta: int, rotate_this: bool,
                     bands: Sequence[int], d_rot: int, base: float, pairing: int,
                     factors: Iterable[Factor] = (), patch: bool = True, positions=None,
                     sections: Sequence[int] = (0, 0, 0)) -> np.ndarray:
    """Eq. 1 for one tensor of one chunk at one layer, fp64, before output rounding.

    x: rows of the stored tensor ([T][F], fp64). `rotate_this` says whether this
    tensor carries the rope band (K for GQA/MHA, the 576-row for MLA; never V).
    With `positions` ([T][3] integer offsets), token t is rotated by its own offsets
    (per-token re-anchoring) and delta is not used.
    """
    if not rotate_this:
        y = np.array(x, dtype=np.float64)
    elif positions is not None:
        y = rotate_positions(x, positions, sections, bands, d_rot, base, pairing)
    else:
        y = rotate(x, delta, bands, d_rot, base, pairing)
    if patch:
        for f in factors:
            if f.tensor == tensor:
                add_patch(y, f.u, f.vt, f.col0)
    return y


def abs_terms(x: np.ndarray, *, tensor: int, delta: int, rotate_this: bool, bands: Sequence[int],
              d_rot: int, base: float, pairing: int, factors: Iterable[Factor] = (),
              patch: bool = True, positions=None, sections: Sequence[int] = (0, 0, 0)) -> np.ndarray:
    """S = sum of |terms| of every output element (fp64), for rounding-error bounds.

    Rotated pair: |a||c| + |b||s| and |a||s| + |b||c|; unrotated: |x|; plus
    sum_j |U_tj||Vt_jf| of every factor covering the element.
    """
    ax = np.abs(np.asarray(x, dtype=np.float64))
    s_ = np.array(ax, copy=True)
    if rotate_this:
        if positions is not None:
            c, s = token_phases(positions, d_rot, base, sections)
        else:
            c, s = phases(delta, d_rot, base)
        c, s = np.abs(c), np.abs(s)
        p, q = pair_columns(d_rot, pairing)
        for o in bands:
            a, b = ax[:, o + p], ax[:, o + q]
            s_[:, o + p] = a * c + b * s
            s_[:, o + q] = a * s + b * c
    if patch:
        for f in factors:
            if f.tensor == tensor:
                add_patch(s_, np.abs(f.u), np.abs(f.vt), f.col0)
    return s_


def angle_terms(x: np.ndarray, *, tensor: int, delta: int, rotate_this: bool, bands: Sequence[int],
                d_rot: int, base: float, pairing: int, factors: Iterable[Factor] = (), patch: bool = True,
                positions=None, sections: Sequence[int] = (0, 0, 0)) -> np.ndarray:
    """A = (|a| + |b|) |phi| 2^-51 for both elements of every rotated pair, 0 elsewhere (fp64).

    The angle phi = p theta_i is formed in fp64, which fixes it only to a few fp64 ulps of
    |phi| (the product is rounded, and theta_i = base^(-2i/d_rot) from two correct fp64 pow
    evaluations may differ by an ulp); 4 ulps, |phi| 2^-51, bound the difference of two such
    evaluations, and a rotated output a c - b s or a s + b c moves by at most (|a| + |b|) |dphi|.
    Same keywords as abs_terms (factors and patch do not enter).
    """
    ax = np.abs(np.asarray(x, dtype=np.float64))
    A = np.zeros_like(ax)
    if rotate_this:
        th = inv_freq(d_rot, base)
        if positions is not None:
            pos = np.asarray(positions, dtype=np.int64).reshape(len(positions), -1)
            phi = np.abs(pos[:, pair_sections(d_rot, sections)].astype(np.float64) * th[None, :])
        else:
            phi = np.abs(np.float64(delta) * th)[None, :]
        p, q = pair_columns(d_rot, pairing)
        for o in bands:
            w = (ax[:, o + p] + ax[:, o + q]) * phi * 2.0 ** -51
            A[:, o + p] = w
            A[:, o + q] = w
    return A


# ----------------------------------------------------------------------------
# Paged KV pool placement (KAMERA §6: the rebuilt KV is written into the pool)
# ----------------------------------------------------------------------------
def page_slots(num_tokens: int, block_table: np.ndarray, slot0: int, page_size: int):
    """(page id, offset in page) of each token t: slot s = slot0 + t lives at
    page block_table[s // page_size], offset s % page_size."""
    s = slot0 + np.arange(num_tokens)
    return np.asarray(block_table)[s // page_size], s % page_size


def scatter_to_pool(pool: np.ndarray, rows: np.ndarray, block_table: np.ndarray, slot0: int) -> None:
    """pool[page][off] = rows[t] for every token, pool shaped [num_pages][page_size][F]."""
    page_size = pool.shape[1]
    pages, offs = page_slots(rows.shape[0], block_table, slot0, page_size)
    for t in range(rows.shape[0]):
        pool[pages[t], offs[t]] = rows[t]


# ----------------------------------------------------------------------------
# One-call helpers for the two layouts
# ----------------------------------------------------------------------------
def rehydrate_gqa(k: np.ndarray, v: np.ndarray, delta: int, *, num_kv_heads: int, head_dim: int,
                  base: float, pairing: int = NEOX, factors: Iterable[Factor] = (),
                  patch: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """GQA/MHA (KAMERA §3): rotate every key head, patch K and V; V is never rotated."""
    bands = band_offsets(GQA, num_kv_heads, head_dim)
    factors = list(factors)
    kw = dict(family=GQA, delta=delta, bands=bands, d_rot=head_dim, base=base, pairing=pairing,
              factors=factors, patch=patch)
    return (rehydrate_tensor(k, tensor=0, rotate_this=True, **kw),
            rehydrate_tensor(v, tensor=1, rotate_this=False, **kw))


def rehydrate_mla(row: np.ndarray, delta: int, *, latent_dim: int, rope_dim: int, base: float,
                  pairing: int = NEOX, factors: Iterable[Factor] = (), patch: bool = True) -> np.ndarray:
    """MLA (KAMERA §3): rotate only the k_rope band; c_KV passes as stored; patch both."""
    return rehydrate_tensor(row, tensor=0, family=MLA, delta=delta, rotate_this=True,
                            bands=band_offsets(MLA, latent_dim=latent_dim), d_rot=rope_dim,
                            base=base, pairing=pairing, factors=list(factors), patch=patch)


def relocate(x: np.ndarray, delta: int, *, family: int, num_kv_heads: int = 0, head_dim: int = 0,
             latent_dim: int = 0, rope_dim: int = 0, base: float, pairing: int = NEOX) -> np.ndarray:
    """Rotation only (KAMERA §5 sliding-window survivors): K, or the MLA rope band."""
    return rotate(x, delta, band_offsets(family, num_kv_heads, head_dim, latent_dim),
                  rotary_width(family, head_dim, rope_dim), base, pairing)
