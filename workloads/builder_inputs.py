"""Seeded inputs for the patch builder: stored canonical rows and a planted deficit.

A case draws the position-free rows KV(B|empty) of one layer and tensor, and a
deficit matrix with a known spectrum on the patched columns:

  planted   Q1 diag(sigma) Q2^T, Q1 [T][r] and Q2 [width][r] with orthonormal
            columns (QR of Gaussian draws), r = len(sigma)
  gaussian  i.i.d. N(0, scale^2) entries (a flat spectrum, no gap)
  zero      all zeros

The conditioned rows KV(B|A) are not drawn here: a test forms them from the
canonical and the deficit with the relocation of its own reference and stores
them, so this module holds none of the method's arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .configs import F32, LayoutSpec

_P_BUILD_CANON, _P_BUILD_DEFICIT = 101, 102


@dataclass(frozen=True)
class BuilderCase:
    layout: LayoutSpec
    tensor: int
    num_tokens: int
    delta: int
    col0: int
    width: int
    spectrum: str = "planted"       # planted | gaussian | zero
    sigma0: float = 0.3             # planted: sigma_i = sigma0 * ratio**i
    ratio: float = 0.9
    planted_rank: int = 0           # planted: r (0: min(T, width))
    scale: float = 1.0              # gaussian: entry scale
    seed: int = 0

    @property
    def sigma(self) -> np.ndarray:
        r = self.planted_rank or min(self.num_tokens, self.width)
        return self.sigma0 * self.ratio ** np.arange(r, dtype=np.float64)

    def to_storage(self, x32: np.ndarray) -> np.ndarray:
        if self.layout.dtype == F32:
            return np.ascontiguousarray(x32, dtype=np.float32)
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    def canonical(self) -> np.ndarray:
        """Stored KV(B|empty) rows [T][F] (storage dtype)."""
        rng = np.random.default_rng([self.seed, _P_BUILD_CANON, self.tensor])
        x = rng.standard_normal((self.num_tokens, self.layout.row_width), dtype=np.float32)
        return self.to_storage(x)

    def deficit(self) -> np.ndarray:
        """The drawn deficit [T][width] in fp64 (before any storage rounding)."""
        T, W = self.num_tokens, self.width
        rng = np.random.default_rng([self.seed, _P_BUILD_DEFICIT, self.tensor])
        if self.spectrum == "zero":
            return np.zeros((T, W))
        if self.spectrum == "gaussian":
            return self.scale * rng.standard_normal((T, W))
        s = self.sigma
        q1, _ = np.linalg.qr(rng.standard_normal((T, len(s))))
        q2, _ = np.linalg.qr(rng.standard_normal((W, len(s))))
        return (q1 * s[None, :]) @ q2.T


_P_ORBIT = 103


def orbit_parts(case: BuilderCase, num_orderings: int, spread: float) -> list:
    """Per-ordering deficits for an orbit: the case's drawn deficit (the part every
    ordering shares) plus a per-ordering Gaussian part of scale `spread`, centred so the
    parts sum to zero over the orderings. Returns num_orderings fp64 [T][width] arrays."""
    base = case.deficit()
    rng = np.random.default_rng([case.seed, _P_ORBIT, case.tensor, num_orderings])
    extra = spread * rng.standard_normal((num_orderings,) + base.shape)
    extra -= extra.mean(axis=0, keepdims=True)
    return [base + extra[k] for k in range(num_orderings)]
