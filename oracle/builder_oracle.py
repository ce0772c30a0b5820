"""fp64 oracle of the compile step that forms a conditioning patch.

TEST INFRASTRUCTURE ONLY (see oracle/kamera_oracle.py).

Kamera preprint, Eq. 2 (§2): the deficit is Delta = KV(B|A) - KV(B|empty).
Kamera preprint, §5 (reorder): the orbit patch is formed from the deficit
averaged over the orderings of a cached set (the test ordering held out).
Kamera preprint, App. A (compile listing) and §3: as formed, Delta is the
conditioned KV minus the *relocated* canonical R(delta).KV(B|empty); its SVD
is truncated to the top m components and stored as (U*Sigma, V^T) (Fig. 2(d):
"store U Sigma, V^T").

The SVD is LAPACK's (scipy.linalg.svd, gesdd driver): the truncated factorisation
that a builder's factors are checked against through their Eckart-Young residual
energy (the optimum rank-m residual is the sum of the discarded sigma_i^2).
"""
from __future__ import annotations

import numpy as np
import scipy.linalg

from .kamera_oracle import rotate


def deficit(x_cond: np.ndarray, x_canon: np.ndarray, delta: int, *, bands, d_rot: int, base: float,
            pairing: int, rotate_this: bool = True) -> np.ndarray:
    """Delta = KV(B|A) - R(delta).KV(B|empty), fp64 ([T][F])."""
    solo = rotate(x_canon, delta, bands, d_rot, base, pairing) if rotate_this else np.asarray(x_canon, np.float64)
    return np.asarray(x_cond, dtype=np.float64) - solo


def orbit_deficit(x_conds, x_canon: np.ndarray, deltas, *, bands, d_rot: int, base: float, pairing: int,
                  rotate_this: bool = True) -> np.ndarray:
    """Mean deficit over a set of orderings (Kamera preprint §5, reorder: one patch
    averaged over the permutation orbit). Ordering k placed the chunk at offset
    deltas[k] and produced the conditioned rows x_conds[k]; its deficit is
    x_conds[k] - R(deltas[k]).x_canon, and the orbit deficit is their plain average.
    The ordering held out for evaluation is simply not passed in."""
    if len(x_conds) != len(deltas) or len(x_conds) == 0:
        raise ValueError("one delta per conditioned block, at least one block")
    acc = None
    for xc, d in zip(x_conds, deltas):
        dk = deficit(xc, x_canon, int(d), bands=bands, d_rot=d_rot, base=base, pairing=pairing,
                     rotate_this=rotate_this)
        acc = dk if acc is None else acc + dk
    return acc / len(x_conds)


def truncated_svd(delta_mat: np.ndarray, m: int):
    """Top-m factors of Delta: (U[:, :m] * S[:m], Vt[:m]) and the full singular spectrum."""
    u, s, vt = scipy.linalg.svd(np.asarray(delta_mat, dtype=np.float64), full_matrices=False,
                                lapack_driver="gesdd")
    return u[:, :m] * s[:m][None, :], vt[:m], s


def residual_energy(delta_mat: np.ndarray, u_sigma: np.ndarray, vt: np.ndarray) -> float:
    """||Delta - U Vt||_F^2, evaluated with a plain elementwise difference."""
    r = np.asarray(delta_mat, dtype=np.float64) - np.asarray(u_sigma, np.float64) @ np.asarray(vt, np.float64)
    return float(np.sum(r * r))
