"""fp64 oracle of the compile step that forms a conditioning patch.

TEST INFRASTRUCTURE ONLY (see oracle/kamera_oracle.py).

Kamera preprint, Eq. 2 (§2): the deficit is Delta = KV(B|A) - KV(B|empty).
Kamera preprint, App. A (compile listing) and §3: as formed, Delta is the
conditioned KV minus the *relocated* canonical R(delta).KV(B|empty); its SVD
is truncated to the top m components and stored as (U*Sigma, V^T) (Fig. 2(d):
"store U Sigma, V^T").

The SVD is LAPACK's (scipy.linalg.svd, gesdd driver), the library routine the
north star names as the reference for the truncated factorisation.
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


def truncated_svd(delta_mat: np.ndarray, m: int):
    """Top-m factors of Delta: (U[:, :m] * S[:m], Vt[:m]) and the full singular spectrum."""
    u, s, vt = scipy.linalg.svd(np.asarray(delta_mat, dtype=np.float64), full_matrices=False,
                                lapack_driver="gesdd")
    return u[:, :m] * s[:m][None, :], vt[:m], s


def residual_energy(delta_mat: np.ndarray, u_sigma: np.ndarray, vt: np.ndarray) -> float:
    """||Delta - U Vt||_F^2, evaluated with a plain elementwise difference."""
    r = np.asarray(delta_mat, dtype=np.float64) - np.asarray(u_sigma, np.float64) @ np.asarray(vt, np.float64)
    return float(np.sum(r * r))
