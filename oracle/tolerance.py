"""Acceptance predicates for comparing device outputs with the fp64 oracle.

TEST INFRASTRUCTURE ONLY (see oracle/kamera_oracle.py).

The fidelity bar comes from the Kamera preprint §6: the rebuilt KV agrees with a
recompute to within one bf16 unit in the last place. With y the exact fp64 result,
r = bf16(y) rounded once, and g the device output (fp32 accumulation, then one rounding):

  P1  |ord(g) - ord(r)| <= 1          ord = monotone integer order of bf16 codes, +0 == -0
  P2  |g - y| <= ulp_bf16(g)/2 + gamma_n * S + A
  P3  (fp32 outputs) |g - y| <= ulp_f32(y)/2 + gamma_n * S + A

S is the fp64 sum of |terms| (oracle.kamera_oracle.abs_terms) and
gamma_n = n u / (1 - n u), u = 2^-24 (Higham's bound for n fp32 roundings).
A (oracle.kamera_oracle.angle_terms; 0 when not given) covers the angle itself: the
method forms phi = p theta_i in fp64, which fixes phi only to a few fp64 ulps of |phi|
(the product is rounded, and two correct fp64 evaluations of theta_i = base^(-2i/d_rot)
may differ by an ulp), so for |phi| ~ 1e9 cos and sin are not determined to fp32
precision by any fp64 evaluation; A = (|a| + |b|) |phi| 2^-51 bounds what that moves.
P2 exists because with fp32 accumulation an element whose value nearly cancels
(|y| << S) can miss P1 with no defect in the kernel. An element passes a bf16
comparison if P1 or P2 holds; the count that passes only through P2 is reported.
"""
from __future__ import annotations

import numpy as np

U32 = 2.0 ** -24


def bf16_ord(bits: np.ndarray) -> np.ndarray:
    """Map bf16 codes to integers whose order is the numeric order (+0 and -0 both 0)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _binade(x: np.ndarray) -> np.ndarray:
    """e with |x| = f 2^e, 1/2 <= f < 1, clamped at the lowest normal binade of fp32 and bf16
    (both have 8 exponent bits); zero belongs to that lowest binade, whose spacing is the
    smallest subnormal."""
    f, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.where(f == 0, -125, np.maximum(e, -125))


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of the bf16 grid in the binade of |x| (2^-133 for subnormals and zero)."""
    return np.ldexp(1.0, _binade(x) - 8)


def ulp_f32(x: np.ndarray) -> np.ndarray:
    """Spacing of the fp32 grid in the binade of |x| (2^-149 for subnormals and zero)."""
    return np.ldexp(1.0, _binade(x) - 24)


def gamma(n: int) -> float:
    return n * U32 / (1.0 - n * U32)


def check_bf16(g_bits: np.ndarray, y: np.ndarray, r_bits: np.ndarray, S: np.ndarray, n: int, A=None) -> dict:
    """Element-wise P1-or-P2 over arrays of equal shape. Returns counts and the fail mask."""
    g_bits = np.asarray(g_bits, dtype=np.uint16)
    p1 = np.abs(bf16_ord(g_bits) - bf16_ord(r_bits)) <= 1
    g = bf16_value(g_bits)
    with np.errstate(invalid="ignore"):
        p2 = np.abs(g - y) <= 0.5 * ulp_bf16(g) + gamma(n) * S + (0.0 if A is None else A)
    ok = p1 | p2
    return {"n": int(ok.size), "fail": int((~ok).sum()), "p2_only": int((p2 & ~p1).sum()),
            "exact": int((g_bits == r_bits).sum()), "mask": ~ok}


def check_f32(g: np.ndarray, y: np.ndarray, S: np.ndarray, n: int, A=None) -> dict:
    g = np.asarray(g, dtype=np.float32).astype(np.float64)
    ok = np.abs(g - y) <= 0.5 * ulp_f32(y) + gamma(n) * S + (0.0 if A is None else A)
    return {"n": int(ok.size), "fail": int((~ok).sum()), "p2_only": 0,
            "exact": int((g == np.asarray(y, dtype=np.float64).astype(np.float32)).sum()), "mask": ~ok}
