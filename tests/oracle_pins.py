"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each pin takes the oracle module as an argument so the mutation test can run
the same pins against a copy of the oracle with a planted mistake.

Sources: Kamera preprint ("Kamera: Unified Position-Invariant Multimodal KV
Cache for Training-Free Reuse") §1 (R(delta)R(p) = R(p+delta)), §3 (V and c_KV
never rotated; MLA rotates only the 64-d k_rope; patch both channels), §5
(survivors need rotation only), §6 (paged KV pool), Fig. 2 (layout sizes),
App. A (rotate first, then add U @ V^T; factors kept as U*Sigma, V^T).
"""
from __future__ import annotations

import math

import numpy as np

try:
    import mpmath
except ImportError:  # pragma: no cover
    mpmath = None

RNG = np.random.default_rng(20260602)


def _x(T, F, seed=0):
    return np.random.default_rng(seed).standard_normal((T, F))


# --------------------------------------------------------------------- theta
def pin_theta_geometric(o):
    """Textbook RoPE frequencies: a geometric run that starts at 1 and would reach
    1/base after d_rot/2 steps; checked against 40-digit mpmath."""
    mpmath.mp.dps = 40
    for d, base in [(64, 1e4), (128, 1e4), (128, 1e6), (64, 1e6)]:
        th = o.inv_freq(d, base)
        assert th.shape == (d // 2,)
        ratio = mpmath.power(mpmath.mpf(base), mpmath.mpf(-2) / d)
        for i in range(d // 2):
            want = mpmath.power(ratio, i)
            assert abs(th[i] - float(want)) <= 4e-16 * float(want), (d, base, i)
        assert abs(float(mpmath.power(ratio, d // 2)) * base - 1) < 1e-30 + 1e-15


def pin_pairs_from_pages(o):
    """Kamera Fig. 2: 128-d GQA heads carry 64 rope pairs; MLA k_rope 64-d = 32 pairs,
    and the band is the trailing 64 columns after the 512-d c_KV."""
    p, q = o.pair_columns(128, o.NEOX)
    assert len(p) == 64 and sorted(np.concatenate([p, q]).tolist()) == list(range(128))
    p, q = o.pair_columns(64, o.NEOX)
    assert len(p) == 32
    assert o.band_offsets(o.MLA, latent_dim=512) == [512]
    assert o.band_offsets(o.GQA, num_kv_heads=4, head_dim=128) == [0, 128, 256, 384]


# --------------------------------------------------------------------- rotation
def pin_complex_multiply(o):
    """R(delta) on a pair equals (a + ib) * exp(i delta theta) (RoFormer's RoPE).
    NeoX pairs column i with i + d/2; GPT-J uses numpy's own complex layout
    (interleaved re, im) via a dtype view. Phase from mpmath at 30 digits."""
    mpmath.mp.dps = 30
    for d, base, delta in [(128, 1e6, 32768), (64, 1e4, 4096), (128, 1e4, -1234), (64, 1e4, 65536)]:
        x = _x(5, d, seed=d + abs(delta))
        th = [mpmath.power(mpmath.mpf(base), mpmath.mpf(-2 * i) / d) for i in range(d // 2)]
        e = np.array([complex(mpmath.cos(delta * t), mpmath.sin(delta * t)) for t in th])
        # NeoX
        z = x[:, : d // 2] + 1j * x[:, d // 2:]
        want = z * e[None, :]
        y = o.rotate(x, delta, [0], d, base, o.NEOX)
        got = y[:, : d // 2] + 1j * y[:, d // 2:]
        tol = 1e-14 + abs(delta) * 2.0 ** -52 * 4
        assert np.max(np.abs(got - want)) <= tol * np.max(np.abs(x)) * 2, (d, delta)
        # GPT-J: numpy complex128 memory layout is (re, im) interleaved
        zc = np.ascontiguousarray(x).view(np.complex128)
        wantj = (zc * e[None, :]).view(np.float64)
        yj = o.rotate(x, delta, [0], d, base, o.GPTJ)
        assert np.max(np.abs(yj - wantj)) <= tol * np.max(np.abs(x)) * 2, (d, delta)


def pin_composition(o):
    """Kamera §1: R(d) R(p) = R(p + d), against direct rotation at p + d."""
    rng = np.random.default_rng(7)
    for _ in range(12):
        p, d = (int(v) for v in rng.integers(-2 ** 17, 2 ** 17, size=2))
        x = _x(4, 128, seed=abs(p) % 1000)
        a = o.rotate(o.rotate(x, p, [0], 128, 1e6, o.NEOX), d, [0], 128, 1e6, o.NEOX)
        b = o.rotate(x, p + d, [0], 128, 1e6, o.NEOX)
        # angles are rounded fp64 products: |phi| 2^-52 per product, three products
        assert np.max(np.abs(a - b)) <= 1e-10 * np.max(np.abs(x)), (p, d)


def pin_norm_and_inverse(o):
    """A rotation keeps each pair's norm, and R(-delta) undoes R(delta)."""
    x = _x(16, 256, seed=3)
    for delta in (1, 777, -40000, 65536):
        y = o.rotate(x, delta, [0, 128], 128, 1e4, o.NEOX)
        p, q = o.pair_columns(128, o.NEOX)
        for off in (0, 128):
            n0 = x[:, off + p] ** 2 + x[:, off + q] ** 2
            n1 = y[:, off + p] ** 2 + y[:, off + q] ** 2
            assert np.max(np.abs(n1 - n0) / n0) < 1e-14
        back = o.rotate(y, -delta, [0, 128], 128, 1e4, o.NEOX)
        assert np.max(np.abs(back - x)) < 1e-13


def pin_identity(o):
    """delta = 0 with no patch returns the stored codes bit for bit (bf16 and fp32)."""
    bits = np.random.default_rng(1).integers(0, 0x7F00, size=(32, 256), dtype=np.uint16)
    bits[:, ::7] |= 0x8000
    x = o.upcast(bits, o.BF16)
    yk, yv = o.rehydrate_gqa(x, x, 0, num_kv_heads=2, head_dim=128, base=1e6, patch=False)
    assert np.array_equal(o.round_bf16(yk), bits) and np.array_equal(o.round_bf16(yv), bits)
    f = np.random.default_rng(2).standard_normal((8, 128)).astype(np.float32)
    yk, _ = o.rehydrate_gqa(f.astype(np.float64), f.astype(np.float64), 0, num_kv_heads=2, head_dim=64,
                            base=1e4, patch=False)
    assert np.array_equal(o.round_f32(yk).view(np.uint32), f.view(np.uint32))


def pin_large_delta_phase(o):
    """cos/sin of delta*theta_i at large |delta| against 40-digit mpmath: error is only
    the fp64 rounding of the product (|phi| 2^-53) plus the libm rounding."""
    mpmath.mp.dps = 40
    for delta in (65536, 2 ** 31 - 1, -(2 ** 31 - 1), 1_000_003):
        c, s = o.phases(delta, 128, 1e6)
        th = [mpmath.power(mpmath.mpf(10) ** 6, mpmath.mpf(-2 * i) / 128) for i in range(64)]
        for i in (0, 1, 17, 63):
            phi = delta * th[i]
            bound = abs(float(phi)) * 2.0 ** -52 + 2.0 ** -52
            assert abs(c[i] - float(mpmath.cos(phi))) <= bound, (delta, i)
            assert abs(s[i] - float(mpmath.sin(phi))) <= bound, (delta, i)


# --------------------------------------------------------------------- patch
def pin_patch_is_matmul(o):
    """Y(patch) - Y(no patch) = U @ V^T by BLAS dgemm, on K (rotated) and V; the
    patch is added after the rotation and is itself not rotated (App. A)."""
    T, H, d, m = 40, 2, 64, 8
    k, v = _x(T, H * d, 4), _x(T, H * d, 5)
    fac = [o.Factor(0, 0, _x(T, m, 6), _x(m, H * d, 7)), o.Factor(1, 0, _x(T, m, 8), _x(m, H * d, 9))]
    yk, yv = o.rehydrate_gqa(k, v, 321, num_kv_heads=H, head_dim=d, base=1e4, factors=fac)
    zk, zv = o.rehydrate_gqa(k, v, 321, num_kv_heads=H, head_dim=d, base=1e4, factors=fac, patch=False)
    for got, f in ((yk - zk, fac[0]), (yv - zv, fac[1])):
        want = f.u @ f.vt
        assert np.max(np.abs(got - want)) <= 1e-13 * np.max(np.abs(want)) * 4
    # V rows are not rotated: no-patch V equals the input exactly
    assert np.array_equal(zv, v)
    # a factor covering part of a row touches only its columns
    row = _x(T, 576, 10)
    fb = o.Factor(0, 512, _x(T, m, 11), _x(m, 64, 12))
    y = o.rehydrate_mla(row, 99, latent_dim=512, rope_dim=64, base=1e4, factors=[fb])
    z = o.rehydrate_mla(row, 99, latent_dim=512, rope_dim=64, base=1e4, factors=[fb], patch=False)
    d_ = y - z
    assert np.all(d_[:, :512] == 0)
    assert np.max(np.abs(d_[:, 512:] - fb.u @ fb.vt)) <= 1e-13 * 8


def pin_full_rank_reconstructs(o):
    """A full-rank patch from LAPACK's SVD of a random Delta rebuilds it (rank = min(T,F))."""
    import scipy.linalg
    T, F = 24, 16
    delta = _x(T, F, 13)
    u, s, vt = scipy.linalg.svd(delta, full_matrices=False)
    x = _x(T, F, 14)
    y = o.rehydrate_tensor(x, tensor=1, family=o.GQA, delta=0, rotate_this=False, bands=[], d_rot=16,
                           base=1e4, pairing=o.NEOX, factors=[o.Factor(1, 0, u * s, vt)])
    assert np.max(np.abs(y - (x + delta))) < 1e-12


# --------------------------------------------------------------------- survivors / MLA
def pin_survivor_rotation_only(o):
    """Kamera §5: survivors get R(delta) only; V (and MLA c_KV) untouched."""
    k, v = _x(20, 256, 15), _x(20, 256, 16)
    y = o.relocate(k, -3000, family=o.GQA, num_kv_heads=2, head_dim=128, base=1e6)
    z, zv = o.rehydrate_gqa(k, v, -3000, num_kv_heads=2, head_dim=128, base=1e6, patch=False)
    assert np.array_equal(y, z) and np.array_equal(zv, v)
    row = _x(20, 576, 17)
    ym = o.relocate(row, 12345, family=o.MLA, latent_dim=512, rope_dim=64, base=1e4)
    assert np.array_equal(ym[:, :512], row[:, :512])          # c_KV byte-for-byte
    assert not np.allclose(ym[:, 512:], row[:, 512:])          # the band did move


# --------------------------------------------------------------------- paging
def pin_paging_bruteforce(o):
    """Every slot0 in a 16-token page: gather by block table returns the rows in order,
    and every slot outside [slot0, slot0+T) keeps its sentinel."""
    P, F = 16, 4
    for T in (1, 15, 16, 17, 33, 48):
        for slot0 in range(P):
            npg = -(-(slot0 + T) // P)
            table = np.random.default_rng(T * 31 + slot0).permutation(8)[:npg]
            pool = np.full((8, P, F), -7.0)
            rows = np.arange(T * F, dtype=np.float64).reshape(T, F)
            o.scatter_to_pool(pool, rows, table, slot0)
            written = np.zeros((8, P), bool)
            for t in range(T):                       # independent walk of the slots
                slot = slot0 + t
                pg, off = table[slot // P], slot % P
                assert np.array_equal(pool[pg, off], rows[t])
                written[pg, off] = True
            assert np.all(pool[~written] == -7.0)


# --------------------------------------------------------------------- rounding
def pin_bf16_rounding(o):
    """Exhaustive over bf16 codes: exact values round to themselves; midpoints between
    neighbours go to the even code; a hair above/below goes to the nearer one; torch's
    fp32 -> bf16 cast (RNE) agrees on random fp32 values."""
    import torch
    codes = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    vals = o.upcast(codes, o.BF16)
    finite = np.isfinite(vals)
    assert np.array_equal(o.round_bf16(vals[finite]), codes[finite])
    pos = codes[(codes < 0x7F7F) & (codes > 0)]                # positive finite with a finite successor
    lo, hi = o.upcast(pos, o.BF16), o.upcast(pos + 1, o.BF16)
    mid = (lo + hi) / 2                                        # exact in fp64
    even = np.where(pos % 2 == 0, pos, pos + 1).astype(np.uint16)
    assert np.array_equal(o.round_bf16(mid), even)
    assert np.array_equal(o.round_bf16(-mid), even | 0x8000)
    up = np.nextafter(mid, np.inf)
    dn = np.nextafter(mid, -np.inf)
    assert np.array_equal(o.round_bf16(up), (pos + 1).astype(np.uint16))
    assert np.array_equal(o.round_bf16(dn), pos)
    r = np.random.default_rng(5).integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = r.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.3e38)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(o.round_bf16(f.astype(np.float64)), want)


# --------------------------------------------------------------------- builder
def pin_reanchor(o):
    """Per-token re-anchoring (QV-PIC Eq. 2; KAMERA §4 for the uniform case).
    (a) a uniform offset (d, d, d) on every token is R(d) for any sections, bit for bit;
    (b) 1-D offsets p_t = p0 + t on unrotated keys equal a complex multiply by
        exp(i p_t theta) per token (independent formula, NeoX halves);
    (c) with blocked sections (16, 24, 24) of a 128-wide head, pair i follows t, h or w
        by its index, using the band's global frequency theta_i: each section checked
        against a complex multiply with its own component."""
    rng = np.random.default_rng(41)
    T, d, base = 24, 128, 1e6
    x = rng.standard_normal((T, d))
    for sec in [(0, 0, 0), (16, 24, 24), (32, 16, 16)]:
        dl = 12345
        y = o.rotate_positions(x, np.full((T, 3), dl), sec, [0], d, base, o.NEOX)
        assert np.array_equal(y, o.rotate(x, dl, [0], d, base, o.NEOX)), sec
    th = base ** (-2.0 * np.arange(d // 2) / d)
    pos1 = 1000 + np.arange(T)
    y = o.rotate_positions(x, np.stack([pos1, 0 * pos1, 0 * pos1], 1), (0, 0, 0), [0], d, base, o.NEOX)
    z = (x[:, : d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * pos1[:, None] * th[None, :])
    assert np.max(np.abs(y - np.concatenate([z.real, z.imag], 1))) <= 1e-12
    pos = np.stack([rng.integers(0, 4096, T), rng.integers(0, 64, T), rng.integers(0, 64, T)], 1)
    y = o.rotate_positions(x, pos, (16, 24, 24), [0], d, base, o.NEOX)
    comp = np.concatenate([np.zeros(16, int), np.ones(24, int), 2 * np.ones(24, int)])
    z = (x[:, : d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * pos[:, comp] * th[None, :])
    assert np.max(np.abs(y - np.concatenate([z.real, z.imag], 1))) <= 1e-12


def pin_builder_planted(b):
    """Planted spectrum Delta = Q1 diag(sigma) Q2^T with sigma_i = 0.3*0.9^i: the top-m
    singular values are the planted ones, and the Eckart-Young residual
    ||Delta - U_m V_m^T||_F^2 equals sum_{i>=m} sigma_i^2 (closed form)."""
    rng = np.random.default_rng(11)
    T, F, r, m = 96, 64, 40, 8
    q1, _ = np.linalg.qr(rng.standard_normal((T, r)))
    q2, _ = np.linalg.qr(rng.standard_normal((F, r)))
    sig = 0.3 * 0.9 ** np.arange(r)
    delta = (q1 * sig) @ q2.T
    us, vt, s = b.truncated_svd(delta, m)
    assert np.allclose(s[:r], sig, rtol=1e-12, atol=1e-15)
    res = b.residual_energy(delta, us, vt)
    assert abs(res - np.sum(sig[m:] ** 2)) <= 1e-12 * np.sum(sig ** 2)
    # storage convention (Fig. 2(d), App. A): sigma folded into U, V^T with orthonormal rows
    assert np.allclose(np.linalg.norm(us, axis=0), sig[:m], rtol=1e-12)
    assert np.allclose(vt @ vt.T, np.eye(m), atol=1e-12)
    # the compile-step deficit subtracts the relocated canonical (App. A): conditioned
    # rows equal to the canonical rotated by delta (as a complex multiply, NeoX halves)
    # plus a known matrix P give back exactly P
    x = rng.standard_normal((T, 128))
    cond = x + 0.0
    d = b.deficit(cond, x, 0, bands=[0], d_rot=128, base=1e4, pairing=0)
    assert np.all(d == 0)
    delta, base = 777, 1e4
    th = base ** (-2.0 * np.arange(64) / 128)
    z = (x[:, :64] + 1j * x[:, 64:]) * np.exp(1j * delta * th)[None, :]
    P = 0.01 * rng.standard_normal((T, 128))
    cond = np.concatenate([z.real, z.imag], axis=1) + P
    d = b.deficit(cond, x, delta, bands=[0], d_rot=128, base=base, pairing=0)
    assert np.max(np.abs(d - P)) <= 1e-12
    # ... and only for the rotated tensor: V's deficit is a plain difference
    dv = b.deficit(x + P, x, delta, bands=[0], d_rot=128, base=base, pairing=0, rotate_this=False)
    assert np.max(np.abs(dv - P)) <= 1e-15


def pin_orbit_mean(b):
    """Orbit deficit (preprint §5, reorder): with conditioned blocks built as the
    canonical rotated to each ordering's offset (complex multiply, NeoX halves) plus a
    common matrix P and per-ordering parts N_k that sum to zero, the orbit deficit is
    exactly P. One ordering reduces to the single deficit; the order of the orderings
    does not matter."""
    rng = np.random.default_rng(21)
    T, d, base = 40, 64, 1e6
    x = rng.standard_normal((T, d))
    P = 0.1 * rng.standard_normal((T, d))
    deltas = [0, 2048, -4096, 6144, 123457]
    N = rng.standard_normal((len(deltas), T, d))
    N -= N.mean(axis=0, keepdims=True)
    th = base ** (-2.0 * np.arange(d // 2) / d)
    conds = []
    for k, dl in enumerate(deltas):
        z = (x[:, : d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * dl * th)[None, :]
        conds.append(np.concatenate([z.real, z.imag], axis=1) + P + N[k])
    kw = dict(bands=[0], d_rot=d, base=base, pairing=0)
    got = b.orbit_deficit(conds, x, deltas, **kw)
    assert np.max(np.abs(got - P)) <= 1e-12
    assert np.max(np.abs(b.orbit_deficit(conds[:1], x, deltas[:1], **kw) - b.deficit(conds[0], x, deltas[0], **kw))) == 0
    perm = [3, 0, 4, 2, 1]
    rev = b.orbit_deficit([conds[i] for i in perm], x, [deltas[i] for i in perm], **kw)
    assert np.max(np.abs(rev - got)) <= 1e-14


ORACLE_PINS = [pin_theta_geometric, pin_pairs_from_pages, pin_complex_multiply, pin_composition,
               pin_norm_and_inverse, pin_identity, pin_large_delta_phase, pin_patch_is_matmul,
               pin_full_rank_reconstructs, pin_survivor_rotation_only, pin_paging_bruteforce,
               pin_bf16_rounding, pin_reanchor]


# --------------------------------------------------------------------- error-bound terms
def _brute_abs_terms(x, *, bands, d_rot, base, pairing, rotate_this, delta=0, positions=None,
                     sections=(0, 0, 0), factors=(), tensor=0):
    """Pure-Python walk over every output element: list the terms that the definition
    adds up for it and sum their magnitudes. The frequencies and phases come from the
    math module, the rotary partner and the position component of a pair are found by
    walking the band, and every factor covering the column contributes its m products."""
    T, F = len(x), len(x[0])
    half = d_rot // 2
    freqs = [math.pow(base, -2.0 * i / d_rot) for i in range(half)]

    def component(i):
        if not any(sections):
            return 0
        if i < sections[0]:
            return 0
        return 1 if i < sections[0] + sections[1] else 2

    out = [[0.0] * F for _ in range(T)]
    for t in range(T):
        for f in range(F):
            terms = [x[t][f]]
            if rotate_this:
                for o in bands:
                    j = f - o
                    if not 0 <= j < d_rot:
                        continue
                    if pairing == 0:                      # NeoX: halves of the band
                        i, first = (j, True) if j < half else (j - half, False)
                        pa, pb = o + i, o + i + half
                    else:                                 # GPT-J: neighbours
                        i, first = j // 2, j % 2 == 0
                        pa, pb = o + 2 * i, o + 2 * i + 1
                    p = delta if positions is None else positions[t][component(i)]
                    c, s = math.cos(p * freqs[i]), math.sin(p * freqs[i])
                    a, b = x[t][pa], x[t][pb]
                    terms = [a * c, -b * s] if first else [a * s, b * c]
            for fac in factors:
                if fac.tensor != tensor or not fac.col0 <= f < fac.col0 + fac.vt.shape[1]:
                    continue
                terms += [fac.u[t][k] * fac.vt[k][f - fac.col0] for k in range(fac.u.shape[1])]
            out[t][f] = sum(abs(v) for v in terms)
    return np.array(out)


def pin_abs_terms_bruteforce(o):
    """The error bound's S (sum of |terms| of each output) against a brute-force listing of
    every term: GQA with NeoX and GPT-J pairs and two factors on K, V with none rotated, an
    MLA-shaped row with two overlapping factors (whole row and rope band), per-token offsets
    with three sections, and the patch switched off."""
    rng = np.random.default_rng(77)
    T, H, d = 6, 2, 8
    k = rng.standard_normal((T, H * d))
    fk = [o.Factor(0, 0, rng.standard_normal((T, 3)), rng.standard_normal((3, H * d))),
          o.Factor(0, 4, rng.standard_normal((T, 2)), rng.standard_normal((2, 6))),
          o.Factor(1, 0, rng.standard_normal((T, 3)), rng.standard_normal((3, H * d)))]
    bands = [0, d]
    cases = []
    for pairing in (0, 1):
        for tensor, rot in ((0, True), (1, False)):
            cases.append(dict(x=k, tensor=tensor, rotate_this=rot, delta=-4321, bands=bands, d_rot=d, base=1e4,
                              pairing=pairing, factors=fk, patch=True))
    cases.append(dict(x=k, tensor=0, rotate_this=True, delta=99991, bands=bands, d_rot=d, base=1e6, pairing=0,
                      factors=fk, patch=False))
    row = rng.standard_normal((T, 16))                  # latent 8 + rope band 8 at column 8
    fm = [o.Factor(0, 0, rng.standard_normal((T, 4)), rng.standard_normal((4, 16))),
          o.Factor(0, 8, rng.standard_normal((T, 3)), rng.standard_normal((3, 8)))]
    cases.append(dict(x=row, tensor=0, rotate_this=True, delta=65536, bands=[8], d_rot=8, base=1e4, pairing=0,
                      factors=fm, patch=True))
    pos = np.stack([rng.integers(-3000, 3000, T), rng.integers(0, 64, T), rng.integers(0, 64, T)], 1)
    cases.append(dict(x=k, tensor=0, rotate_this=True, delta=0, bands=bands, d_rot=d, base=1e6, pairing=0,
                      factors=fk, patch=True, positions=pos, sections=(1, 1, 2)))
    for cs in cases:
        kw = dict(cs)
        x = kw.pop("x")
        patch = kw.pop("patch")
        got = o.abs_terms(x, **kw, patch=patch)
        want = _brute_abs_terms(x.tolist(), bands=kw["bands"], d_rot=kw["d_rot"], base=kw["base"],
                                pairing=kw["pairing"], rotate_this=kw["rotate_this"], delta=kw["delta"],
                                positions=None if kw.get("positions") is None else kw["positions"].tolist(),
                                sections=kw.get("sections", (0, 0, 0)),
                                factors=kw["factors"] if patch else (), tensor=kw["tensor"])
        assert got.shape == want.shape
        assert np.max(np.abs(got - want) / want) <= 1e-13, {k_: v for k_, v in kw.items() if k_ != "factors"}


ORACLE_PINS.append(pin_abs_terms_bruteforce)


# --------------------------------------------------------------------- tolerance predicates
# These take the tolerance module t (and the oracle o for S), so planted mistakes in
# either module can be run against them.
def _bf16_code_values():
    """All positive finite bf16 codes and their values, decoded from the bit fields
    directly (sign 1, exponent 8, fraction 7; exponent 0 = subnormal)."""
    codes = np.arange(0x7F80, dtype=np.int64)            # +0 .. largest finite
    ex, fr = codes >> 7, codes & 0x7F
    vals = np.where(ex == 0, np.ldexp(fr.astype(np.float64), -133),
                    np.ldexp((128 + fr).astype(np.float64), (ex - 134).astype(np.int64)))
    return codes, vals


def pin_ulp_spacing(t, o=None):
    """ulp_bf16 at every bf16 value is the gap to the next code (exhaustive, zero and
    subnormals included), and inside each binade stays that gap; ulp_f32 equals numpy's
    float32 spacing over every binade, subnormals and zero included."""
    codes, vals = _bf16_code_values()
    gap = vals[1:] - vals[:-1]                            # value(code + 1) - value(code)
    assert np.array_equal(t.ulp_bf16(vals[:-1]), gap)
    assert np.array_equal(t.ulp_bf16(-vals[:-1]), gap)
    inside = vals[:-1] + 0.25 * gap                       # between two codes: same binade
    assert np.array_equal(t.ulp_bf16(inside), gap)
    # float32: powers of two, their neighbours and random values of every exponent
    e = np.arange(-149, 128)
    p2 = np.ldexp(np.float32(1), e).astype(np.float32)
    rnd = np.random.default_rng(3).integers(0, 0x7F800000, size=200000, dtype=np.int64).astype(np.uint32)
    f = np.concatenate([p2, np.nextafter(p2, np.float32(0)), np.nextafter(p2, np.float32(np.inf)),
                        rnd.view(np.float32), np.float32([0.0, 1e-45, 1.17549435e-38])])
    f = f[np.isfinite(f) & (f < np.float32(3.4e38))]
    want = np.spacing(f).astype(np.float64)
    assert np.array_equal(t.ulp_f32(f.astype(np.float64)), want)
    assert np.array_equal(t.ulp_f32(-f.astype(np.float64)), want)


def _c1_block(o, seed=5):
    """A single-layer fp32 GQA block of the small workload's shape: 256 tokens, 2 heads x 64,
    delta in [0, 4096], a rank-8 factor on the rotated keys."""
    rng = np.random.default_rng(seed)
    T, H, d, m = 256, 2, 64, 8
    x = rng.standard_normal((T, H * d)).astype(np.float32).astype(np.float64)
    u = (0.5 * rng.standard_normal((T, m))).astype(np.float32).astype(np.float64)
    vt = (rng.standard_normal((m, H * d)) / np.sqrt(T)).astype(np.float32).astype(np.float64)
    delta = int(rng.integers(0, 4097))
    kw = dict(tensor=0, delta=delta, rotate_this=True, bands=[0, d], d_rot=d, base=1e4, pairing=0,
              factors=[o.Factor(0, 0, u, vt)], patch=True)
    y = o.rehydrate_tensor(x, family=o.GQA, **kw)
    S = o.abs_terms(x, **kw)
    return x, u, vt, delta, y, S, m


def _fp32_evaluation(x, u, vt, delta, d=64, base=1e4):
    """The same block evaluated the way a device in fp32 would, but independently: cos and
    sin rounded once to float32, the pair rotation and every patch term in float32 products
    and sums (no fused multiply-add), terms added in order."""
    x32, u32, vt32 = x.astype(np.float32), u.astype(np.float32), vt.astype(np.float32)
    half = d // 2
    th = np.array([math.pow(base, -2.0 * i / d) for i in range(half)])
    c = np.array([math.cos(delta * v) for v in th], dtype=np.float32)
    s = np.array([math.sin(delta * v) for v in th], dtype=np.float32)
    y = x32.copy()
    for o_ in range(0, x.shape[1], d):
        a, b = x32[:, o_:o_ + half], x32[:, o_ + half:o_ + d]
        y[:, o_:o_ + half] = a * c - b * s
        y[:, o_ + half:o_ + d] = a * s + b * c
    for j in range(u.shape[1]):
        y = y + u32[:, j:j + 1] * vt32[j:j + 1, :]
    return y


def pin_check_f32(t, o):
    """P3 on a block of the fp32 workload's shape: accepts the oracle's own rounding and an
    independent float32 evaluation; rejects a planted relative error of 2^-12 on nearly every
    element; with S = 0 and no angle term, half an fp32 ulp passes and two ulps do not."""
    x, u, vt, delta, y, S, m = _c1_block(o)
    n = m + 4
    assert t.check_f32(o.round_f32(y), y, S, n)["fail"] == 0
    g = _fp32_evaluation(x, u, vt, delta)
    res = t.check_f32(g, y, S, n)
    assert res["fail"] == 0, res["fail"]
    off_ulp = np.abs(g.astype(np.float64) - y) > 0.5 * np.spacing(np.abs(y).astype(np.float32))
    assert off_ulp.sum() > 0.01 * y.size          # the evaluation really does differ by more than rounding
    bad = t.check_f32(o.round_f32(y * (1 + 2.0 ** -12)), y, S, n)
    assert bad["fail"] >= 0.97 * y.size, bad["fail"]
    # S = 0, A = 0: exact half-ulp rule against the float32 grid
    f = np.random.default_rng(9).standard_normal(4096).astype(np.float32)
    f = f[np.abs(f) > 1e-3]
    yv = f.astype(np.float64) + 0.25 * np.spacing(np.abs(f)).astype(np.float64)   # inside the ulp above f
    zero = np.zeros_like(yv)
    assert t.check_f32(f, yv, zero, 1)["fail"] == 0                                 # |g - y| = ulp/4
    two = np.nextafter(np.nextafter(f, np.float32(np.inf)), np.float32(np.inf))      # two codes up
    assert t.check_f32(two, yv, zero, 1)["fail"] == len(f)
    tiny = np.array([0.0, 2.0 ** -140])                                             # at and near zero
    assert t.check_f32(np.float32([2.0 ** -149, 0.0]), tiny, np.zeros(2), 1)["fail"] == 2


def pin_check_bf16(t, o):
    """P1/P2 on a bf16 block: accepts the oracle's rounding and an fp32 evaluation rounded to
    bf16 (a second rounding: one code off at most); rejects a planted relative error of 2^-6
    (three or more bf16 codes) on nearly every element; a zero output for a small non-zero
    value is not covered by the zero's own spacing."""
    x, u, vt, delta, y, S, m = _c1_block(o, seed=6)
    n = m + 4
    r = o.round_bf16(y)
    assert t.check_bf16(r, y, r, S, n)["fail"] == 0
    g32 = _fp32_evaluation(x, u, vt, delta)
    g = o.round_bf16(g32.astype(np.float64))
    res = t.check_bf16(g, y, r, S, n)
    assert res["fail"] == 0 and res["exact"] > 0.9 * y.size
    bad = t.check_bf16(o.round_bf16(y * (1 + 2.0 ** -6)), y, r, S, n)
    assert bad["fail"] >= 0.97 * y.size, bad["fail"]
    yv = np.array([1e-6, -3e-5])
    rv = o.round_bf16(yv)
    assert t.check_bf16(np.zeros(2, np.uint16), yv, rv, np.abs(yv), 1)["fail"] == 2


TOLERANCE_PINS = [pin_ulp_spacing, pin_check_f32, pin_check_bf16]
