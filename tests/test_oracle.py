"""The fp64 oracle against its pins, and planted mistakes against the pins (CPU only)."""
import importlib.util
import os

import numpy as np
import pytest

import oracle.builder_oracle as builder
import oracle.kamera_oracle as O
from oracle import tolerance as tol
from tests.oracle_pins import ORACLE_PINS, TOLERANCE_PINS, pin_builder_planted, pin_orbit_mean

ORACLE_PATH = os.path.join(os.path.dirname(O.__file__), "kamera_oracle.py")


@pytest.mark.parametrize("pin", ORACLE_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(O)


@pytest.mark.parametrize("pin", TOLERANCE_PINS, ids=lambda p: p.__name__)
def test_tolerance_pin(pin):
    pin(tol, O)


def test_builder_pin():
    pin_builder_planted(builder)


def test_orbit_pin():
    pin_orbit_mean(builder)


# ---------------------------------------------------------------- planted mistakes
def _fresh_oracle():
    spec = importlib.util.spec_from_file_location("kamera_oracle_mutant", ORACLE_PATH)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _mut_sign(m):
    orig = m.phases
    m.phases = lambda d, r, b: (orig(d, r, b)[0], -orig(d, r, b)[1])


def _mut_cos_sin_swapped(m):
    orig = m.phases
    m.phases = lambda d, r, b: tuple(reversed(orig(d, r, b)))


def _mut_pairing(m):
    orig = m.pair_columns
    m.pair_columns = lambda d, p: orig(d, m.GPTJ if p == m.NEOX else m.NEOX)


def _mut_theta_half(m):
    m.inv_freq = lambda d, b: np.float64(b) ** (-1.0 * np.arange(d // 2) / d)


def _mut_theta_shift(m):
    m.inv_freq = lambda d, b: np.float64(b) ** (-2.0 * (np.arange(d // 2) + 1) / d)


def _mut_theta_f32(m):
    m.inv_freq = lambda d, b: (np.float32(b) ** (np.float32(-2.0) * np.arange(d // 2, dtype=np.float32)
                                                 / np.float32(d))).astype(np.float64)


def _mut_patch_before_rotate(m):
    def rt(x, *, tensor, family, delta, rotate_this, bands, d_rot, base, pairing, factors=(), patch=True):
        y = np.array(x, dtype=np.float64)
        if patch:
            for f in factors:
                if f.tensor == tensor:
                    m.add_patch(y, f.u, f.vt, f.col0)
        return m.rotate(y, delta, bands, d_rot, base, pairing) if rotate_this else y
    m.rehydrate_tensor = rt


def _mut_patch_rank_reversed(m):
    def ap(y, u, vt, col0):
        w, k = vt.shape[1], u.shape[1]
        for j in range(k):
            y[:, col0:col0 + w] += np.outer(u[:, j], vt[k - 1 - j, :])
        return y
    m.add_patch = ap


def _mut_round_truncate(m):
    def rb(y):
        r32 = np.asarray(y, np.float64).astype(np.float32)
        return (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    m.round_bf16 = rb


def _mut_round_double(m):
    import torch
    def rb(y):
        f = np.asarray(y, np.float64).astype(np.float32)
        return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    m.round_bf16 = rb


def _mut_page_no_slot0(m):
    def ps(T, bt, slot0, P):
        s = np.arange(T)
        return np.asarray(bt)[s // P], s % P
    m.page_slots = ps


def _mut_v_rotated(m):
    orig = m.rehydrate_gqa
    def rg(k, v, delta, **kw):
        yk, yv = orig(k, v, delta, **kw)
        return yk, m.rotate(yv, delta, m.band_offsets(m.GQA, kw["num_kv_heads"], kw["head_dim"]),
                            kw["head_dim"], kw["base"], kw.get("pairing", m.NEOX))
    m.rehydrate_gqa = rg


def _mut_mla_latent_band(m):
    orig = m.band_offsets
    m.band_offsets = lambda fam, h=0, d=0, lat=0: [0] if fam == m.MLA else orig(fam, h, d, lat)


def _mut_sections_off_by_one(m):
    orig = m.pair_sections
    m.pair_sections = lambda d, sec: np.roll(orig(d, sec), 1)


def _mut_sections_all_t(m):
    m.pair_sections = lambda d, sec: np.zeros(d // 2, dtype=np.int64)


def _mut_theta_within_section(m):
    def token_phases(positions, d_rot, base, sections):
        pos = np.asarray(positions, dtype=np.int64).reshape(len(positions), -1)
        sec = m.pair_sections(d_rot, sections)
        idx = np.arange(d_rot // 2) - np.array([0, sections[0], sections[0] + sections[1]])[sec]
        phi = pos[:, sec] * (np.float64(base) ** (-2.0 * idx / d_rot))[None, :]
        return np.cos(phi), np.sin(phi)
    m.token_phases = token_phases


def _mut_first_token_positions(m):
    orig = m.token_phases
    m.token_phases = lambda pos, d, b, sec: orig(np.repeat(np.asarray(pos)[:1], len(pos), 0), d, b, sec)


def _mut_abs_terms_scaled(m):
    orig = m.abs_terms
    m.abs_terms = lambda x, **kw: orig(x, **kw) * 1000.0


def _mut_abs_terms_no_patch(m):
    orig = m.abs_terms
    m.abs_terms = lambda x, **kw: orig(x, **dict(kw, patch=False))


def _mut_abs_terms_signed(m):
    """|sum of terms| instead of the sum of |terms|: a bound that shrinks where terms cancel."""
    def at(x, **kw):
        kw.pop("family", None)
        return np.abs(m.rehydrate_tensor(x, family=m.GQA, **kw))
    m.abs_terms = at


def _mut_abs_terms_cos_only(m):
    """The rotated pair's sin terms dropped from S."""
    orig_phases = m.phases
    orig = m.abs_terms

    def at(x, **kw):
        m.phases = lambda d, r, b: (orig_phases(d, r, b)[0], 0.0 * orig_phases(d, r, b)[1])
        try:
            return orig(x, **kw)
        finally:
            m.phases = orig_phases
    m.abs_terms = at


MUTANTS = [_mut_sign, _mut_cos_sin_swapped, _mut_pairing, _mut_theta_half, _mut_theta_shift,
           _mut_theta_f32, _mut_patch_before_rotate, _mut_patch_rank_reversed, _mut_round_truncate,
           _mut_round_double, _mut_page_no_slot0, _mut_v_rotated, _mut_mla_latent_band,
           _mut_sections_off_by_one, _mut_sections_all_t, _mut_theta_within_section, _mut_first_token_positions,
           _mut_abs_terms_scaled, _mut_abs_terms_no_patch, _mut_abs_terms_signed, _mut_abs_terms_cos_only]


@pytest.mark.parametrize("mutate", MUTANTS, ids=lambda f: f.__name__[5:])
def test_pins_catch_planted_mistake(mutate):
    m = _fresh_oracle()
    mutate(m)
    caught = []
    for pin in ORACLE_PINS:
        try:
            pin(m)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutation {mutate.__name__}"


BUILDER_PATH = os.path.join(os.path.dirname(builder.__file__), "builder_oracle.py")


def _fresh_builder():
    spec = importlib.util.spec_from_file_location("oracle.builder_oracle_mutant", BUILDER_PATH)
    m = importlib.util.module_from_spec(spec)
    m.__package__ = "oracle"
    spec.loader.exec_module(m)
    return m


def _bmut_unrotated(m):
    m.rotate = lambda x, *a, **k: np.asarray(x, dtype=np.float64)


def _bmut_sigma_in_v(m):
    orig = m.truncated_svd

    def f(d, k):
        us, vt, s = orig(d, k)
        return us / s[:k][None, :], vt * s[:k][:, None], s
    m.truncated_svd = f


def _bmut_smallest(m):
    def f(d, k):
        u, s, vt = np.linalg.svd(d, full_matrices=False)
        return u[:, -k:] * s[-k:][None, :], vt[-k:], s
    m.truncated_svd = f


def _bmut_rank_minus_one(m):
    orig = m.truncated_svd

    def f(d, k):
        us, vt, s = orig(d, k)
        return us[:, : k - 1], vt[: k - 1], s
    m.truncated_svd = f


@pytest.mark.parametrize("mutate", [_bmut_unrotated, _bmut_sigma_in_v, _bmut_smallest, _bmut_rank_minus_one],
                         ids=lambda f: f.__name__[6:])
def test_builder_pin_catches_planted_mistake(mutate):
    m = _fresh_builder()
    mutate(m)
    with pytest.raises(AssertionError):
        pin_builder_planted(m)


def _omut_sum_not_mean(m):
    orig = m.orbit_deficit
    m.orbit_deficit = lambda xs, x, ds, **kw: orig(xs, x, ds, **kw) * len(xs)


def _omut_first_delta(m):
    orig = m.orbit_deficit
    m.orbit_deficit = lambda xs, x, ds, **kw: orig(xs, x, [ds[0]] * len(ds), **kw)


def _omut_unrotated(m):
    m.rotate = lambda x, *a, **k: np.asarray(x, dtype=np.float64)


def _omut_drop_last(m):
    orig = m.orbit_deficit
    m.orbit_deficit = lambda xs, x, ds, **kw: orig(xs[:-1], x, ds[:-1], **kw) if len(xs) > 1 else orig(xs, x, ds, **kw)


@pytest.mark.parametrize("mutate", [_omut_sum_not_mean, _omut_first_delta, _omut_unrotated, _omut_drop_last],
                         ids=lambda f: f.__name__[6:])
def test_orbit_pin_catches_planted_mistake(mutate):
    m = _fresh_builder()
    mutate(m)
    with pytest.raises(AssertionError):
        pin_orbit_mean(m)


# ---------------------------------------------------------------- tolerance predicate
def test_angle_term_bounds_the_fp64_angle_uncertainty():
    """The tolerance's angle term A covers what an angle formed in fp64 leaves open: with
    every theta_i moved by one fp64 ulp (two correct pow evaluations may differ so), the
    rotated outputs at delta = 2^31 - 1 move by at most A, and by a visible share of it
    (the bound is not vacuous). A vanishes where nothing turns."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((20, 128))
    bands, d_rot, base = [0, 64], 64, 1e4
    kw = dict(tensor=0, rotate_this=True, bands=bands, d_rot=d_rot, base=base, pairing=O.NEOX)
    for delta in (2 ** 31 - 1, -(2 ** 31 - 1), 123457):
        A = O.angle_terms(x, delta=delta, **kw)
        y0 = O.rotate(x, delta, bands, d_rot, base, O.NEOX)
        for direction in (np.inf, -np.inf):
            th = np.nextafter(O.inv_freq(d_rot, base), direction)   # one ulp off, every pair
            c, s = np.cos(np.float64(delta) * th), np.sin(np.float64(delta) * th)
            y1 = np.array(x, copy=True)
            p, q = O.pair_columns(d_rot, O.NEOX)
            for o in bands:
                y1[:, o + p] = x[:, o + p] * c - x[:, o + q] * s
                y1[:, o + q] = x[:, o + p] * s + x[:, o + q] * c
            moved = np.abs(y1 - y0)
            assert np.all(moved <= A + 1e-15), (delta, float((moved - A).max()))
            if abs(delta) > 2 ** 30:
                assert moved.max() > 0.02 * A.max()
    assert np.all(O.angle_terms(x, delta=0, **kw) == 0)
    assert np.all(O.angle_terms(x, delta=5000, **dict(kw, rotate_this=False)) == 0)
    uni = O.angle_terms(x, delta=0, positions=np.full((20, 3), 777), sections=(8, 12, 12), **kw)
    assert np.array_equal(uni, O.angle_terms(x, delta=777, **kw))   # uniform offsets: the delta path


def test_tolerance_predicate():
    y = np.array([1.0, -2.5, 3.0e-3, 100.0])
    r = O.round_bf16(y)
    S = np.abs(y)
    assert tol.check_bf16(r, y, r, S, 8)["fail"] == 0
    one_up = (r.astype(np.int64) + 1).astype(np.uint16)
    assert tol.check_bf16(one_up, y, r, S, 8)["fail"] == 0          # one ulp away: P1
    two_up = (r.astype(np.int64) + 2).astype(np.uint16)
    assert tol.check_bf16(two_up, y, r, S, 8)["fail"] == 4          # two ulps, small S: both fail
    # cancellation: |y| tiny next to S; an error within gamma_n*S passes through P2 only
    y2 = np.array([1e-9]); S2 = np.array([4.0]); r2 = O.round_bf16(y2)
    g2 = O.round_bf16(np.array([1e-9 + 5 * 4.0 * 2.0 ** -24]))
    res = tol.check_bf16(g2, y2, r2, S2, 8)
    assert res["fail"] == 0 and res["p2_only"] == 1
    assert tol.bf16_ord(np.array([0x0000, 0x8000], np.uint16)).tolist() == [0, 0]
    assert tol.bf16_ord(np.array([0x8001], np.uint16))[0] == -1


# ---------------------------------------------------------------- planted mistakes in the tolerance
TOL_PATH = os.path.join(os.path.dirname(tol.__file__), "tolerance.py")


def _fresh_tolerance():
    spec = importlib.util.spec_from_file_location("tolerance_mutant", TOL_PATH)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _tmut_ulp_f32_is_bf16(t):
    t.ulp_f32 = t.ulp_bf16


def _tmut_gamma_bf16_unit(t):
    t.U32 = 2.0 ** -8


def _tmut_zero_ulp_from_frexp(t):
    """Zero's spacing taken from frexp's exponent 0 (2^-8 and 2^-24) instead of the smallest subnormal."""
    t._binade = lambda x: np.maximum(np.frexp(np.asarray(x, dtype=np.float64))[1], -125)


def _tmut_f32_ignores_S(t):
    orig = t.check_f32
    t.check_f32 = lambda g, y, S, n, A=None: orig(g, y, np.zeros_like(np.asarray(S)), n, A)


def _tmut_ulp_bf16_doubled(t):
    orig = t.ulp_bf16
    t.ulp_bf16 = lambda x: 2.0 * orig(x)


def _tmut_p1_two_codes(t):
    orig = t.bf16_ord
    t.bf16_ord = lambda bits: orig(bits) // 2


@pytest.mark.parametrize("mutate", [_tmut_ulp_f32_is_bf16, _tmut_gamma_bf16_unit, _tmut_zero_ulp_from_frexp,
                                    _tmut_f32_ignores_S, _tmut_ulp_bf16_doubled, _tmut_p1_two_codes],
                         ids=lambda f: f.__name__[6:])
def test_tolerance_pins_catch_planted_mistake(mutate):
    t = _fresh_tolerance()
    mutate(t)
    caught = []
    for pin in TOLERANCE_PINS:
        try:
            pin(t, O)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutation {mutate.__name__}"
