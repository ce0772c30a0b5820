"""GPU patch builder against LAPACK (Kamera preprint §2 Eq. 2 and App. A compile step).

The builder returns U*Sigma, V and sigma for the deficit of stored rows. The
oracle forms the same deficit in fp64 and takes LAPACK's SVD (gesdd). Checks:

* Eckart-Young: the builder's rank-m residual ||Delta - U V^T||_F^2 is never
  below LAPACK's optimum sum_{i>=m} sigma_i^2, and exceeds it by no more than
  the subspace-iteration error of the case plus the bound that rounding U and V
  to the storage dtype allows (derived below);
* sigma (fp64) against LAPACK's singular values;
* for planted spectra, sigma against the planted values within Weyl's bound
  ||Delta_stored - Delta_planted||_2 (the storage rounding of KV(B|A));
* V has orthonormal columns (to the storage rounding);
* a full-rank patch from the builder, applied by the operator, reproduces the
  conditioned rows (Eq. 1 with m = T).

Rounding bound: U' = U(1+e), |e| <= u elementwise (u = 2^-8 bf16, 2^-24 fp32),
so ||U V^T - U' V'^T||_F <= ||U - U'||_F ||V||_2 + ||U'||_2 ||V - V'||_F with
||U - U'||_F <= u/(1-u) ||U'||_F and the same for V.
"""
import numpy as np
import pytest
import torch

import oracle.kamera_oracle as O
from oracle import tolerance as tol
from oracle.builder_oracle import deficit, orbit_deficit, residual_energy, truncated_svd
from tests.gpu_util import say
from workloads.builder_inputs import BuilderCase, orbit_parts
from workloads.configs import BF16, F32, GPTJ, GQA, MLA, NEOX, LayoutSpec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from position_free_kv_amd import abi
    abi.lib()
    yield


def _abi_layout(lay: LayoutSpec):
    from position_free_kv_amd import abi
    return abi.make_layout(lay.family, lay.dtype, 1, num_kv_heads=lay.num_kv_heads, head_dim=lay.head_dim,
                           latent_dim=lay.latent_dim, rope_dim=lay.rope_dim, pairing=lay.pairing,
                           rope_base=lay.rope_base, page_size=lay.page_size)


def _geometry(lay: LayoutSpec):
    bands = O.band_offsets(lay.family, lay.num_kv_heads, lay.head_dim, lay.latent_dim)
    d_rot = O.rotary_width(lay.family, lay.head_dim, lay.rope_dim)
    return bands, d_rot


def conditioned_rows(case: BuilderCase, canon: np.ndarray) -> np.ndarray:
    """Stored KV(B|A) = round(R(delta) KV(B|empty) + planted deficit on the patched columns)."""
    lay = case.layout
    if case.spectrum == "zero" and case.delta == 0:
        return canon.copy()
    x = O.upcast(canon, lay.dtype)
    bands, d_rot = _geometry(lay)
    y = O.rotate(x, case.delta, bands, d_rot, lay.rope_base, lay.pairing) if case.tensor == 0 else x.copy()
    y[:, case.col0:case.col0 + case.width] += case.deficit()
    return O.round_to(y, lay.dtype)


def _dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def run_builder(case: BuilderCase, rank: int, iterations: int, canon=None, cond=None):
    from position_free_kv_amd import abi
    lay = case.layout
    canon = case.canonical() if canon is None else canon
    cond = conditioned_rows(case, canon) if cond is None else cond
    T, W = case.num_tokens, case.width
    tdt, fill = (torch.int16, 0x7FA5) if lay.dtype == BF16 else (torch.float32, float("nan"))
    u = torch.full((T, rank), fill, dtype=tdt, device="cuda")   # NaN fill: every entry must be written
    v = torch.full((W, rank), fill, dtype=tdt, device="cuda")
    sig = torch.full((rank,), float("nan"), dtype=torch.float64, device="cuda")
    ws = torch.empty(abi.build_workspace_bytes(T, W, rank), dtype=torch.uint8, device="cuda")
    xc, xk = _dev(cond), _dev(canon)
    abi.build_patch(_abi_layout(lay), case.tensor, xc, xk, T, case.delta, case.col0, W, rank, iterations,
                    u, v, sig, ws)
    torch.cuda.synchronize()
    un, vn = u.cpu().numpy(), v.cpu().numpy()
    if lay.dtype == BF16:
        un, vn = un.view(np.uint16), vn.view(np.uint16)
    return canon, cond, un, vn, sig.cpu().numpy()


def oracle_deficit(case: BuilderCase, canon, cond) -> np.ndarray:
    lay = case.layout
    bands, d_rot = _geometry(lay)
    d = deficit(O.upcast(cond, lay.dtype), O.upcast(canon, lay.dtype), case.delta, bands=bands, d_rot=d_rot,
                base=lay.rope_base, pairing=lay.pairing, rotate_this=case.tensor == 0)
    return d[:, case.col0:case.col0 + case.width]


def unit_roundoff(dtype: int) -> float:
    return 2.0 ** -8 if dtype == BF16 else 2.0 ** -24


def check_case(case: BuilderCase, rank: int, iterations: int, sub_tol: float, sig_tol: float):
    """Run the builder and apply every check of the module docstring; returns the figures."""
    lay = case.layout
    canon, cond, u, v, sig = run_builder(case, rank, iterations)
    D = oracle_deficit(case, canon, cond)
    us_l, vt_l, s = truncated_svd(D, rank)
    opt = float(np.sum(s[rank:] ** 2))
    U, V = O.upcast(u, lay.dtype), O.upcast(v, lay.dtype)
    assert np.all(np.isfinite(U)) and np.all(np.isfinite(V)) and np.all(np.isfinite(sig))
    res = residual_energy(D, U, V.T)
    uu = unit_roundoff(lay.dtype) * (1 + 4 * unit_roundoff(lay.dtype))
    nV2 = np.linalg.norm(V, 2) * (1 + uu)
    rnd = uu * (np.linalg.norm(U) * nV2 + np.linalg.norm(U, 2) * np.linalg.norm(V))
    fro = float(np.linalg.norm(D))
    bound = np.sqrt(opt * (1 + sub_tol)) + rnd + 1e-10 * fro
    say(f"  T={case.num_tokens} W={case.width} m={rank} res={res:.6e} opt={opt:.6e} "
        f"excess={(np.sqrt(res) - np.sqrt(opt)):.3e} allowed={(bound - np.sqrt(opt)):.3e}")
    assert res >= opt * (1 - 1e-9) - 1e-13 * fro ** 2       # Eckart-Young: nothing beats the optimum
    assert np.sqrt(res) <= bound
    # singular values (fp64 on the device) against LAPACK's
    lam_err = np.abs(sig ** 2 - s[:rank] ** 2)
    assert np.all(lam_err <= sig_tol * s[:rank] ** 2 + 1e-12 * s[0] ** 2), (sig[:4], s[:4])
    # orthonormal columns of V, to the storage rounding: |(V'^T V')_ij - d_ij| <= 2u + u^2 (Cauchy-Schwarz)
    gram = V.T @ V
    assert np.abs(gram - np.eye(rank)).max() <= 2.5 * uu + 1e-12
    return dict(D=D, s=s, sig=sig, U=U, V=V, res=res, opt=opt)


def gqa(dtype, H, hd, base=1e6, pairing=NEOX):
    return LayoutSpec(GQA, dtype, 1, num_kv_heads=H, head_dim=hd, rope_base=base, pairing=pairing)


MLA_BF16 = LayoutSpec(MLA, BF16, 1, latent_dim=512, rope_dim=64, rope_base=1e4)


# ---------------------------------------------------------------------------------- planted spectra
def test_planted_fp32_gqa_keys():
    """Planted sigma_i = 0.3*0.9^i on K (rotated), fp32; builder sigma = planted within Weyl's bound."""
    case = BuilderCase(gqa(F32, 2, 64, base=1e4), tensor=0, num_tokens=300, delta=777, col0=0, width=128, seed=11)
    say("[builder] planted fp32 GQA K 300x128 m=16")
    r = check_case(case, rank=16, iterations=8, sub_tol=1e-9, sig_tol=1e-9)
    weyl = np.linalg.norm(r["D"] - case.deficit(), 2)
    assert np.all(np.abs(r["sig"] - case.sigma[:16]) <= weyl + 1e-12), (r["sig"][:4], case.sigma[:4], weyl)


@pytest.mark.parametrize("tensor,col0,width,rank", [(0, 0, 512, 32), (1, 128, 256, 8)])
def test_planted_bf16_c2_shape(tensor, col0, width, rank):
    """C2 row shape (4 heads x 128, base 1e6), 1024 tokens; K rotated, V slice not rotated."""
    case = BuilderCase(gqa(BF16, 4, 128), tensor=tensor, num_tokens=1024, delta=5000, col0=col0, width=width,
                       sigma0=8.0, ratio=0.85, seed=12)
    say(f"[builder] planted bf16 C2-shape tensor={tensor} cols=[{col0},{col0 + width}) m={rank}")
    # the bf16 rounding of KV(B|A) gives the deficit a flat tail near sigma_m: slower Ritz values
    check_case(case, rank=rank, iterations=16, sub_tol=1e-6, sig_tol=1e-4)


def test_planted_bf16_c4_shape():
    """C4 row shape (32 heads x 128, base 1e4): the whole 4096-wide K row of a 2048-token chunk,
    rank 32 (the widest rows the builder is measured on; p = 80 of 2048 directions). The bf16
    rounding of 2048 x 4096 stored rows leaves a noise floor of about 2^-9 (sqrt(T) + sqrt(W))
    ~ 0.2 in the deficit's spectrum, so the planted values decay slowly enough (0.95) that all
    32 kept ones stay well above it."""
    case = BuilderCase(gqa(BF16, 32, 128, base=1e4), tensor=0, num_tokens=2048, delta=4096, col0=0, width=4096,
                       sigma0=8.0, ratio=0.95, planted_rank=96, seed=14)
    say("[builder] planted bf16 C4-shape 2048x4096 m=32")
    check_case(case, rank=32, iterations=16, sub_tol=1e-6, sig_tol=1e-4)


@pytest.mark.parametrize("col0,width,rank,delta", [(0, 576, 32, -3000), (512, 64, 16, 4096)])
def test_planted_bf16_mla(col0, width, rank, delta):
    """MLA 512 + 64 row: the factor over the whole row, and the k_rope-only factor (exact: p = width)."""
    case = BuilderCase(MLA_BF16, tensor=0, num_tokens=512, delta=delta, col0=col0, width=width, sigma0=8.0,
                       ratio=0.85, seed=13)
    say(f"[builder] planted bf16 MLA cols=[{col0},{col0 + width}) m={rank} delta={delta}")
    check_case(case, rank=rank, iterations=16, sub_tol=1e-6, sig_tol=1e-4)


def test_planted_fp32_gptj_negative_delta():
    case = BuilderCase(gqa(F32, 1, 256, base=1e4, pairing=GPTJ), tensor=0, num_tokens=200, delta=-1234, col0=0,
                       width=256, seed=14)
    say("[builder] planted fp32 GPT-J pairing, delta=-1234")
    check_case(case, rank=24, iterations=8, sub_tol=1e-9, sig_tol=1e-9)


# ---------------------------------------------------------------------------------- other spectra
def test_exact_when_subspace_spans_everything():
    """T = 40 < 80: the iterated block spans the whole row space, so the result is the exact SVD."""
    case = BuilderCase(gqa(F32, 2, 64), tensor=0, num_tokens=40, delta=99, col0=0, width=128, spectrum="gaussian",
                       seed=15)
    say("[builder] exact case T=40, gaussian deficit")
    check_case(case, rank=32, iterations=0, sub_tol=1e-9, sig_tol=1e-9)


def test_exact_wide_ragged_row():
    """Width 2050 (65 column tiles, the last 2 columns wide: the Gram product takes its
    wide-row kernel) with T = 60: p = 60 spans the row space, so the result is the exact SVD."""
    case = BuilderCase(gqa(F32, 17, 128), tensor=0, num_tokens=60, delta=4321, col0=100, width=2050,
                       spectrum="gaussian", seed=23)
    say("[builder] exact case T=60 width=2050 (wide-row Gram kernel, ragged last tile)")
    check_case(case, rank=20, iterations=1, sub_tol=1e-9, sig_tol=1e-9)


@pytest.mark.parametrize("num_tokens,col0,width,rank", [(37, 0, 128, 16), (300, 40, 33, 33), (1, 0, 64, 1),
                                                        (5, 7, 2, 2), (200, 0, 79, 24)])
def test_exact_at_odd_and_tiny_subspaces(num_tokens, col0, width, rank):
    """p = min(80, width, T) = 37, 33, 1, 2, 79: the block spans the row space, so the result is
    the exact SVD; an odd p gives the eigensolver's round-robin tournament a bye (an empty
    player), and p <= 2 leaves it one pair or none."""
    case = BuilderCase(gqa(F32, 2, 64), tensor=0, num_tokens=num_tokens, delta=-77, col0=col0, width=width,
                       spectrum="gaussian", seed=19 + num_tokens)
    say(f"[builder] exact case T={num_tokens} width={width} (p={min(80, width, num_tokens)}) rank={rank}")
    check_case(case, rank=rank, iterations=1, sub_tol=1e-9, sig_tol=1e-9)


def test_flat_gaussian_spectrum():
    """No spectral gap: subspace iteration approaches the optimum more slowly (16 iterations, p = 80)."""
    case = BuilderCase(gqa(F32, 4, 128), tensor=0, num_tokens=1024, delta=321, col0=0, width=512,
                       spectrum="gaussian", seed=16)
    say("[builder] flat gaussian spectrum 1024x512 m=32")
    check_case(case, rank=32, iterations=16, sub_tol=1e-4, sig_tol=2e-3)


def test_zero_deficit():
    """KV(B|A) = KV(B|empty) at delta 0: sigma = 0, U*Sigma = +0 exactly, V still orthonormal."""
    case = BuilderCase(gqa(BF16, 4, 128), tensor=0, num_tokens=256, delta=0, col0=0, width=512, spectrum="zero",
                       seed=17)
    say("[builder] zero deficit")
    canon, cond, u, v, sig = run_builder(case, 16, 4)
    assert np.array_equal(canon, cond)
    assert np.all(u == 0) and np.all(sig == 0.0)
    V = O.upcast(v, BF16)
    assert np.abs(V.T @ V - np.eye(16)).max() <= 2.5 * 2.0 ** -8


# ---------------------------------------------------------------------------------- builder -> operator
def test_full_rank_patch_reproduces_conditioned_rows():
    """Eq. 1 with m = T: R(delta) KV(B|empty) + U V^T from the builder gives back KV(B|A) (fp32)."""
    from position_free_kv_amd import abi
    lay = gqa(F32, 2, 64, base=1e4)
    T, F, delta = 48, 128, 1234
    say("[builder] full-rank K and V patches through kamera_rehydrate")
    cases = [BuilderCase(lay, tensor=t, num_tokens=T, delta=delta, col0=0, width=F, spectrum="gaussian",
                         scale=0.5, seed=18) for t in (0, 1)]
    outs = []
    for c in cases:
        canon, cond, u, v, sig = run_builder(c, rank=T, iterations=2)
        outs.append((canon, cond, u, v))
    dev = [[_dev(a) for a in o] for o in outs]
    k_dst = torch.empty((T, F), dtype=torch.float32, device="cuda")
    v_dst = torch.empty((T, F), dtype=torch.float32, device="cuda")
    ch = abi.ChunkDesc(num_tokens=T, delta=delta, flags=abi.PATCH, k_src=dev[0][0], v_src=dev[1][0],
                       src_layer_stride=T * F, k_dst=k_dst, v_dst=v_dst, dst_layer_stride=T * F,
                       factors=[dict(u=dev[0][2], v=dev[0][3], tensor=0, width=F, rank=T),
                                dict(u=dev[1][2], v=dev[1][3], tensor=1, width=F, rank=T)])
    ws = torch.empty(abi.workspace_bytes(1, 0), dtype=torch.uint8, device="cuda")
    abi.rehydrate(_abi_layout(lay), ch, None, ws)
    torch.cuda.synchronize()
    for got, (canon, cond, u, v) in zip((k_dst, v_dst), outs):
        g = got.cpu().numpy().astype(np.float64)
        want = cond.astype(np.float64)
        err = np.abs(g - want)
        say(f"  max |rehydrated - KV(B|A)| = {err.max():.3e}")
        assert err.max() <= 2e-5 * (1 + np.abs(want).max())


# ---------------------------------------------------------------------------------- orbit patch
def stored_rows(lay: LayoutSpec, canon: np.ndarray, tensor: int, delta: int, col0: int, part: np.ndarray):
    """Stored KV(B|A) of one ordering: round(R(delta) canonical + part on the patched columns)."""
    x = O.upcast(canon, lay.dtype)
    bands, d_rot = _geometry(lay)
    y = O.rotate(x, delta, bands, d_rot, lay.rope_base, lay.pairing) if tensor == 0 else x.copy()
    y[:, col0:col0 + part.shape[1]] += part
    return O.round_to(y, lay.dtype)


def run_orbit(case: BuilderCase, conds, deltas, rank: int, iterations: int):
    from position_free_kv_amd import abi
    lay = case.layout
    T, W = case.num_tokens, case.width
    tdt, fill = (torch.int16, 0x7FA5) if lay.dtype == BF16 else (torch.float32, float("nan"))
    u = torch.full((T, rank), fill, dtype=tdt, device="cuda")
    v = torch.full((W, rank), fill, dtype=tdt, device="cuda")
    sig = torch.full((rank,), float("nan"), dtype=torch.float64, device="cuda")
    ws = torch.empty(abi.build_workspace_bytes(T, W, rank), dtype=torch.uint8, device="cuda")
    dconds = [_dev(c) for c in conds]
    abi.build_orbit_patch(_abi_layout(lay), case.tensor, dconds, deltas, _dev(case.canonical()), T, case.col0, W,
                          rank, iterations, u, v, sig, ws)
    torch.cuda.synchronize()
    un, vn = u.cpu().numpy(), v.cpu().numpy()
    if lay.dtype == BF16:
        un, vn = un.view(np.uint16), vn.view(np.uint16)
    return un, vn, sig.cpu().numpy()


@pytest.mark.parametrize("dtype,K", [(F32, 6), (BF16, 6), (BF16, 24)])
def test_orbit_patch_matches_lapack(dtype, K):
    """Orbit patch (preprint §5, reorder): K orderings place the chunk at offsets
    slot * 512; each ordering's conditioned rows carry a shared planted part plus a
    per-ordering part that averages to zero. The GPU factors of the mean deficit are
    checked against LAPACK on the oracle's orbit deficit (Eckart-Young, sigma), and sigma
    against the planted spectrum within Weyl's bound."""
    lay = gqa(dtype, 4, 128, base=1e4)
    case = BuilderCase(lay, tensor=0, num_tokens=512, delta=0, col0=0, width=512, sigma0=6.0, ratio=0.85,
                       planted_rank=48, seed=31)
    rank = 32
    say(f"[orbit] dtype={dtype} K={K}")
    canon = case.canonical()
    deltas = [512 * ((3 * k) % 4) + 7 * k for k in range(K)]
    parts = orbit_parts(case, K, spread=0.05)
    conds = [stored_rows(lay, canon, 0, d, 0, p) for d, p in zip(deltas, parts)]
    u, v, sig = run_orbit(case, conds, deltas, rank, 16)
    bands, d_rot = _geometry(lay)
    D = orbit_deficit([O.upcast(c, dtype) for c in conds], O.upcast(canon, dtype), deltas, bands=bands,
                      d_rot=d_rot, base=lay.rope_base, pairing=lay.pairing)
    _, _, s = truncated_svd(D, rank)
    opt = float(np.sum(s[rank:] ** 2))
    U, V = O.upcast(u, dtype), O.upcast(v, dtype)
    res = residual_energy(D, U, V.T)
    uu = unit_roundoff(dtype) * (1 + 4 * unit_roundoff(dtype))
    rnd = uu * (np.linalg.norm(U) * np.linalg.norm(V, 2) * (1 + uu) + np.linalg.norm(U, 2) * np.linalg.norm(V))
    bound = np.sqrt(opt * (1 + 1e-6)) + rnd + 1e-10 * np.linalg.norm(D)
    say(f"  res={res:.6e} opt={opt:.6e} excess={np.sqrt(res) - np.sqrt(opt):.3e} allowed={bound - np.sqrt(opt):.3e}")
    assert res >= opt * (1 - 1e-9) - 1e-13 * np.linalg.norm(D) ** 2
    assert np.sqrt(res) <= bound
    assert np.all(np.abs(sig ** 2 - s[:rank] ** 2) <= 1e-4 * s[:rank] ** 2 + 1e-12 * s[0] ** 2), (sig[:4], s[:4])
    weyl = np.linalg.norm(D - case.deficit(), 2)
    assert np.all(np.abs(sig - case.sigma[:rank]) <= weyl + 1e-9), (sig[:4], case.sigma[:4], weyl)


def test_orbit_of_one_is_the_single_patch():
    """One ordering: kamera_build_orbit_patch and kamera_build_patch give the same bytes."""
    case = BuilderCase(gqa(BF16, 2, 128), tensor=0, num_tokens=300, delta=4321, col0=0, width=256, sigma0=4.0,
                       ratio=0.85, seed=32)
    say("[orbit] K=1 vs single")
    canon, cond, u1, v1, s1 = run_builder(case, 16, 8)
    u2, v2, s2 = run_orbit(case, [cond], [case.delta], 16, 8)
    assert np.array_equal(u1, u2) and np.array_equal(v1, v2) and np.array_equal(s1, s2)


# ---------------------------------------------------------------------------------- removal patch
def test_removal_patch_in_place():
    """Removal patch (preprint §5, sliding-window survival): a survivor keeps its conditioned
    rows X in the pool; re-prefilled without the evicted chunk it would hold
    Y = R(-E) X + D with D low-rank (rank 48 planted). The builder forms the rank-64 patch
    of Y - R(-E) X from the stored rows, and the operator applies it in place
    (IN_PLACE | PATCH): the pool then matches the oracle applying the same factors, and
    lies within the truncation and rounding error of Y."""
    from position_free_kv_amd import abi
    P, H, hd, T, E, rank = 16, 4, 128, 200, 1500, 64
    lay = LayoutSpec(GQA, BF16, 1, num_kv_heads=H, head_dim=hd, rope_base=1e6, page_size=P)
    F = H * hd
    case = BuilderCase(lay, tensor=0, num_tokens=T, delta=-E, col0=0, width=F, sigma0=3.0, ratio=0.9,
                       planted_rank=48, seed=33)
    say("[removal] rank-64 removal patch applied in place")
    kept = case.canonical()                       # the survivor's stored (conditioned) rows
    target = conditioned_rows(case, kept)         # round(R(-E) kept + D)
    _, _, u, v, sig = run_builder(case, rank, 16, canon=kept, cond=target)
    pages = np.random.default_rng(3).permutation(24).astype(np.int32)[: (T + P - 1) // P]
    pool = torch.full((1, 24, P, F), 0x7FA5, dtype=torch.int16, device="cuda")
    slots = np.arange(T)
    flat = torch.from_numpy(pages[slots // P].astype(np.int64) * P + slots % P).cuda()
    pool.view(-1, F)[flat] = torch.from_numpy(kept.view(np.int16)).cuda()
    du, dv = _dev(u), _dev(v)
    ch = abi.ChunkDesc(num_tokens=T, delta=-E, flags=abi.PATCH | abi.IN_PLACE, block_table=pages, slot0=0,
                       factors=[dict(u=du, v=dv, tensor=0, col0=0, width=F, rank=rank)])
    lay_abi = _abi_layout(lay)
    ws = torch.empty(abi.batch_workspace_bytes(lay_abi, [ch]), dtype=torch.uint8, device="cuda")
    abi.rehydrate(lay_abi, ch, abi.make_pool(pool, None, num_pages=24), ws)
    torch.cuda.synchronize()
    got = pool.view(-1, F)[flat].cpu().numpy().view(np.uint16)
    # the operator against the oracle with the same (GPU-built) factors
    bands, d_rot = _geometry(lay)
    x = O.upcast(kept, BF16)
    fac = [O.Factor(0, 0, O.upcast(u, BF16), O.upcast(v, BF16).T)]
    kw = dict(tensor=0, delta=-E, rotate_this=True, bands=bands, d_rot=d_rot, base=lay.rope_base,
              pairing=lay.pairing, factors=fac, patch=True)
    y = O.rehydrate_tensor(x, family=GQA, **kw)
    res = tol.check_bf16(got, y, O.round_to(y, BF16), O.abs_terms(x, **kw), rank + 4)
    assert res["fail"] == 0, res
    # the pool now holds (close to) the re-prefilled rows
    err = O.upcast(got, BF16) - O.upcast(target, BF16)
    D = oracle_deficit(case, kept, target)
    _, _, s = truncated_svd(D, rank)
    floor = np.sqrt(np.sum(s[rank:] ** 2))
    say(f"  ||pool - target||_F = {np.linalg.norm(err):.4e}; Eckart-Young floor {floor:.4e}; "
        f"||D||_F = {np.linalg.norm(D):.4e}")
    # the pool is rounded to bf16 once more: allow one bf16 rounding of the result on top of the floor
    assert np.linalg.norm(err) <= floor + 2.0 ** -8 * np.linalg.norm(O.upcast(target, BF16)) + 1e-6
    # untouched slots keep their sentinel
    mask = np.ones(24 * P, bool)
    mask[flat.cpu().numpy()] = False
    assert bool((pool.view(-1, F)[torch.from_numpy(np.nonzero(mask)[0]).cuda()] == 0x7FA5).all())
