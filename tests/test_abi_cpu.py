"""C-ABI checks that need no GPU: symbols, struct layout, host-side validation.

Validation happens on the host before any HIP call, so every error path below
returns its status on a machine without a GPU. Device pointers here are fake
addresses that are never dereferenced.
"""
import ctypes
import os
import re

import time

import numpy as np
import pytest

from position_free_kv_amd import abi

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "kamera.h")
FAKE = 0x10_0000_0000  # 256-byte aligned fake device address, never dereferenced


def _gpu_present() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # noqa: BLE001
        return False


# Every call below is meant to stop in host validation. On a machine with a GPU a
# validation gap would send fake addresses to a real device, so the module does not run there.
pytestmark = pytest.mark.skipif(_gpu_present(), reason="host-validation tests use fake device addresses")


def header_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(kamera_\w+)\s*\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    L = abi.lib()
    names = header_functions()
    assert set(names) == set(abi.EXPORTED), names
    for n in names:
        assert hasattr(L, n), n
    assert abi.version().startswith("kamera-gfx950")


@pytest.mark.parametrize("lang,std", [("c", "c11"), ("c++", "c++11")])
def test_header_compiles_on_its_own(lang, std):
    """include/kamera.h is a self-contained C ABI: strict C11 and C++11 accept it alone."""
    import subprocess
    cc = "gcc" if lang == "c" else "g++"
    r = subprocess.run([cc, f"-std={std}", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only", "-x", lang,
                        HEADER], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_struct_sizes_match_header():
    # natural C layout on x86_64 (checked against the header's field order)
    assert ctypes.sizeof(abi.Layout) == 64
    assert ctypes.sizeof(abi.Factor) == 40
    assert ctypes.sizeof(abi.Chunk) == 88 + 4 * 40
    assert ctypes.sizeof(abi.Pool) == 32
    assert ctypes.sizeof(abi.Plan) == 64


def test_status_strings():
    L = abi.lib()
    for i, name in enumerate(abi.STATUS):
        assert L.kamera_status_string(i).decode() == name


def test_workspace_bytes_monotone():
    a = abi.workspace_bytes(1, 0)
    b = abi.workspace_bytes(64, 0)
    c = abi.workspace_bytes(64, 5000)
    assert 0 < a < b < c and c % 256 == 0
    assert abi.workspace_bytes(-1, 0) == 0


def gqa_layout(**kw):
    d = dict(num_kv_heads=4, head_dim=128, rope_base=1e6, page_size=16)
    d.update(kw)
    return abi.make_layout(abi.GQA, abi.BF16, 2, **d)


def chunk(**kw):
    d = dict(num_tokens=32, delta=100, flags=abi.PATCH, k_src=FAKE, v_src=FAKE + 0x100000, k_dst=FAKE + 0x200000,
             v_dst=FAKE + 0x300000, factors=[dict(u=FAKE + 0x400000, v=FAKE + 0x500000, tensor=0, width=512, rank=32)])
    d.update(kw)
    return abi.ChunkDesc(**d)


WS = (FAKE + 0x1000000, 1 << 20)


def status_of(fn):
    try:
        fn()
    except abi.KameraError as e:
        return e.name, str(e)
    return "KAMERA_OK", ""


@pytest.mark.parametrize("case,expect", [
    ("null_layout", "KAMERA_E_NULL"),
    ("bad_family", "KAMERA_E_UNSUPPORTED"),
    ("bad_dtype", "KAMERA_E_DTYPE"),
    ("zero_layers", "KAMERA_E_SHAPE"),
    ("odd_head_dim", "KAMERA_E_SHAPE"),
    ("bad_base", "KAMERA_E_SHAPE"),
    ("bad_pairing", "KAMERA_E_UNSUPPORTED"),
    ("negative_tokens", "KAMERA_E_SHAPE"),
    ("unknown_flag", "KAMERA_E_UNSUPPORTED"),
    ("delta_2_31", "KAMERA_E_DELTA"),
    ("rank_too_big", "KAMERA_E_RANK"),
    ("factor_cols_outside", "KAMERA_E_SHAPE"),
    ("factor_null", "KAMERA_E_NULL"),
    ("factor_bad_tensor", "KAMERA_E_SHAPE"),
    ("null_src", "KAMERA_E_NULL"),
    ("null_dst", "KAMERA_E_NULL"),
    ("misaligned_src", "KAMERA_E_ALIGN"),
    ("page_out_of_range", "KAMERA_E_PAGE"),
    ("slot0_out_of_page", "KAMERA_E_PAGE"),
    ("pages_overlap", "KAMERA_E_OVERLAP"),
    ("pool_missing", "KAMERA_E_NULL"),
    ("workspace_small", "KAMERA_E_WORKSPACE"),
    ("workspace_null", "KAMERA_E_WORKSPACE"),
    ("too_many_factors", "KAMERA_E_SHAPE"),
    ("positions_null", "KAMERA_E_NULL"),
    ("positions_misaligned", "KAMERA_E_ALIGN"),
    ("mrope_sum", "KAMERA_E_SHAPE"),
    ("mrope_negative", "KAMERA_E_SHAPE"),
    ("reserved2", "KAMERA_E_SHAPE"),
    ("positions_table_not_in_workspace", "KAMERA_E_WORKSPACE"),
])
def test_validation_errors(case, expect):
    lay = gqa_layout()
    pool = abi.make_pool(FAKE + 0x4000000, FAKE + 0x8000000, num_pages=8)
    run = lambda L=lay, cs=None, p=None, ws=WS: abi.rehydrate_batched(L, cs or [chunk()], p, ws, 0)
    if case == "null_layout":
        f = lambda: abi._check(abi.lib().kamera_rehydrate_batched(None, None, 0, None, None, 0, None))
    elif case == "bad_family":
        f = lambda: run(L=abi.make_layout(7, abi.BF16, 2, num_kv_heads=4, head_dim=128))
    elif case == "bad_dtype":
        f = lambda: run(L=abi.make_layout(abi.GQA, 9, 2, num_kv_heads=4, head_dim=128))
    elif case == "zero_layers":
        f = lambda: run(L=abi.make_layout(abi.GQA, abi.BF16, 0, num_kv_heads=4, head_dim=128))
    elif case == "odd_head_dim":
        f = lambda: run(L=gqa_layout(head_dim=127))
    elif case == "bad_base":
        f = lambda: run(L=gqa_layout(rope_base=-1.0))
    elif case == "bad_pairing":
        f = lambda: run(L=gqa_layout(pairing=5))
    elif case == "negative_tokens":
        f = lambda: run(cs=[chunk(num_tokens=-1)])
    elif case == "unknown_flag":
        f = lambda: run(cs=[chunk(flags=8)])
    elif case == "delta_2_31":
        f = lambda: run(cs=[chunk(delta=2 ** 31)])
    elif case == "rank_too_big":
        f = lambda: run(cs=[chunk(factors=[dict(u=FAKE, v=FAKE, width=512, rank=abi.MAX_RANK + 1)])])
    elif case == "factor_cols_outside":
        f = lambda: run(cs=[chunk(factors=[dict(u=FAKE, v=FAKE, col0=500, width=64, rank=8)])])
    elif case == "factor_null":
        f = lambda: run(cs=[chunk(factors=[dict(u=None, v=FAKE, width=512, rank=8)])])
    elif case == "factor_bad_tensor":
        f = lambda: run(cs=[chunk(factors=[dict(u=FAKE, v=FAKE, tensor=2, width=512, rank=8)])])
    elif case == "null_src":
        f = lambda: run(cs=[chunk(v_src=None)])
    elif case == "null_dst":
        f = lambda: run(cs=[chunk(k_dst=None)])
    elif case == "misaligned_src":
        f = lambda: run(cs=[chunk(k_src=FAKE + 1)])
    elif case == "page_out_of_range":
        f = lambda: run(cs=[chunk(block_table=np.array([0, 8]), k_dst=None, v_dst=None)], p=pool)
    elif case == "slot0_out_of_page":
        f = lambda: run(cs=[chunk(block_table=np.array([0, 1, 2]), slot0=16, k_dst=None, v_dst=None)], p=pool)
    elif case == "pages_overlap":
        f = lambda: run(cs=[chunk(block_table=np.array([0, 1]), k_dst=None, v_dst=None),
                            chunk(num_tokens=20, block_table=np.array([3, 1]), k_dst=None, v_dst=None)], p=pool)
    elif case == "pool_missing":
        f = lambda: run(cs=[chunk(block_table=np.array([0, 1]), k_dst=None, v_dst=None)], p=None)
    elif case == "workspace_small":
        f = lambda: run(ws=(WS[0], 64))
    elif case == "workspace_null":
        f = lambda: run(ws=(0, 1 << 20))
    elif case == "too_many_factors":
        c = chunk()
        c.c.num_factors = 5
        f = lambda: run(cs=[c])
    elif case == "positions_null":
        f = lambda: run(cs=[chunk(flags=abi.PATCH | abi.POSITIONS)])
    elif case == "positions_misaligned":
        f = lambda: run(cs=[chunk(flags=abi.POSITIONS, positions=FAKE + 2)])
    elif case == "mrope_sum":
        f = lambda: run(L=gqa_layout(mrope_section=(16, 24, 23)))
    elif case == "mrope_negative":
        f = lambda: run(L=gqa_layout(mrope_section=(-8, 36, 36)))
    elif case == "reserved2":
        L2 = gqa_layout()
        L2.reserved2 = 1
        f = lambda: run(L=L2)
    elif case == "positions_table_not_in_workspace":
        # sized for the packed descriptors alone: the per-token cos/sin table does not fit
        c = chunk(flags=abi.POSITIONS, positions=FAKE + 0x900000)
        f = lambda: run(cs=[c], ws=(WS[0], abi.workspace_bytes(1, 0)))
    name, msg = status_of(f)
    assert name == expect, (case, name, msg)


def test_batch_workspace_bytes_counts_tables():
    """Per-token cos/sin tables: (cos, sin) fp32 per pair of every token of a re-anchored chunk, tokens padded
    to whole 16-token tiles, 256-byte rounded."""
    lay = gqa_layout(mrope_section=(16, 24, 24))
    plain = abi.batch_workspace_bytes(lay, [chunk(), chunk(num_tokens=100)])
    assert plain == abi.workspace_bytes(2, 0)
    withpos = abi.batch_workspace_bytes(lay, [chunk(), chunk(num_tokens=100, flags=abi.POSITIONS, positions=FAKE)])
    assert withpos - plain == -(-112 * 64 * 8 // 256) * 256
    paged = abi.batch_workspace_bytes(lay, [chunk(num_tokens=40, slot0=3, block_table=np.array([1, 2, 3]))])
    assert paged == abi.workspace_bytes(1, 3)


def test_partial_page_sharing_is_not_an_overlap():
    """Two chunks may share a page when their slots do not collide: validation passes the
    overlap check and stops at the (deliberately too small) workspace, before any upload
    or launch, so the fake addresses are never touched on any machine."""
    pool = abi.make_pool(FAKE + 0x4000000, FAKE + 0x8000000, num_pages=8)
    a = chunk(num_tokens=10, block_table=np.array([2]), slot0=0, k_dst=None, v_dst=None)
    b = chunk(num_tokens=6, block_table=np.array([2]), slot0=10, k_dst=None, v_dst=None)
    tiny = (WS[0], 1)
    name, msg = status_of(lambda: abi.rehydrate_batched(gqa_layout(), [a, b], pool, tiny, 0))
    assert name == "KAMERA_E_WORKSPACE", msg
    c = chunk(num_tokens=6, block_table=np.array([2]), slot0=8, k_dst=None, v_dst=None)   # slots 8..13 collide
    name, msg = status_of(lambda: abi.rehydrate_batched(gqa_layout(), [a, c], pool, tiny, 0))
    assert name == "KAMERA_E_OVERLAP", msg


@pytest.mark.parametrize("P", [1, 3, 24])
def test_slot_overlap_at_other_page_sizes(P):
    """The slot check follows the layout's page size: with P-token pages, chunk a owns slots
    [s0, s0 + T) of its table's pages counted in P; a chunk on the next free slot of a's last
    page passes (and stops at the too-small workspace), one on a's last slot collides."""
    lay = gqa_layout(page_size=P)
    pool = abi.make_pool(FAKE + 0x4000000, FAKE + 0x8000000, num_pages=64)
    s0, T = (P - 1, 2 * P)                        # ends one slot before the end of its last page (P > 1)
    npg = -(-(s0 + T) // P)
    a = chunk(num_tokens=T, block_table=np.arange(10, 10 + npg), slot0=s0, k_dst=None, v_dst=None)
    end = (s0 + T) % P                            # first free slot of a's last page (0: the page is full)
    last = 10 + npg - 1
    tiny = (WS[0], 1)
    if end:
        b = chunk(num_tokens=P - end, block_table=np.array([last]), slot0=end, k_dst=None, v_dst=None)
        name, msg = status_of(lambda: abi.rehydrate_batched(lay, [a, b], pool, tiny, 0))
        assert name == "KAMERA_E_WORKSPACE", msg
    c = chunk(num_tokens=1, block_table=np.array([last]), slot0=(s0 + T - 1) % P, k_dst=None, v_dst=None)
    name, msg = status_of(lambda: abi.rehydrate_batched(lay, [a, c], pool, tiny, 0))
    assert name == "KAMERA_E_OVERLAP" and f"page {last}" in msg, msg
    name, msg = status_of(lambda: abi.rehydrate_batched(lay, [chunk(num_tokens=1, block_table=np.array([1]), slot0=P,
                                                                    k_dst=None, v_dst=None)], pool, tiny, 0))
    assert name == "KAMERA_E_PAGE", msg


def test_kernel_argument_route_still_checks_the_workspace():
    """A small dense batch is launched with the batch as the kernel's argument and the
    workspace unused, yet the call's contract is the same as on the workspace route: the
    workspace is checked (NULL, alignment, size) after the batch itself is validated."""
    lay = gqa_layout()
    name, _ = status_of(lambda: abi.rehydrate_batched(lay, [chunk()], None, (0, 1 << 20), 0))
    assert name == "KAMERA_E_WORKSPACE"
    name, _ = status_of(lambda: abi.rehydrate_batched(lay, [chunk()], None, (FAKE + 8, 1 << 20), 0))
    assert name == "KAMERA_E_ALIGN"
    need = abi.batch_workspace_bytes(lay, [chunk()])
    name, msg = status_of(lambda: abi.rehydrate_batched(lay, [chunk()] * 3, None, (FAKE, need), 0))
    assert name == "KAMERA_E_WORKSPACE" and "needed" in msg
    name, _ = status_of(lambda: abi.rehydrate_batched(lay, [chunk(delta=1 << 31)], None, (0, 0), 0))
    assert name == "KAMERA_E_DELTA"   # the batch is validated before the workspace


def test_empty_batches_need_no_gpu():
    abi.rehydrate_batched(gqa_layout(), [], None, WS, 0)
    abi.rehydrate_batched(gqa_layout(), [chunk(num_tokens=0)], None, WS, 0)
    pool = abi.make_pool(FAKE, FAKE + 0x100000, num_pages=4)
    abi.relocate(gqa_layout(), pool, None, 0, 0, 5, WS, 0)


def test_relocate_validates_pages():
    pool = abi.make_pool(FAKE, FAKE + 0x100000, num_pages=2)
    name, _ = status_of(lambda: abi.relocate(gqa_layout(), pool, None, 0, 40, 5, WS, 0))   # needs 3 pages
    assert name == "KAMERA_E_PAGE"
    name, _ = status_of(lambda: abi.relocate(gqa_layout(), pool, np.array([0, 5]), 0, 20, 5, WS, 0))
    assert name == "KAMERA_E_PAGE"
    # dense rows (no table): the range is checked against the pool before any table is built,
    # so the largest token count fails at once instead of allocating a table of 2^27 pages
    t0 = time.perf_counter()
    name, _ = status_of(lambda: abi.relocate(gqa_layout(), pool, None, 3, 2 ** 31 - 1, 5, WS, 0))
    assert name == "KAMERA_E_PAGE" and time.perf_counter() - t0 < 1.0
    name, _ = status_of(lambda: abi.relocate(gqa_layout(), pool, None, 32, 1, 5, WS, 0))   # row 32 of 32
    assert name == "KAMERA_E_PAGE"


def test_plan_struct_roundtrip_empty():
    plan = abi.plan_upload(gqa_layout(), [], None, WS, 0)
    assert plan.num_tasks == 0 and plan.kernel == 0
    abi.plan_launch(plan, 0)


# --------------------------------------------------------------------------- patch builder
def build_call(layout=None, **kw):
    lay = layout or gqa_layout()
    d = dict(tensor=0, x_cond=FAKE, x_canon=FAKE + 0x100000, num_tokens=64, delta=100, col0=0, width=512,
             rank=32, iterations=16, u_out=FAKE + 0x200000, v_out=FAKE + 0x300000, sigma_out=FAKE + 0x400000)
    d.update(kw)
    need = abi.build_workspace_bytes(d["num_tokens"], d["width"], d["rank"]) if d["num_tokens"] > 0 else 0
    ws = kw.pop("ws", None) if "ws" in kw else (FAKE + 0x1000000, need)
    d.pop("ws", None)
    return lambda: abi.build_patch(lay, workspace=ws, **d)


def test_build_workspace_bytes():
    a = abi.build_workspace_bytes(64, 512, 32)
    b = abi.build_workspace_bytes(1024, 512, 32)
    # Delta [T][W], G [W][W], Q and Z [p][W], H and E [p][p], lambda [p], V_m [W][m], all fp64
    p = 64
    assert a >= 8 * (64 * 512 + 512 * 512 + 2 * p * 512 + 2 * p * p + p + 512 * 32)
    assert a < b and a % 256 == 0 and b % 256 == 0
    assert abi.build_workspace_bytes(0, 512, 32) == 0 and abi.build_workspace_bytes(8, 512, 0) == 0


MLA_LAYOUT = dict(latent_dim=512, rope_dim=64, rope_base=1e4, page_size=16)


@pytest.mark.parametrize("kw,expect", [
    (dict(x_cond=None), "KAMERA_E_NULL"),
    (dict(v_out=None), "KAMERA_E_NULL"),
    (dict(tensor=2), "KAMERA_E_SHAPE"),
    (dict(num_tokens=0), "KAMERA_E_SHAPE"),
    (dict(col0=500, width=13), "KAMERA_E_SHAPE"),
    (dict(col0=-1), "KAMERA_E_SHAPE"),
    (dict(rank=0), "KAMERA_E_RANK"),
    (dict(rank=65), "KAMERA_E_RANK"),
    (dict(num_tokens=16, rank=17), "KAMERA_E_RANK"),
    (dict(width=8, rank=9), "KAMERA_E_RANK"),
    (dict(iterations=-1), "KAMERA_E_SHAPE"),
    (dict(iterations=65), "KAMERA_E_SHAPE"),
    (dict(delta=1 << 31), "KAMERA_E_DELTA"),
    (dict(x_canon=FAKE + 1), "KAMERA_E_ALIGN"),
    (dict(sigma_out=FAKE + 4), "KAMERA_E_ALIGN"),
    (dict(ws=(FAKE + 0x1000000, 1024)), "KAMERA_E_WORKSPACE"),
    (dict(ws=(0, 1 << 30)), "KAMERA_E_WORKSPACE"),
    (dict(ws=(FAKE + 0x1000008, 1 << 30)), "KAMERA_E_ALIGN"),
])
def test_build_patch_validation(kw, expect):
    name, msg = status_of(build_call(**kw))
    assert name == expect, msg


def test_build_patch_mla_has_one_tensor():
    lay = abi.make_layout(abi.MLA, abi.BF16, 1, **MLA_LAYOUT)
    name, _ = status_of(build_call(lay, tensor=1, width=576))
    assert name == "KAMERA_E_SHAPE"
    name, _ = status_of(build_call(lay, tensor=0, col0=512, width=65))
    assert name == "KAMERA_E_SHAPE"


def orbit_call(k=3, **kw):
    lay = kw.pop("layout", None) or gqa_layout()
    conds = kw.pop("conds", [FAKE + 0x100000 * (i + 1) for i in range(k)])
    deltas = kw.pop("deltas", [2048 * i for i in range(len(conds))])
    d = dict(tensor=0, x_canon=FAKE, num_tokens=64, col0=0, width=512, rank=32, iterations=16,
             u_out=FAKE + 0x4000000, v_out=FAKE + 0x5000000, sigma_out=FAKE + 0x6000000)
    d.update(kw)
    ws = (FAKE + 0x10000000, abi.build_workspace_bytes(d["num_tokens"], d["width"], d["rank"]))
    return lambda: abi.build_orbit_patch(lay, d.pop("tensor"), conds, deltas, workspace=ws, **d)


@pytest.mark.parametrize("kw,expect", [
    (dict(k=0), "KAMERA_E_SHAPE"),
    (dict(k=33), "KAMERA_E_SHAPE"),
    (dict(conds=[FAKE, 0, FAKE + 0x200000]), "KAMERA_E_NULL"),
    (dict(conds=[FAKE, FAKE + 1], deltas=[0, 1]), "KAMERA_E_ALIGN"),
    (dict(deltas=[0, 1 << 31, 5]), "KAMERA_E_DELTA"),
    (dict(rank=65), "KAMERA_E_RANK"),
    (dict(x_canon=None), "KAMERA_E_NULL"),
])
def test_build_orbit_patch_validation(kw, expect):
    name, msg = status_of(orbit_call(**kw))
    assert name == expect, msg


def test_in_place_patch_needs_v_pool_only_for_v_factors():
    """In place, V is touched only by a V factor: a K-only patch needs no V pool."""
    pool = abi.make_pool(FAKE + 0x4000000, None, num_pages=8)
    tiny = (WS[0], 1)
    kf = dict(u=FAKE + 0x400000, v=FAKE + 0x500000, tensor=0, width=512, rank=32)
    vf = dict(u=FAKE + 0x600000, v=FAKE + 0x700000, tensor=1, width=512, rank=32)
    k_only = chunk(num_tokens=20, flags=abi.PATCH | abi.IN_PLACE, block_table=np.array([1, 4]), slot0=0,
                   k_src=None, v_src=None, k_dst=None, v_dst=None, factors=[kf])
    name, msg = status_of(lambda: abi.rehydrate_batched(gqa_layout(), [k_only], pool, tiny, 0))
    assert name == "KAMERA_E_WORKSPACE", msg
    with_v = chunk(num_tokens=20, flags=abi.PATCH | abi.IN_PLACE, block_table=np.array([1, 4]), slot0=0,
                   k_src=None, v_src=None, k_dst=None, v_dst=None, factors=[kf, vf])
    name, msg = status_of(lambda: abi.rehydrate_batched(gqa_layout(), [with_v], pool, tiny, 0))
    assert name == "KAMERA_E_NULL" and "v_pool" in msg, msg


def test_noalloc_rejects_batches_beyond_its_scratch():
    """The allocation-free entry point validates the batch like kamera_rehydrate_batched, then
    rejects one whose packed form and cos/sin tables exceed its fixed scratch, before any HIP
    call (so the fake addresses are never touched)."""
    lay = gqa_layout(mrope_section=(16, 24, 24))
    name, _ = status_of(lambda: abi.rehydrate_batched_noalloc(lay, [chunk(delta=1 << 31)], None, 0))
    assert name == "KAMERA_E_DELTA"
    big = chunk(num_tokens=10000, flags=abi.POSITIONS, positions=FAKE + 0x900000)   # 5 MB of cos/sin table
    assert abi.batch_workspace_bytes(lay, [big]) > abi.NOALLOC_SCRATCH_BYTES
    name, msg = status_of(lambda: abi.rehydrate_batched_noalloc(lay, [big], None, 0))
    assert name == "KAMERA_E_WORKSPACE" and "at most" in msg, msg
    name, _ = status_of(lambda: abi.rehydrate_batched_noalloc(lay, [], None, 0))   # nothing to do
    assert name == "KAMERA_OK"


def test_overlap_check_scales_with_the_batch_not_the_pool():
    """Overlapping pool slots are found from the batch's own page entries: a pool of 2^30
    pages costs no more than a small one, a repeated page inside one chunk's table is an
    overlap, and chunks sharing a page on disjoint slots are not."""
    big_pool = abi.make_pool(FAKE + 0x4000000, FAKE + 0x8000000, num_pages=1 << 30)
    a = chunk(num_tokens=40, block_table=np.array([5, 1 << 29, 7]), slot0=3, k_dst=None, v_dst=None)
    b = chunk(num_tokens=20, block_table=np.array([(1 << 30) - 1, 7]), slot0=0, k_dst=None, v_dst=None)
    t0 = time.perf_counter()
    name, msg = status_of(lambda: abi.rehydrate_batched(gqa_layout(), [a, b], big_pool, (WS[0], 1), 0))
    assert time.perf_counter() - t0 < 0.5
    assert name == "KAMERA_E_OVERLAP" and "chunks 0 and 1" in msg and "page 7" in msg, msg
    rep = chunk(num_tokens=40, block_table=np.array([4, 6, 4]), slot0=0, k_dst=None, v_dst=None)
    name, msg = status_of(lambda: abi.rehydrate_batched(gqa_layout(), [rep], big_pool, (WS[0], 1), 0))
    assert name == "KAMERA_E_OVERLAP" and "twice" in msg, msg
    c = chunk(num_tokens=3, block_table=np.array([7]), slot0=8, k_dst=None, v_dst=None)   # after a's slots 0..10
    d = chunk(num_tokens=10, block_table=np.array([9, 7]), slot0=10, k_dst=None, v_dst=None)
    name, msg = status_of(lambda: abi.rehydrate_batched(gqa_layout(), [a, c, d], big_pool, (WS[0], 1), 0))
    assert name == "KAMERA_E_OVERLAP", msg
    e = chunk(num_tokens=5, block_table=np.array([7]), slot0=11, k_dst=None, v_dst=None)  # slots 11..15: free
    name, msg = status_of(lambda: abi.rehydrate_batched(gqa_layout(), [a, e], big_pool, (WS[0], 1), 0))
    assert name == "KAMERA_E_WORKSPACE", msg


@pytest.mark.parametrize("case", ["unknown_unit", "valu_head64", "valu_positions", "valu_rank96", "mfma_f32"])
def test_patch_unit_validation(case):
    """Which unit adds the patch is validated on the host: the VALU form exists for bf16 heads of
    128 columns with at most two k-steps and no per-token offsets; the MFMA unit for batches the
    bf16 matrix-core kernel can run."""
    lay, cs = gqa_layout(patch_unit=abi.PATCH_UNIT_VALU), [chunk()]
    if case == "unknown_unit":
        lay = gqa_layout(patch_unit=3)
    elif case == "valu_head64":
        lay = gqa_layout(num_kv_heads=8, head_dim=64, patch_unit=abi.PATCH_UNIT_VALU)
    elif case == "valu_positions":
        lay = gqa_layout(patch_unit=abi.PATCH_UNIT_VALU, mrope_section=(16, 24, 24))
        cs = [chunk(flags=abi.PATCH | abi.POSITIONS, positions=FAKE + 0x900000)]
    elif case == "valu_rank96":
        cs = [chunk(factors=[dict(u=FAKE + 0x400000, v=FAKE + 0x500000, tensor=0, width=512, rank=96)])]
    elif case == "mfma_f32":
        lay = abi.make_layout(abi.GQA, abi.F32, 2, num_kv_heads=4, head_dim=128, rope_base=1e6,
                              patch_unit=abi.PATCH_UNIT_MFMA)
    name, msg = status_of(lambda: abi.rehydrate_batched(lay, cs, None, WS, 0))
    assert name == "KAMERA_E_UNSUPPORTED", (case, name, msg)
    ok = gqa_layout(patch_unit=abi.PATCH_UNIT_VALU)
    name, _ = status_of(lambda: abi.rehydrate_batched(ok, [chunk()], None, (WS[0], 64), 0))
    assert name == "KAMERA_E_WORKSPACE"   # a supported batch passes validation and stops at the workspace


def test_stream_probe_validation():
    """The measurement probes validate kind, size and alignment on the host before any launch."""
    cases = [((5, FAKE, FAKE + 4096, 4096), "KAMERA_E_UNSUPPORTED"), ((0, FAKE, FAKE + 4096, 100), "KAMERA_E_SHAPE"),
             ((0, None, FAKE, 4096), "KAMERA_E_NULL"), ((2, None, None, 4096), "KAMERA_E_NULL"),
             ((1, FAKE + 8, FAKE, 4096), "KAMERA_E_ALIGN"), ((0, FAKE, FAKE, 0), "KAMERA_OK")]
    for (kind, src, dst, n), want in cases:
        name, msg = status_of(lambda: abi.stream_probe(kind, src, dst, n, 0, 0))
        assert name == want, (kind, n, name, msg)
