"""GPU parity: the HIP library against the fp64 oracle, element by element (small sizes).

Bar (Kamera preprint §6: the rebuilt KV agrees with a recompute to one bf16 ulp): every bf16 output
is within one bf16 step of the once-rounded fp64 result (P1) or within the fp32
accumulation bound (P2); fp32 outputs meet P3. Indexing, untouched bytes and the
identity case are bit-exact.
"""
import dataclasses

import numpy as np
import pytest
import torch

from tests.gpu_util import (check_all, custom_workload, factor, gqa_chunks, pool_untouched_ok, say,
                            sentinel_code, touched_tensors)
from workloads import make_workload
from workloads.configs import (BF16, F32, GPTJ, GQA, IN_PLACE, MLA, NEOX, PATCH, POSITIONS, ChunkSpec, LayoutSpec,
                               grid_positions)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from position_free_kv_amd import abi
    abi.lib()   # fails loudly when the HIP library is missing
    yield


def run_dw(wl):
    from workloads.device import DeviceWorkload
    dw = DeviceWorkload(wl)
    dw.run()
    torch.cuda.synchronize()
    return dw


def assert_parity(dw, **kw):
    tot = check_all(dw, **kw)
    say(f"  compared {tot['n']} elements: fail={tot['fail']} p2_only={tot['p2_only']} exact={tot['exact']}")
    assert tot["fail"] == 0, tot["bad"][:3]
    return tot


# ---------------------------------------------------------------- the five configs, shrunk
@pytest.mark.parametrize("name,kw", [
    ("C1", {}),                                                        # full size (fp32, generic kernel)
    ("C2", dict(num_layers=2, num_chunks=3, tokens=200)),
    ("C3", dict(num_layers=2, num_chunks=2, tokens=150)),
    ("C4", dict(num_layers=1, tokens=48)),
    ("C5", dict(num_layers=2, num_chunks=8, max_tokens=300)),
])
def test_config_parity_small(name, kw):
    say(f"[parity-small] {name} {kw}")
    wl = make_workload(name, **kw)
    dw = run_dw(wl)
    assert_parity(dw)
    assert pool_untouched_ok(dw)
    if name == "C5":   # survivors: V pages untouched, byte for byte
        for ch in wl.chunks:
            if ch.role == "survivor":
                for layer in range(dw.L):
                    assert np.array_equal(dw.out_rows(ch, layer, 1), wl.pool_rows(ch, layer, 1))


def test_generic_kernel_large_fp32_batch():
    """fp32 batches run the generic kernel; one large enough to fill the chip takes 16-token
    workgroups (small ones take 4-token workgroups, as in the single-layer config above)."""
    say("[generic fp32, 16-token blocks]")
    wl = make_workload("C1", num_layers=8, num_chunks=8)
    assert sum(c.num_tokens for c in wl.chunks) * 8 * 2 >= 16 * 1024
    assert_parity(run_dw(wl))


# ---------------------------------------------------------------- bit-exact identity
@pytest.mark.parametrize("family", ["gqa128", "gqa64", "mla", "gqa_f32"])
def test_identity_delta0_nopatch(family):
    say(f"[identity] {family}")
    if family == "mla":
        lay = LayoutSpec(MLA, BF16, 2, latent_dim=512, rope_dim=64)
        chunks = [ChunkSpec(index=0, num_tokens=77, delta=0, flags=0, canon_id=0, dst_buffer=0)]
    else:
        hd = 64 if family == "gqa64" else 128
        dt = F32 if family == "gqa_f32" else BF16
        lay = LayoutSpec(GQA, dt, 2, num_kv_heads=3, head_dim=hd)
        chunks = gqa_chunks(2, [77, 16], 0, 3, hd, 0, patch=False)
    wl = custom_workload(lay, chunks)
    dw = run_dw(wl)
    for ch in wl.chunks:
        for layer in range(2):
            for t in touched_tensors(wl, ch):
                assert np.array_equal(dw.out_rows(ch, layer, t), wl.canonical(ch.canon_id, layer, t))


def test_mla_cache_passthrough_bytes():
    """Preprint §3 / Fig. 2: c_KV is reused byte for byte; only k_rope rotates."""
    wl = make_workload("C3", num_layers=2, num_chunks=3, tokens=70, patch=False)
    dw = run_dw(wl)
    for ch in wl.chunks:
        for layer in range(2):
            g = dw.out_rows(ch, layer, 0)
            assert np.array_equal(g[:, :512], wl.canonical(ch.canon_id, layer, 0)[:, :512])
    assert_parity(dw)


# ---------------------------------------------------------------- shapes and ranks
@pytest.mark.parametrize("T", [1, 15, 16, 17, 129, 300])
def test_ragged_token_counts(T):
    say(f"[ragged] T={T}")
    lay = LayoutSpec(GQA, BF16, 2, num_kv_heads=2, head_dim=128, rope_base=1e6)
    wl = custom_workload(lay, gqa_chunks(2, T, [513, -77], 2, 128, 32))
    assert_parity(run_dw(wl))


@pytest.mark.parametrize("rank", [1, 5, 8, 13, 32, 40, 64, 96, 128])
def test_ranks(rank):
    say(f"[rank] m={rank}")
    lay = LayoutSpec(GQA, BF16, 1, num_kv_heads=2, head_dim=128, rope_base=1e4)
    wl = custom_workload(lay, gqa_chunks(2, 70, [1000, 31], 2, 128, rank))
    assert_parity(run_dw(wl))


@pytest.mark.parametrize("delta", [1, -1, -65536, 2 ** 31 - 1, -(2 ** 31 - 1), 123457])
def test_deltas(delta):
    say(f"[delta] {delta}")
    lay = LayoutSpec(GQA, BF16, 1, num_kv_heads=1, head_dim=128, rope_base=1e6)
    wl = custom_workload(lay, gqa_chunks(1, 40, delta, 1, 128, 8))
    assert_parity(run_dw(wl))


@pytest.mark.parametrize("variant", ["gqa64", "gptj128", "gptj64", "mla_gptj", "gqa96_generic", "mla_f32",
                                     "mla_latent_odd_generic", "mla_latent448", "mla_rope_only"])
def test_layout_variants(variant):
    say(f"[layout] {variant}")
    if variant.startswith("mla"):
        dt = F32 if variant == "mla_f32" else BF16
        # 512: 128-column latent groups + a half group for the band; 448: 64-column groups;
        # 0: the band alone (one half group); 200: not a multiple of 64 (generic kernel)
        lat = {"mla_latent_odd_generic": 200, "mla_latent448": 448, "mla_rope_only": 0}.get(variant, 512)
        lay = LayoutSpec(MLA, dt, 2, latent_dim=lat, rope_dim=64, pairing=GPTJ if "gptj" in variant else NEOX)
        F = lat + 64
        chunks = [ChunkSpec(index=i, num_tokens=45 + 20 * i, delta=9000 * (i + 1), flags=PATCH, canon_id=i,
                            factors=[factor(i, 0, 0, 0, F, 16), factor(i, 1, 0, lat, 64, 8)], dst_buffer=i)
                  for i in range(2)]
    else:
        hd = {"gqa64": 64, "gptj128": 128, "gptj64": 64, "gqa96_generic": 96}[variant]
        lay = LayoutSpec(GQA, BF16, 2, num_kv_heads=3, head_dim=hd, pairing=GPTJ if "gptj" in variant else NEOX)
        chunks = gqa_chunks(2, [50, 33], [4000, -250], 3, hd, 16)
    wl = custom_workload(lay, chunks)
    assert_parity(run_dw(wl))


def test_partial_and_per_head_factors():
    """Factors covering a head each, and one covering an unaligned column range."""
    say("[factors] per-head + unaligned")
    lay = LayoutSpec(GQA, BF16, 2, num_kv_heads=4, head_dim=128, rope_base=1e6)
    facs = [factor(0, h, 0, 128 * h, 128, 8) for h in range(3)] + [factor(0, 3, 1, 40, 100, 24)]
    ch = ChunkSpec(index=0, num_tokens=90, delta=777, flags=PATCH, canon_id=0, factors=facs, dst_buffer=0)
    assert_parity(run_dw(custom_workload(lay, [ch])))


def test_layer_sparse_patch():
    """A factor with layer0 > 0 patches only the deeper layers (deep-half patches)."""
    say("[layer0]")
    lay = LayoutSpec(GQA, BF16, 4, num_kv_heads=2, head_dim=128, rope_base=1e6)
    ch = ChunkSpec(index=0, num_tokens=64, delta=321, flags=PATCH, canon_id=0,
                   factors=[factor(0, 0, 0, 0, 256, 32, layer0=2), factor(0, 1, 1, 0, 256, 32, layer0=3)],
                   dst_buffer=0)
    assert_parity(run_dw(custom_workload(lay, [ch])))


# ---------------------------------------------------------------- paged pool
@pytest.mark.parametrize("slot0", [0, 5, 15])
def test_paged_slot0(slot0):
    say(f"[paged] slot0={slot0}")
    P = 16
    lay = LayoutSpec(GQA, BF16, 2, num_kv_heads=2, head_dim=128, rope_base=1e6, page_size=P)
    rng = np.random.default_rng(slot0)
    chunks, pages = [], rng.permutation(40).astype(np.int32)
    cur = 0
    for i, T in enumerate([37, 16, 5]):
        n = -(-(slot0 + T) // P)
        chunks.append(ChunkSpec(index=i, num_tokens=T, delta=100 * i + 7, flags=PATCH, canon_id=i,
                                factors=[factor(i, 0, 0, 0, 256, 32), factor(i, 1, 1, 0, 256, 32)],
                                block_table=pages[cur:cur + n].copy(), slot0=slot0))
        cur += n
    wl = custom_workload(lay, chunks, dense_rows=[], num_pages=40)
    dw = run_dw(wl)
    assert_parity(dw)
    assert pool_untouched_ok(dw)


_PAGE_LAYOUTS = {
    # two-slab MFMA path (128-wide heads), one-slab MFMA path (64-wide heads), MLA rows, generic fp32 kernel
    "gqa128": (LayoutSpec(GQA, BF16, 2, num_kv_heads=2, head_dim=128, rope_base=1e6), 32),
    "gqa64": (LayoutSpec(GQA, BF16, 2, num_kv_heads=4, head_dim=64, rope_base=1e4), 32),
    "mla": (LayoutSpec(MLA, BF16, 2, latent_dim=512, rope_dim=64), 32),
    "f32": (LayoutSpec(GQA, F32, 2, num_kv_heads=2, head_dim=64, rope_base=1e4), 8),
}


@pytest.mark.parametrize("P", [1, 3, 8, 24, 32, 64, 256])
@pytest.mark.parametrize("kind", list(_PAGE_LAYOUTS))
def test_page_sizes(kind, P):
    """Pool pages of other sizes than 16 tokens ([K] §6 scatter into a paged pool): pages
    smaller than a 16-token tile (1, 3, 8: every row looks its page up), sizes that are not
    powers of two (3, 24: division instead of shifts; a tile straddles two 24-token pages), and
    pages of 32 to 256 tokens. Each batch holds a patched chunk starting on a page's last slot,
    an unpatched one starting mid-page, an in-place survivor and an in-place chunk with a patch;
    outputs are checked against the oracle and every slot no chunk owns keeps its sentinel."""
    say(f"[page size] {kind} P={P}")
    base, rank = _PAGE_LAYOUTS[kind]
    lay = dataclasses.replace(base, page_size=P)
    if lay.family == MLA:
        facs = lambda i: [factor(i, 0, 0, 0, 576, rank), factor(i, 1, 0, 512, 64, rank)]
    else:
        F = lay.num_kv_heads * lay.head_dim
        facs = lambda i: [factor(i, 0, 0, 0, F, rank), factor(i, 1, 1, 0, F, rank)]
    specs = [  # (tokens, slot0, delta, flags, role)
        (150, P - 1, 12345, PATCH, "rehydrate"),
        (37, P // 2, -777, 0, "rehydrate"),
        (70, min(P - 1, 5), -4096, IN_PLACE, "survivor"),
        (20, 0, 300, IN_PLACE | PATCH, "survivor"),
    ]
    need = [-(-(s0 + T) // P) for T, s0, _, _, _ in specs]
    num_pages = sum(need) + 5
    pages = np.random.default_rng(1000 + P).permutation(num_pages).astype(np.int32)
    chunks, cur = [], 0
    for i, ((T, s0, d, fl, role), n) in enumerate(zip(specs, need)):
        chunks.append(ChunkSpec(index=i, num_tokens=T, delta=d, flags=fl, canon_id=i,
                                factors=facs(i) if fl & PATCH else [], block_table=pages[cur:cur + n].copy(),
                                slot0=s0, role=role))
        cur += n
    dw = run_dw(custom_workload(lay, chunks, dense_rows=[], num_pages=num_pages))
    assert_parity(dw)
    assert pool_untouched_ok(dw)


@pytest.mark.parametrize("case", ["gqa_mfma", "gqa_stride_not_8", "mla"])
def test_strided_sources_and_pool_layers(case):
    """Sources that are slices of larger buffers (src_layer_stride > T*F, first row at an
    offset) and a pool whose layers are further apart than num_pages pages (layer_stride):
    the operator must follow the strides it is given. A source stride that is not a multiple
    of 8 elements takes the plain kernel (the 16-byte row loads need 8-element alignment);
    the others run on the matrix-core kernel. Destinations are checked against the oracle
    and every pool slot no chunk owns, the padding pages included, keeps its sentinel."""
    from position_free_kv_amd import abi
    from workloads.device import DeviceWorkload
    say(f"[strides] {case}")
    P = 16
    if case == "mla":
        lay = LayoutSpec(MLA, BF16, 3, latent_dim=512, rope_dim=64, page_size=P)
        facs = lambda i: [factor(i, 0, 0, 0, 576, 32), factor(i, 1, 0, 512, 64, 32)]
    else:
        lay = LayoutSpec(GQA, BF16, 3, num_kv_heads=2, head_dim=128, rope_base=1e6, page_size=P)
        facs = lambda i: [factor(i, 0, 0, 0, 256, 32), factor(i, 1, 1, 0, 256, 32)]
    pages = np.random.default_rng(11).permutation(24).astype(np.int32)
    chunks = [ChunkSpec(index=0, num_tokens=150, delta=4321, flags=PATCH, canon_id=0, factors=facs(0), dst_buffer=0),
              ChunkSpec(index=1, num_tokens=70, delta=-999, flags=PATCH, canon_id=1, factors=facs(1),
                        block_table=pages[0:5].copy(), slot0=3),
              ChunkSpec(index=2, num_tokens=100, delta=-2048, flags=IN_PLACE, canon_id=2,
                        block_table=pages[5:12].copy(), slot0=7, role="survivor")]
    wl = custom_workload(lay, chunks, dense_rows=[150], num_pages=24)
    dw = DeviceWorkload(wl)
    L, F = dw.L, dw.F
    keep = []
    # sources: every layer's rows inside a larger buffer, the first row `off` elements in
    extra = 4 if case == "gqa_stride_not_8" else 8 * F
    off = 8 * 3
    for ch, d in zip(wl.chunks, dw.descs):
        if ch.in_place:
            continue
        stride = ch.num_tokens * F + extra
        ptrs = []
        for src in dw.canon[ch.canon_id]:
            flat = torch.full((off + L * stride,), -1, dtype=src.dtype, device=src.device)
            for layer in range(L):
                flat[off + layer * stride: off + layer * stride + ch.num_tokens * F] = src[layer].reshape(-1)
            keep.append(flat)
            ptrs.append(flat.data_ptr() + off * flat.element_size())
        d.c.k_src = ptrs[0]
        d.c.v_src = ptrs[1] if len(ptrs) > 1 else None
        d.c.src_layer_stride = stride
    # pool: 3 pages of padding after each layer's 24 pages (sentinel-filled, never written)
    pad = 3
    padded = []
    for t in dw.pool:
        q = torch.full((L, wl.num_pages + pad, P, F), int(np.uint16(sentinel_code(BF16)).view(np.int16)),
                       dtype=t.dtype, device=t.device)
        q[:, :wl.num_pages] = t
        padded.append(q)
    dw.pool = padded
    dw.pool_desc = abi.make_pool(padded[0], padded[1] if len(padded) == 2 else None, wl.num_pages,
                                 layer_stride=(wl.num_pages + pad) * P * F)
    plan = abi.plan_upload(dw.layout, dw.descs, dw.pool_desc, dw.workspace)
    assert plan.kernel == (2 if case == "gqa_stride_not_8" else 1)   # 1: matrix-core kernel, 2: plain kernel
    abi.plan_launch(plan)
    torch.cuda.synchronize()
    assert_parity(dw)
    assert pool_untouched_ok(dw)
    code = int(np.uint16(sentinel_code(BF16)).view(np.int16))
    for q in padded:   # the padding pages between layers
        assert bool((q[:, wl.num_pages:] == code).all())


def test_mixed_dense_paged_and_in_place_batch():
    """One batch mixing dense destinations, paged destinations, an in-place survivor and an
    empty chunk: a batch with any paged chunk runs in layer-major task order, so every
    chunk type is decoded from within-layer offsets."""
    say("[mixed batch]")
    P = 16
    lay = LayoutSpec(GQA, BF16, 3, num_kv_heads=2, head_dim=128, rope_base=1e6, page_size=P)
    pages = np.random.default_rng(5).permutation(48).astype(np.int32)
    facs = lambda i: [factor(i, 0, 0, 0, 256, 32), factor(i, 1, 1, 0, 256, 32)]
    chunks = [ChunkSpec(index=0, num_tokens=150, delta=900, flags=PATCH, canon_id=0, factors=facs(0), dst_buffer=0),
              ChunkSpec(index=1, num_tokens=0, delta=5, flags=PATCH, canon_id=1, factors=facs(1), dst_buffer=1),
              ChunkSpec(index=2, num_tokens=70, delta=-300, flags=PATCH, canon_id=2, factors=facs(2),
                        block_table=pages[0:5].copy(), slot0=3),
              ChunkSpec(index=3, num_tokens=200, delta=-1234, flags=IN_PLACE, canon_id=3,
                        block_table=pages[5:18].copy(), slot0=0, role="survivor"),
              ChunkSpec(index=4, num_tokens=33, delta=77, flags=0, canon_id=4, dst_buffer=2)]
    wl = custom_workload(lay, chunks, dense_rows=[150, 1, 33], num_pages=48)
    dw = run_dw(wl)
    assert_parity(dw)
    assert pool_untouched_ok(dw)


@pytest.mark.parametrize("name", ["C2", "C3"])
def test_shared_basis_across_chunks(name):
    """One per-layer V basis aliased by every chunk's factor of a slot (only U differs):
    the kernel reads the same V rows for all chunks."""
    say(f"[shared basis] {name}")
    wl = make_workload(name, num_layers=2, num_chunks=3, tokens=140, shared_basis=True)
    dw = run_dw(wl)
    ptrs = {dw.factors[(f.key, f.slot)][1].data_ptr() for c in wl.chunks for f in c.factors}
    assert len(ptrs) == len({f.slot for c in wl.chunks for f in c.factors})   # one V buffer per slot
    assert_parity(dw)


def test_in_place_with_patch_mla_and_gqa():
    """In place with a patch: re-conditioning a resident chunk (rotate + add)."""
    say("[in-place+patch]")
    for lay, facs in [(LayoutSpec(GQA, BF16, 2, num_kv_heads=2, head_dim=128, rope_base=1e6),
                       [factor(0, 0, 0, 0, 256, 32), factor(0, 1, 1, 0, 256, 32)]),
                      (LayoutSpec(MLA, BF16, 2, latent_dim=512, rope_dim=64),
                       [factor(0, 0, 0, 0, 576, 32), factor(0, 1, 0, 512, 64, 32)])]:
        ch = ChunkSpec(index=0, num_tokens=50, delta=-4096, flags=IN_PLACE | PATCH, canon_id=0, factors=facs,
                       block_table=np.array([3, 0, 7, 1], np.int32), slot0=2, role="survivor")
        wl = custom_workload(lay, [ch], dense_rows=[], num_pages=8)
        dw = run_dw(wl)
        assert_parity(dw)
        assert pool_untouched_ok(dw)


def test_mla_survivor_in_place_touches_rope_only():
    lay = LayoutSpec(MLA, BF16, 3, latent_dim=512, rope_dim=64)
    ch = ChunkSpec(index=0, num_tokens=40, delta=-3000, flags=IN_PLACE, canon_id=0,
                   block_table=np.array([5, 2, 0], np.int32), slot0=0, role="survivor")
    wl = custom_workload(lay, [ch], dense_rows=[], num_pages=6)
    dw = run_dw(wl)
    assert_parity(dw)
    for layer in range(3):
        assert np.array_equal(dw.out_rows(ch, layer, 0)[:, :512], wl.pool_rows(ch, layer, 0)[:, :512])
    assert pool_untouched_ok(dw)


# ---------------------------------------------------------------- determinism, composition, plan reuse
def test_run_twice_bitwise_identical_and_plan_reuse():
    from position_free_kv_amd import abi
    wl = make_workload("C2", num_layers=2, num_chunks=2, tokens=130)
    from workloads.device import DeviceWorkload
    dw = DeviceWorkload(wl)
    dw.run()
    torch.cuda.synchronize()
    first = [t.clone() for buf in dw.dense for t in buf]
    plan = dw.plan()
    for _ in range(3):
        abi.plan_launch(plan)
    torch.cuda.synchronize()
    again = [t for buf in dw.dense for t in buf]
    assert all(torch.equal(a, b) for a, b in zip(first, again))


def test_reorder_same_slot_identical():
    """Two orderings that put the same chunk at the same slot (same delta, same stored
    patch) give bit-identical rows."""
    wl = make_workload("C4", num_layers=1, tokens=32)
    dw = run_dw(wl)
    seen = {}
    for ch in wl.chunks:
        key = (ch.canon_id, ch.dst_row0)
        rows = dw.out_rows(ch, 0, 0)
        if key in seen:
            assert np.array_equal(rows, seen[key])
        seen[key] = rows


def test_relocation_composes_on_gpu():
    """R(d2) R(d1) in place vs R(d1 + d2) at once (preprint §1: R(d)R(p) = R(p+d)).
    The two-step result carries one extra bf16 rounding of the intermediate pair, which
    the second rotation mixes across the pair, so the bound is in units of the pair's
    norm: |a - b| <= 2 ulp_bf16(|(x_p, x_q)|) per element."""
    from position_free_kv_amd import abi
    from oracle.tolerance import bf16_value, ulp_bf16
    lay = abi.make_layout(abi.GQA, abi.BF16, 2, num_kv_heads=2, head_dim=128, rope_base=1e6, page_size=16)
    x = torch.randn(2, 4, 16, 256, device="cuda").to(torch.bfloat16).view(torch.int16)
    a, b = x.clone(), x.clone()
    ws = torch.empty(abi.workspace_bytes(1, 8), dtype=torch.uint8, device="cuda")
    pa, pb = abi.make_pool(a, None, 4), abi.make_pool(b, None, 4)
    abi.relocate(lay, pa, None, 0, 64, 3000, ws)
    abi.relocate(lay, pa, None, 0, 64, -1234, ws)
    abi.relocate(lay, pb, None, 0, 64, 3000 - 1234, ws)
    torch.cuda.synchronize()
    va = bf16_value(a.cpu().numpy().view(np.uint16)).reshape(-1, 2, 2, 64)   # [row][head][half][pair]
    vb = bf16_value(b.cpu().numpy().view(np.uint16)).reshape(-1, 2, 2, 64)
    vx = bf16_value(x.cpu().numpy().view(np.uint16)).reshape(-1, 2, 2, 64)
    norm = np.sqrt(vx[:, :, 0] ** 2 + vx[:, :, 1] ** 2)[:, :, None, :]
    assert np.all(np.abs(va - vb) <= 2 * ulp_bf16(norm))


# ---------------------------------------------------------------- limits
@pytest.mark.parametrize("case", ["rank256_gqa128", "head512", "head512_gptj", "mla_rope512", "mla_rank256",
                                  "four_factors_rank256"])
def test_maximum_sizes(case):
    """The ABI's upper limits: rank KAMERA_MAX_RANK (256), 512-wide heads and rope bands,
    four factors of the largest rank on one tensor (all past the MFMA variants' register
    budget, so the generic kernel runs them)."""
    say(f"[limits] {case}")
    if case.startswith("mla"):
        rope = 512 if case == "mla_rope512" else 64
        lat = 64 if case == "mla_rope512" else 512
        rank = 256 if case == "mla_rank256" else 16
        lay = LayoutSpec(MLA, BF16, 1, latent_dim=lat, rope_dim=rope, rope_base=1e4)
        F = lat + rope
        chunks = [ChunkSpec(index=0, num_tokens=40, delta=77777, flags=PATCH, canon_id=0,
                            factors=[factor(0, 0, 0, 0, F, rank), factor(0, 1, 0, lat, rope, rank)], dst_buffer=0)]
    elif case == "four_factors_rank256":
        lay = LayoutSpec(GQA, BF16, 1, num_kv_heads=2, head_dim=128, rope_base=1e6)
        facs = [factor(0, s, 0, 64 * s, 128, 256, sigma0=0.1) for s in range(3)] + [factor(0, 3, 1, 0, 256, 256)]
        chunks = [ChunkSpec(index=0, num_tokens=300, delta=-5000, flags=PATCH, canon_id=0, factors=facs,
                            dst_buffer=0)]
    else:
        hd = 512 if case.startswith("head512") else 128
        rank = 256 if case == "rank256_gqa128" else 24
        lay = LayoutSpec(GQA, BF16, 1, num_kv_heads=2, head_dim=hd, rope_base=1e6,
                         pairing=GPTJ if "gptj" in case else NEOX)
        chunks = gqa_chunks(2, [300, 33], [123456, -99], 2, hd, rank)
    assert_parity(run_dw(custom_workload(lay, chunks)))


def test_many_chunks_in_one_batch():
    """300 chunks of 0 to 40 tokens in one launch (the task decode searches a long chunk
    list; empty chunks own no tasks), half of them paged, every third one re-anchored token
    by token (the cos/sin table kernel searches the same list)."""
    say("[many chunks]")
    P = 16
    lay = LayoutSpec(GQA, BF16, 2, num_kv_heads=2, head_dim=128, rope_base=1e6, page_size=P,
                     mrope_section=(16, 24, 24))
    rng = np.random.default_rng(77)
    pages = rng.permutation(2000).astype(np.int32)
    chunks, cur = [], 0
    for i in range(300):
        T = int(rng.integers(0, 41))
        kw = dict(index=i, num_tokens=T, delta=int(rng.integers(-50000, 50000)), flags=PATCH, canon_id=i,
                  factors=[factor(i, 0, 0, 0, 256, 8), factor(i, 1, 1, 0, 256, 8)])
        if i % 2:
            n = -(-(3 + T) // P)
            kw.update(block_table=pages[cur:cur + n].copy(), slot0=3)
            cur += n
        else:
            kw.update(dst_buffer=i // 2)
        if i % 3 == 0:
            kw.update(positions=grid_positions(T, int(rng.integers(0, 9000)), frame_tokens=16, grid_w=4),
                      flags=PATCH | POSITIONS)
        chunks.append(ChunkSpec(**kw))
    wl = custom_workload(lay, chunks, num_pages=2000)
    dw = run_dw(wl)
    assert_parity(dw)
    assert pool_untouched_ok(dw)


@pytest.mark.parametrize("positions", [False, True])
def test_plan_launch_in_a_captured_graph(positions):
    """kamera_plan_launch recorded in a HIP graph (the plan was uploaded eagerly; a launch
    enqueues only the main kernel): every replay, with the outputs cleared eagerly in between,
    reproduces the eager result bit for bit."""
    from position_free_kv_amd import abi
    from workloads.device import DeviceWorkload
    say(f"[graph] positions={positions}")
    wl = make_workload("C2", num_layers=2, num_chunks=3, tokens=150, positions=positions)
    dw = DeviceWorkload(wl)
    dw.run()
    torch.cuda.synchronize()
    eager = [t.clone() for buf in dw.dense for t in buf]
    assert_parity(dw)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan = dw.plan()          # uploads (and builds the cos/sin tables) on the side stream, eagerly
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        abi.plan_launch(plan)     # captured on torch's capture stream
    for rep in range(3):
        for buf in dw.dense:
            for t in buf:
                t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t for buf in dw.dense for t in buf]
        assert all(torch.equal(a, b) for a, b in zip(eager, got)), f"replay {rep}"


@pytest.mark.parametrize("positions", [False, True])
def test_one_shot_small_batch_in_a_captured_graph(positions):
    """A one-shot kamera_rehydrate_batched call on a small dense batch passes the packed
    batch as the kernels' argument and makes no other HIP call, so the call itself can be
    recorded in a HIP graph. Every replay, with the outputs and the whole workspace cleared
    eagerly in between, reproduces the eager result bit for bit (with per-token offsets the
    replay recomputes the cos/sin tables into the workspace before the main kernel)."""
    from workloads.device import DeviceWorkload
    say(f"[graph, one-shot] positions={positions}")
    wl = make_workload("C2", num_layers=2, num_chunks=3, tokens=150, positions=positions)
    dw = DeviceWorkload(wl)
    dw.run()
    torch.cuda.synchronize()
    eager = [t.clone() for buf in dw.dense for t in buf]
    assert_parity(dw)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dw.run(stream=torch.cuda.current_stream())   # the capture stream
    for rep in range(3):
        for buf in dw.dense:
            for t in buf:
                t.zero_()
        dw.workspace.fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t for buf in dw.dense for t in buf]
        assert all(torch.equal(a, b) for a, b in zip(eager, got)), f"replay {rep}"


@pytest.mark.parametrize("layout_kind,n", [("gqa128", 16), ("gqa128", 17), ("mla", 16), ("f32", 16), ("f32", 17),
                                            ("three_factors", 2), ("positions", 16), ("positions", 17)])
def test_kernel_argument_route_boundary(layout_kind, n):
    """One-shot calls on dense batches of up to 16 chunks with at most 2 factors each pass
    the packed batch as the kernel's argument; 17 chunks, or a chunk with 3 factors, take the
    workspace. Both routes match the oracle, and a plan (always the workspace route)
    relaunched on the same batch reproduces the call's bytes. With per-token offsets the
    argument route still computes the cos/sin tables into the workspace, but not the
    packed batch at its start."""
    from position_free_kv_amd import abi
    from workloads.device import DeviceWorkload
    say(f"[kernel-argument route] {layout_kind} chunks={n}")
    T = [1, 16, 17, 33, 64, 90, 129, 5, 48, 70, 31, 15, 2, 100, 47, 80, 19][:n]
    deltas = [int(d) for d in np.random.default_rng(n).integers(-40000, 40000, size=n)]
    by_argument = n <= 16 and layout_kind != "three_factors"
    if layout_kind == "mla":
        lay = LayoutSpec(MLA, BF16, 2, latent_dim=512, rope_dim=64)
        chunks = [ChunkSpec(index=i, num_tokens=T[i], delta=deltas[i], flags=PATCH, canon_id=i,
                            factors=[factor(i, 0, 0, 0, 576, 32), factor(i, 1, 0, 512, 64, 16)], dst_buffer=i)
                  for i in range(n)]
    elif layout_kind == "three_factors":
        lay = LayoutSpec(GQA, BF16, 2, num_kv_heads=2, head_dim=128, rope_base=1e6)
        chunks = [ChunkSpec(index=i, num_tokens=T[i] + 20, delta=deltas[i], flags=PATCH, canon_id=i,
                            factors=[factor(i, 0, 0, 0, 256, 16), factor(i, 1, 1, 0, 256, 16),
                                     factor(i, 2, 0, 128, 128, 8)], dst_buffer=i)
                  for i in range(n)]
    elif layout_kind == "positions":
        lay = LayoutSpec(GQA, BF16, 2, num_kv_heads=2, head_dim=128, rope_base=1e6, mrope_section=(16, 24, 24))
        chunks = [dataclasses.replace(c, positions=grid_positions(c.num_tokens, 300 * c.index - 2000),
                                      flags=c.flags | POSITIONS) if c.index % 2 == 0 else c
                  for c in gqa_chunks(n, T, deltas, 2, 128, 16)]
    else:
        dt = F32 if layout_kind == "f32" else BF16
        lay = LayoutSpec(GQA, dt, 2, num_kv_heads=2, head_dim=128 if dt == BF16 else 64, rope_base=1e6)
        chunks = gqa_chunks(n, T, deltas, 2, lay.head_dim, 16)
    dw = DeviceWorkload(custom_workload(lay, chunks))
    dw.workspace.fill_(0xA5)
    dw.run()
    torch.cuda.synchronize()
    # the argument route writes no packed batch (its header would sit at the workspace's start)
    ws = dw.workspace if layout_kind != "positions" else dw.workspace[:256]
    assert bool((ws == 0xA5).all()) == by_argument
    assert_parity(dw)
    first = [t.clone() for buf in dw.dense for t in buf]
    for buf in dw.dense:
        for t in buf:
            t.zero_()
    abi.plan_launch(dw.plan())
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(first, [t for buf in dw.dense for t in buf]))
