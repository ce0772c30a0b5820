"""GPU parity of per-token re-anchoring: every token of a chunk rotated by its own
(t, h, w) position offsets, pairs split into blocked M-RoPE sections (QV-PIC Eq. 2:
keys stored unrotated and placed at their request positions by the model's M-RoPE),
followed by the usual patch (Kamera preprint Eq. 1).

Same bar as the other parity tests (bf16: one step of the once-rounded fp64 result,
or the fp32 accumulation bound; fp32: P3). A uniform offset on all three components
is the 1-D rotation R(delta) (Kamera preprint §4), and there the kernel's output is
bit-identical to the chunk-wide delta path.
"""
import dataclasses
import zlib

import numpy as np
import pytest
import torch

from tests.gpu_util import check_all, custom_workload, factor, gqa_chunks, pool_untouched_ok, say
from workloads import make_workload
from workloads.configs import (BF16, F32, GPTJ, GQA, IN_PLACE, MLA, NEOX, PATCH, POSITIONS, ChunkSpec, LayoutSpec,
                               grid_positions, mrope_sections)

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


def assert_parity(dw):
    tot = check_all(dw)
    say(f"  compared {tot['n']} elements: fail={tot['fail']} p2_only={tot['p2_only']} exact={tot['exact']}")
    assert tot["fail"] == 0, tot["bad"][:3]
    return tot


def with_positions(ch: ChunkSpec, pos: np.ndarray) -> ChunkSpec:
    return dataclasses.replace(ch, positions=np.ascontiguousarray(pos, dtype=np.int32),
                               flags=ch.flags | POSITIONS)


@pytest.mark.parametrize("name,kw", [
    ("C1", {}),                                                  # fp32: generic kernel, 2 x 64 heads
    ("C2", dict(num_layers=2, num_chunks=3, tokens=200)),        # 4 x 128, (16, 24, 24) sections
    ("C3", dict(num_layers=2, num_chunks=2, tokens=150)),        # MLA: 64-wide rope band, (8, 12, 12)
    ("C5", dict(num_layers=2, num_chunks=8, max_tokens=300)),    # paged; survivors keep their delta
])
def test_positions_configs_small(name, kw):
    say(f"[positions] {name} {kw}")
    wl = make_workload(name, positions=True, **kw)
    assert any(c.positions is not None for c in wl.chunks)
    dw = run_dw(wl)
    assert_parity(dw)
    assert pool_untouched_ok(dw)


@pytest.mark.parametrize("variant", ["gqa128", "gqa64", "gptj128", "mla", "gqa_f32"])
def test_uniform_positions_are_the_delta_path_bitwise(variant):
    """(delta, delta, delta) for every token under any section split gives exactly the
    bytes of the chunk-wide delta path: same fp64 angles, same fp32 arithmetic."""
    say(f"[positions=delta] {variant}")
    if variant == "mla":
        lay = LayoutSpec(MLA, BF16, 2, latent_dim=512, rope_dim=64, mrope_section=(8, 12, 12))
        base = [ChunkSpec(index=i, num_tokens=70 + 30 * i, delta=d, flags=PATCH, canon_id=i,
                          factors=[factor(i, 0, 0, 0, 576, 32), factor(i, 1, 0, 512, 64, 32)], dst_buffer=i)
                for i, d in enumerate([40000, -77])]
    else:
        hd = 64 if variant == "gqa64" else 128
        dt = F32 if variant == "gqa_f32" else BF16
        lay = LayoutSpec(GQA, dt, 2, num_kv_heads=2, head_dim=hd, rope_base=1e6,
                         pairing=GPTJ if "gptj" in variant else NEOX, mrope_section=mrope_sections(hd))
        base = gqa_chunks(2, [90, 37], [31000, -4097], 2, hd, 32)
    plain = run_dw(custom_workload(lay, base))
    uni = run_dw(custom_workload(lay, [with_positions(c, np.full((c.num_tokens, 3), c.delta)) for c in base]))
    for ch in base:
        for layer in range(2):
            for t in ([0] if lay.family == MLA else [0, 1]):
                assert np.array_equal(plain.out_rows(ch, layer, t), uni.out_rows(ch, layer, t)), (ch.index, layer, t)
    assert_parity(uni)


@pytest.mark.parametrize("variant", ["gqa64", "gptj128", "gptj64", "rank64", "rank96_generic", "rank8",
                                     "mla_gptj", "one_section", "ragged"])
def test_positions_variants(variant):
    """Kernel variants: 64-wide heads, GPT-J pairs, two k-steps on 128-wide heads (cos/sin
    loaded per tile, not prefetched), three k-steps (generic kernel), a split with only the
    w section, ragged chunk ends."""
    say(f"[positions variant] {variant}")
    rng = np.random.default_rng(zlib.crc32(variant.encode()))
    if variant == "mla_gptj":
        lay = LayoutSpec(MLA, BF16, 2, latent_dim=448, rope_dim=64, pairing=GPTJ, mrope_section=(8, 12, 12))
        chunks = [ChunkSpec(index=i, num_tokens=45 + 20 * i, delta=0, flags=PATCH, canon_id=i,
                            factors=[factor(i, 0, 0, 0, 512, 16), factor(i, 1, 0, 448, 64, 8)], dst_buffer=i)
                  for i in range(2)]
    else:
        hd = 64 if variant in ("gqa64", "gptj64") else 128
        rank = {"rank64": 64, "rank96_generic": 96, "rank8": 8}.get(variant, 32)
        sec = (0, 0, hd // 2) if variant == "one_section" else mrope_sections(hd)
        lay = LayoutSpec(GQA, BF16, 2, num_kv_heads=3, head_dim=hd, rope_base=1e6,
                         pairing=GPTJ if "gptj" in variant else NEOX, mrope_section=sec)
        T = [1, 17, 129] if variant == "ragged" else [50, 33]
        chunks = gqa_chunks(len(T), T, 0, 3, hd, rank)
    out = []
    for c in chunks:
        start = int(rng.integers(-70000, 70000))
        out.append(with_positions(c, grid_positions(c.num_tokens, start, frame_tokens=16, grid_w=4)))
    assert_parity(run_dw(custom_workload(lay, out)))


def test_positions_extreme_offsets():
    """Offsets near +-(2^31 - 1) and arbitrary per-token values on every component."""
    say("[positions extreme]")
    lay = LayoutSpec(GQA, BF16, 1, num_kv_heads=2, head_dim=128, rope_base=1e6, mrope_section=(16, 24, 24))
    rng = np.random.default_rng(11)
    ch = gqa_chunks(1, 96, 0, 2, 128, 32)[0]
    pos = rng.integers(-(2 ** 31 - 1), 2 ** 31 - 1, size=(96, 3), endpoint=True)
    pos[:8] = 2 ** 31 - 1
    pos[8:16] = -(2 ** 31 - 1)
    pos[16:24] = 0
    assert_parity(run_dw(custom_workload(lay, [with_positions(ch, pos)])))


def test_positions_mixed_batch_paged_in_place():
    """A batch mixing re-anchored chunks (dense and paged, one in place) with chunk-wide
    delta chunks and a survivor: each chunk finds its own cos/sin table."""
    say("[positions mixed batch]")
    P = 16
    lay = LayoutSpec(GQA, BF16, 3, num_kv_heads=2, head_dim=128, rope_base=1e6, page_size=P,
                     mrope_section=(16, 24, 24))
    pages = np.random.default_rng(9).permutation(64).astype(np.int32)
    facs = lambda i: [factor(i, 0, 0, 0, 256, 32), factor(i, 1, 1, 0, 256, 32)]
    chunks = [ChunkSpec(index=0, num_tokens=150, delta=900, flags=PATCH, canon_id=0, factors=facs(0), dst_buffer=0),
              ChunkSpec(index=1, num_tokens=0, delta=5, flags=PATCH, canon_id=1, factors=facs(1), dst_buffer=1),
              ChunkSpec(index=2, num_tokens=70, delta=0, flags=PATCH, canon_id=2, factors=facs(2),
                        block_table=pages[0:5].copy(), slot0=3),
              ChunkSpec(index=3, num_tokens=200, delta=-1234, flags=IN_PLACE, canon_id=3,
                        block_table=pages[5:18].copy(), slot0=0, role="survivor"),
              ChunkSpec(index=4, num_tokens=33, delta=0, flags=0, canon_id=4, dst_buffer=2),
              ChunkSpec(index=5, num_tokens=61, delta=0, flags=IN_PLACE | PATCH, canon_id=5, factors=facs(5)[:1],
                        block_table=pages[18:23].copy(), slot0=7, role="survivor")]
    chunks[0] = with_positions(chunks[0], grid_positions(150, 512))
    chunks[2] = with_positions(chunks[2], grid_positions(70, -300, frame_tokens=16, grid_w=4))
    chunks[4] = with_positions(chunks[4], grid_positions(33, 7))
    chunks[5] = with_positions(chunks[5], grid_positions(61, -4096))
    wl = custom_workload(lay, chunks, dense_rows=[150, 1, 33], num_pages=64)
    dw = run_dw(wl)
    assert_parity(dw)
    assert pool_untouched_ok(dw)


def test_positions_plan_reuse_and_determinism():
    """The cos/sin tables are built when the batch is uploaded; relaunching the plan
    reproduces the first output bit for bit."""
    from position_free_kv_amd import abi
    from workloads.device import DeviceWorkload
    wl = make_workload("C2", num_layers=2, num_chunks=2, tokens=130, positions=True)
    dw = DeviceWorkload(wl)
    dw.run()
    torch.cuda.synchronize()
    first = [t.clone() for buf in dw.dense for t in buf]
    plan = dw.plan()
    for buf in dw.dense:
        for t in buf:
            t.zero_()
    for _ in range(3):
        abi.plan_launch(plan)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(first, [t for buf in dw.dense for t in buf]))


def test_offsets_without_the_flag_are_ignored():
    """A chunk that hands over per-token offsets but not KAMERA_POSITIONS turns by its delta
    (the offsets are ignored), on both call routes."""
    say("[positions without the flag]")
    for n in (2, 20):   # 2 chunks: kernel-argument route; 20: workspace route
        lay = LayoutSpec(GQA, BF16, 2, num_kv_heads=2, head_dim=128, rope_base=1e6, mrope_section=(16, 24, 24))
        chunks = [dataclasses.replace(c, positions=grid_positions(c.num_tokens, 5000 + 7 * c.index))
                  for c in gqa_chunks(n, 40, [311 * (i + 1) for i in range(n)], 2, 128, 16)]
        assert all(c.positions is not None and not c.flags & POSITIONS for c in chunks)
        assert_parity(run_dw(custom_workload(lay, chunks)))
