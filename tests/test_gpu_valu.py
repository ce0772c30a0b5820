"""GPU parity of the VALU form of the patch (KAMERA_PATCH_UNIT_VALU: v_dot2c_f32_bf16 with row
broadcasts of the V factor) against the fp64 oracle, to the same bar as the matrix-core form
(Kamera preprint §6: one bf16 step of the once-rounded result, or the fp32 accumulation bound).

The two forms add the patch's products in a different order, so they need not agree bit for
bit; each must meet the bar on its own, and both must leave every byte they do not own alone.
"""
import numpy as np
import pytest
import torch

from tests.gpu_util import check_all, custom_workload, factor, gqa_chunks, pool_untouched_ok, say
from workloads import make_workload
from workloads.configs import BF16, GPTJ, GQA, IN_PLACE, PATCH, ChunkSpec, LayoutSpec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from position_free_kv_amd import abi
    abi.lib()   # fails loudly when the HIP library is missing
    yield


def run_unit(wl, unit):
    from position_free_kv_amd import abi
    from workloads.device import DeviceWorkload
    dw = DeviceWorkload(wl)
    dw.layout.patch_unit = unit
    plan = dw.plan()
    assert plan.kernel == 1 and plan.variant >= 16 if unit == abi.PATCH_UNIT_VALU else plan.variant < 16
    dw.run()
    torch.cuda.synchronize()
    return dw


def assert_parity(dw):
    tot = check_all(dw)
    say(f"  compared {tot['n']} elements: fail={tot['fail']} p2_only={tot['p2_only']} exact={tot['exact']}")
    assert tot["fail"] == 0, tot["bad"][:3]
    return tot


@pytest.mark.parametrize("rank", [1, 7, 8, 16, 31, 32, 33, 48, 64])
def test_valu_ranks(rank):
    from position_free_kv_amd import abi
    say(f"[valu rank] m={rank}")
    lay = LayoutSpec(GQA, BF16, 2, num_kv_heads=2, head_dim=128, rope_base=1e4)
    wl = custom_workload(lay, gqa_chunks(2, [70, 129], [1000, -31], 2, 128, rank))
    assert_parity(run_unit(wl, abi.PATCH_UNIT_VALU))


@pytest.mark.parametrize("name,kw", [("C2", dict(num_layers=2, num_chunks=3, tokens=200)),
                                     ("C4", dict(num_layers=1, tokens=48)),
                                     ("C5", dict(num_layers=2, num_chunks=8, max_tokens=300))])
def test_valu_workloads_both_units(name, kw):
    """The workloads' own shapes through both units: dense, reorder (32 heads) and the paged
    deque with in-place survivors."""
    from position_free_kv_amd import abi
    for unit in (abi.PATCH_UNIT_VALU, abi.PATCH_UNIT_MFMA):
        say(f"[valu workload] {name} unit={unit}")
        dw = run_unit(make_workload(name, **kw), unit)
        assert_parity(dw)
        assert pool_untouched_ok(dw)


def test_valu_factor_shapes_and_pairing():
    """Per-head factors and an unaligned column range with an odd rank (element loads of U and
    V), GPT-J pairing, a rotation-only chunk and an in-place survivor with a patch."""
    from position_free_kv_amd import abi
    say("[valu factors]")
    lay = LayoutSpec(GQA, BF16, 2, num_kv_heads=4, head_dim=128, rope_base=1e6, pairing=GPTJ)
    facs = [factor(0, h, 0, 128 * h, 128, 8) for h in range(2)] + [factor(0, 3, 1, 40, 100, 23)]
    chunks = [ChunkSpec(index=0, num_tokens=90, delta=777, flags=PATCH, canon_id=0, factors=facs, dst_buffer=0),
              ChunkSpec(index=1, num_tokens=33, delta=-4096, flags=0, canon_id=1, dst_buffer=1)]
    assert_parity(run_unit(custom_workload(lay, chunks), abi.PATCH_UNIT_VALU))
    P = 16
    lay = LayoutSpec(GQA, BF16, 2, num_kv_heads=2, head_dim=128, rope_base=1e6, page_size=P)
    pages = np.random.default_rng(3).permutation(12).astype(np.int32)
    chunks = [ChunkSpec(index=0, num_tokens=40, delta=-999, flags=IN_PLACE | PATCH, canon_id=0,
                        factors=[factor(0, 0, 0, 0, 256, 16), factor(0, 1, 1, 0, 256, 16)],
                        block_table=pages[:3].copy(), slot0=0, role="survivor"),
              ChunkSpec(index=1, num_tokens=50, delta=640, flags=PATCH, canon_id=1,
                        factors=[factor(1, 0, 0, 0, 256, 32), factor(1, 1, 1, 0, 256, 32)],
                        block_table=pages[3:7].copy(), slot0=0)]
    dw = run_unit(custom_workload(lay, chunks, dense_rows=[], num_pages=12), abi.PATCH_UNIT_VALU)
    assert_parity(dw)
    assert pool_untouched_ok(dw)
