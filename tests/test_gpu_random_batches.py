"""Randomised parity: small batches drawn from a seeded generator, spanning the layout
families (GQA with 64- and 128-wide heads, MLA, fp32), both pairings, 0 to 4 factors per
chunk with assorted ranks, column ranges and first layers, chunk counts on both sides of the
kernel-argument limit (16), empty chunks, deltas up to +-(2^31 - 1), per-token (t, h, w)
offsets on some chunks (QV-PIC Eq. 2, under an M-RoPE section split), and mixes of dense
destinations, paged destinations (pages of 1 to 64 tokens) and in-place survivors. Every batch is compared with the
oracle element by element (Kamera preprint Eq. 1; same bar as the other parity tests), and
the pool slots no chunk owns must keep their sentinel.
"""
import numpy as np
import pytest
import torch

from tests.gpu_util import check_all, custom_workload, factor, pool_untouched_ok, say
from workloads.configs import (BF16, F32, GPTJ, GQA, IN_PLACE, MLA, NEOX, PATCH, POSITIONS, ChunkSpec, LayoutSpec,
                               mrope_sections)

pytestmark = pytest.mark.gpu

N_BATCHES = 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from position_free_kv_amd import abi
    abi.lib()   # fails loudly when the HIP library is missing
    yield


def draw_batch(seed: int, kind=None, reanchor_ok: bool = True):
    """A seeded random batch; `kind` forces the layout ("gqa128", "gqa64", "mla", "f32") and
    reanchor_ok=False keeps every chunk on a chunk-wide delta."""
    rng = np.random.default_rng([20261202, seed])
    drawn = str(rng.choice(["gqa128", "gqa64", "mla", "f32"]))
    kind = kind or drawn
    pairing = GPTJ if rng.random() < 0.3 else NEOX
    L = int(rng.integers(1, 4))
    # pool page size from a stream of its own (the main stream's draws are those of 16-token pages)
    P = int(np.random.default_rng([20261202, seed, 1]).choice([16, 16, 16, 1, 3, 8, 24, 64]))
    reanchor = rng.random() < 0.35 and reanchor_ok   # some chunks turn token by token under an M-RoPE split
    if kind == "mla":
        lay = LayoutSpec(MLA, BF16, L, latent_dim=512, rope_dim=64, pairing=pairing, page_size=P,
                         mrope_section=(8, 12, 12) if reanchor else (0, 0, 0))
        tensors = [0]
    else:
        hd = 128 if kind == "gqa128" else 64
        lay = LayoutSpec(GQA, F32 if kind == "f32" else BF16, L, num_kv_heads=int(rng.integers(1, 5)), head_dim=hd,
                         rope_base=float(rng.choice([1e4, 1e6])), pairing=pairing, page_size=P,
                         mrope_section=mrope_sections(hd) if reanchor else (0, 0, 0))
        tensors = [0, 1]
    F = lay.row_width
    n = int(rng.choice([1, 3, 8, 16, 17, 24]))
    paged_share = float(rng.choice([0.0, 0.0, 0.0, 0.5, 1.0]))
    max_factors = int(rng.choice([2, 2, 4]))   # at most 2 keeps a dense batch on the kernel-argument route
    lengths = [int(t) for t in rng.integers(0, 101, size=n)]
    lengths[int(rng.integers(0, n))] = int(rng.integers(1, 101))   # at least one chunk with tokens
    slot0s = [int(rng.integers(0, P)) for _ in range(n)]
    paged = [rng.random() < paged_share for _ in range(n)]
    num_pages = sum(-(-(s + t) // P) for s, t, pg in zip(slot0s, lengths, paged) if pg) + 8
    pages = rng.permutation(num_pages).astype(np.int32)
    chunks, cursor, buf = [], 0, 0
    for i in range(n):
        T = lengths[i]
        big = rng.random() < 0.2
        delta = int(rng.integers(-(2 ** 31 - 1), 2 ** 31)) if big else int(rng.integers(-70000, 70001))
        facs = []
        for slot in range(int(rng.integers(0, max_factors + 1))):
            w = int(rng.integers(1, F + 1))
            c0 = int(rng.integers(0, F - w + 1))
            rank = int(rng.choice([1, 5, 8, 16, 32, 40, 64]))
            facs.append(factor(i, slot, int(rng.choice(tensors)), c0, w, rank,
                               layer0=int(rng.integers(0, L)) if rng.random() < 0.3 else 0))
        flags = PATCH if (facs and rng.random() < 0.85) else 0
        kw = dict(index=i, num_tokens=T, delta=delta, flags=flags, canon_id=i, factors=facs)
        if reanchor and rng.random() < 0.5:
            base = int(rng.integers(-70000, 70001))
            pos = base + rng.integers(0, 4096, size=(T, 3))
            if rng.random() < 0.2:
                pos[: T // 2] = rng.integers(-(2 ** 31 - 1), 2 ** 31, size=(T // 2, 3))
            kw.update(positions=np.ascontiguousarray(pos, dtype=np.int32), flags=flags | POSITIONS)
        if paged[i]:
            npg = -(-(slot0s[i] + T) // P)
            kw.update(block_table=pages[cursor:cursor + npg].copy(), slot0=slot0s[i])
            cursor += npg
            if rng.random() < 0.3:   # a survivor: the rows already in its pages turn in place
                kw.update(flags=kw["flags"] | IN_PLACE, role="survivor")
        else:
            kw.update(dst_buffer=buf)
            buf += 1
        chunks.append(ChunkSpec(**kw))
    npos = sum(c.positions is not None for c in chunks)
    desc = (f"{kind} {'gptj' if pairing == GPTJ else 'neox'} L={L} chunks={n} paged={sum(paged)} page_size={P} "
            f"re-anchored={npos}")
    return custom_workload(lay, chunks, num_pages=num_pages if any(paged) else 0), desc


@pytest.mark.parametrize("seed", range(N_BATCHES))
def test_random_batch(seed):
    from workloads.device import DeviceWorkload
    wl, desc = draw_batch(seed)
    say(f"[random batch {seed}] {desc}")
    dw = DeviceWorkload(wl)
    dw.run()
    torch.cuda.synchronize()
    tot = check_all(dw)
    say(f"  compared {tot['n']} elements: fail={tot['fail']} p2_only={tot['p2_only']} exact={tot['exact']}")
    assert tot["fail"] == 0, tot["bad"][:3]
    assert pool_untouched_ok(dw)


@pytest.mark.parametrize("seed", range(1000, 1000 + N_BATCHES // 2))
def test_random_batch_noalloc_and_valu(seed):
    """Batches from the same generator through the other routes: the allocation-free entry
    point (its scratch holds the packed batch and tables), and, where the layout allows it
    (bf16 heads of 128, no per-token offsets, at most two k-steps), the patch on the VALU
    (every odd seed draws such a layout)."""
    from position_free_kv_amd import abi
    from workloads.device import DeviceWorkload
    wl, desc = draw_batch(seed, **({"kind": "gqa128", "reanchor_ok": False} if seed % 2 else {}))
    dw = DeviceWorkload(wl)
    valu = wl.layout.family == GQA and wl.layout.dtype == BF16 and wl.layout.head_dim == 128 \
        and not any(c.positions is not None for c in wl.chunks)
    if valu:
        dw.layout.patch_unit = abi.PATCH_UNIT_VALU
    say(f"[random batch {seed}, no-alloc{', VALU' if valu else ''}] {desc}")
    assert abi.batch_workspace_bytes(dw.layout, dw.descs) <= abi.NOALLOC_SCRATCH_BYTES
    try:
        abi.rehydrate_batched_noalloc(dw.layout, dw.descs, dw.pool_desc)
    except abi.KameraError as e:   # more k-steps than the VALU form holds: the matrix cores instead
        assert valu and e.name == "KAMERA_E_UNSUPPORTED", e
        say("  VALU form not built for this batch's k-steps; matrix cores")
        dw.layout.patch_unit = abi.PATCH_UNIT_AUTO
        abi.rehydrate_batched_noalloc(dw.layout, dw.descs, dw.pool_desc)
    torch.cuda.synchronize()
    tot = check_all(dw)
    say(f"  compared {tot['n']} elements: fail={tot['fail']} p2_only={tot['p2_only']} exact={tot['exact']}")
    assert tot["fail"] == 0, tot["bad"][:3]
    assert pool_untouched_ok(dw)
