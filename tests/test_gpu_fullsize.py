"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times
(one kamera_rehydrate_batched call over every chunk and layer).

The oracle recomputes sampled rows one block at a time (first, last and random
rows of sampled (chunk, layer, tensor) blocks). Properties that hold at any size
are checked on the device over everything: untouched pool slots keep their
sentinel, survivors' V pages and MLA c_KV columns are byte-identical, and a
second run reproduces the first bit for bit.
"""
import numpy as np
import pytest
import torch

from tests.gpu_util import compare, pool_untouched_ok, say, touched_tensors
from workloads import make_workload

pytestmark = pytest.mark.gpu


def _sampled_parity(dw, n_blocks: int, rows: int, seed: int):
    rng = np.random.default_rng(seed)
    wl = dw.wl
    todo = []
    for ch in wl.chunks:
        for t in touched_tensors(wl, ch):
            todo.append((ch, t))
    pick = rng.choice(len(todo), size=min(n_blocks, len(todo)), replace=False)
    tot = {"n": 0, "fail": 0, "p2_only": 0}
    for i in pick:
        ch, t = todo[i]
        layer = int(rng.integers(0, dw.L))
        rr = np.unique(np.concatenate([[0, ch.num_tokens - 1], rng.choice(ch.num_tokens, rows, replace=False)]))
        r = compare(dw, ch, layer, t, rr)
        for k in tot:
            tot[k] += r[k]
        assert r["fail"] == 0, (r["where"], r.get("examples"))
    say(f"  sampled {tot['n']} elements over {len(pick)} blocks: fail={tot['fail']} p2_only={tot['p2_only']}")


def _stage(name, **kw):
    from workloads.device import DeviceWorkload
    say(f"[fullsize] staging {name} {kw}")
    wl = make_workload(name, **kw)
    dw = DeviceWorkload(wl)
    say(f"[fullsize] staged {name}: {wl.total_tokens} tokens, {dw.algorithmic_bytes() / 1e9:.2f} GB moved per call")
    return dw


def _run_twice_identical(dw, snapshot):
    first = [t.clone() for t in snapshot()]
    dw.run()
    torch.cuda.synchronize()
    return all(torch.equal(a, b) for a, b in zip(first, snapshot()))


@pytest.mark.parametrize("name,blocks,rows", [("C2", 24, 40), ("C3", 24, 40), ("C4", 10, 24)])
def test_fullsize_dense(name, blocks, rows):
    """Sampled parity at full size, a second call byte-identical, and the same batch through the
    allocation-free entry point byte-identical too (its scratch holds the whole packed batch)."""
    from position_free_kv_amd import abi
    dw = _stage(name)
    dw.run()
    torch.cuda.synchronize()
    _sampled_parity(dw, blocks, rows, seed=int(name[1:]))
    outs = lambda: [t for buf in dw.dense for t in buf]
    assert _run_twice_identical(dw, outs)
    first = [t.clone() for t in outs()]
    for t in outs():
        t.zero_()
    abi.rehydrate_batched_noalloc(dw.layout, dw.descs, dw.pool_desc)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(first, outs()))
    del dw, first
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["C2", "C3"])
def test_fullsize_positions(name):
    """Per-token (t, h, w) re-anchoring of every chunk at full size (three-section M-RoPE ids
    of 64-token frames at the chunk's start)."""
    dw = _stage(name, positions=True)
    dw.run()
    torch.cuda.synchronize()
    _sampled_parity(dw, 16, 32, seed=100 + int(name[1:]))
    assert _run_twice_identical(dw, lambda: [t for buf in dw.dense for t in buf])
    del dw
    torch.cuda.empty_cache()


def test_fullsize_mla_patch_off_bytes():
    """C3 with the patch off: c_KV columns of every output row equal the stored ones."""
    dw = _stage("C3", patch=False)
    dw.run()
    torch.cuda.synchronize()
    for ch in dw.wl.chunks:
        out = dw.dense[ch.dst_buffer][0]
        assert torch.equal(out[:, :, :512], dw.canon[ch.canon_id][0][:, :, :512])
    _sampled_parity(dw, 8, 24, seed=5)
    del dw
    torch.cuda.empty_cache()


def test_fullsize_deque_paged():
    """C5: survivors rotate in place, recalled chunks land in their pages, nothing else moves."""
    dw = _stage("C5")
    v_before = dw.pool[1].clone()
    k_before = dw.pool[0].clone()
    dw.run()
    torch.cuda.synchronize()
    _sampled_parity(dw, 24, 40, seed=55)
    assert pool_untouched_ok(dw)
    # survivors' V pages: byte-identical (only K rotates, preprint §5)
    P, F = dw.P, dw.F
    for ch in dw.wl.chunks:
        if ch.role == "survivor":
            rows = dw.slot_rows(ch)
            assert torch.equal(dw.pool[1].view(dw.L, -1, F)[:, rows], v_before.view(dw.L, -1, F)[:, rows])
    # undo the survivors' rotation (delta -> -delta) and rerun: same bytes as the first run
    del v_before
    after = dw.pool[0].clone()
    dw.pool[0].copy_(k_before)
    dw.run()
    torch.cuda.synchronize()
    assert torch.equal(dw.pool[0], after)
    del dw, k_before, after
    torch.cuda.empty_cache()


def test_fullsize_deque_positions():
    """C5 with its recalled chunks re-anchored token by token (survivors keep their delta):
    paged, in place and per-token tables in one full-size batch."""
    dw = _stage("C5", positions=True)
    dw.run()
    torch.cuda.synchronize()
    _sampled_parity(dw, 24, 32, seed=155)
    assert pool_untouched_ok(dw)
    del dw
    torch.cuda.empty_cache()
