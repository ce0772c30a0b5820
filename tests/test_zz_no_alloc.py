"""kamera_rehydrate_batched_noalloc against kamera_rehydrate_batched (same kernels, so the
outputs must be byte-identical), through the C ABI, two calls in a row, the second on a
smaller batch: a paged deque batch with in-place survivors (packed batch filled into the
library's scratch by kernel arguments), a small dense batch (the kernel-argument route), and
re-anchored batches whose per-token cos/sin tables live in the scratch."""
import numpy as np
import pytest
import torch

from tests.gpu_util import say
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from position_free_kv_amd import abi
    abi.lib()   # fails loudly when the HIP library is missing
    yield


def _outputs(dw):
    """Every destination byte of the workload: dense buffers and pool pages."""
    out = [t.clone() for bufs in dw.dense for t in bufs]
    if dw.pool is not None:
        out += [t.clone() for t in dw.pool]
    return out


def _restore(dw, snap):
    k = 0
    for bufs in dw.dense:
        for t in bufs:
            t.copy_(snap[k])
            k += 1
    if dw.pool is not None:
        for t in dw.pool:
            t.copy_(snap[k])
            k += 1


def _same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


CASES = [
    ("deque paged, in place", dict(name="C5", num_layers=3, num_chunks=12, max_tokens=300), [0, 1, 2, 3, 4]),
    ("dense small batch", dict(name="C2", num_layers=2, num_chunks=3, tokens=200), [1]),
    ("dense re-anchored", dict(name="C2", num_layers=2, num_chunks=2, tokens=160, positions=True), [0]),
    ("deque re-anchored", dict(name="C5", num_layers=2, num_chunks=8, max_tokens=260, positions=True), [2, 5, 6]),
    ("MLA rows", dict(name="C3", num_layers=2, num_chunks=18, tokens=64), [3, 4]),
]


@pytest.mark.parametrize("label,kw,subset", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_entry_point(label, kw, subset):
    from position_free_kv_amd import abi
    from workloads.device import DeviceWorkload
    kw = dict(kw)
    wl = make_workload(kw.pop("name"), **kw)
    dw = DeviceWorkload(wl, device="cuda:0")
    stream = torch.cuda.current_stream()
    fresh = _outputs(dw)
    for call, idx in enumerate([list(range(len(wl.chunks))), subset]):
        descs = [dw.descs[i] for i in idx]
        need = abi.batch_workspace_bytes(dw.layout, descs)
        say(f"[noalloc] {label}: call {call}, {len(descs)} chunks, {need} bytes of scratch")
        assert need <= abi.NOALLOC_SCRATCH_BYTES
        _restore(dw, fresh)
        abi.rehydrate_batched(dw.layout, descs, dw.pool_desc, dw.workspace, stream)
        torch.cuda.synchronize()
        want = _outputs(dw)
        assert not _same(want, fresh), "the batch changed nothing"
        _restore(dw, fresh)
        abi.rehydrate_batched_noalloc(dw.layout, descs, dw.pool_desc, stream)
        torch.cuda.synchronize()
        got = _outputs(dw)
        assert _same(got, want), f"{label}: call {call} differs from kamera_rehydrate_batched"
    say(f"[noalloc] {label}: both calls byte-identical")


@pytest.mark.parametrize("label,kw", [("deque paged", dict(name="C5", num_layers=2, num_chunks=10, max_tokens=280)),
                                      ("dense re-anchored", dict(name="C2", num_layers=2, num_chunks=3, tokens=150,
                                                                 positions=True))])
def test_noalloc_call_in_a_captured_graph(label, kw):
    """The callers the allocation-free entry point is for include code under graph capture: a
    call recorded in a HIP graph (the packed batch travels in its kernels' arguments) replays to
    the eager result bit for bit, three times, with the destinations restored and other eager
    work between the replays. The first call on the device, which looks up the scratch array's
    address, happens before the capture."""
    from position_free_kv_amd import abi
    from workloads.device import DeviceWorkload
    kw = dict(kw)
    wl = make_workload(kw.pop("name"), **kw)
    dw = DeviceWorkload(wl, device="cuda:0")
    fresh = _outputs(dw)
    say(f"[noalloc graph] {label}")
    abi.rehydrate_batched_noalloc(dw.layout, dw.descs, dw.pool_desc)
    torch.cuda.synchronize()
    eager = _outputs(dw)
    _restore(dw, fresh)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        abi.rehydrate_batched_noalloc(dw.layout, dw.descs, dw.pool_desc, torch.cuda.current_stream())
    for rep in range(3):
        _restore(dw, fresh)
        abi.rehydrate_batched(dw.layout, dw.descs[:1], dw.pool_desc, dw.workspace)   # other work in between
        _restore(dw, fresh)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert _same(_outputs(dw), eager), f"{label}: replay {rep}"


def test_noalloc_at_its_scratch_limit():
    """A re-anchored chunk whose cos/sin table nearly fills the 4 MiB scratch runs (and matches
    the workspace entry point byte for byte); one token more than fits is rejected before
    anything is enqueued, and the library keeps working afterwards."""
    from position_free_kv_amd import abi
    from workloads.device import DeviceWorkload
    limit = abi.NOALLOC_SCRATCH_BYTES
    fixed = abi.batch_workspace_bytes(*_one_chunk_batch(16)) - 16 * 64 * 8
    T = (limit - fixed) // (64 * 8) // 16 * 16          # tokens of whole 16-token tiles that still fit
    wl = make_workload("C2", num_layers=1, num_chunks=1, tokens=T, positions=True)
    dw = DeviceWorkload(wl, device="cuda:0")
    need = abi.batch_workspace_bytes(dw.layout, dw.descs)
    say(f"[noalloc limit] T={T}: {need} of {limit} bytes")
    assert limit - 16 * 64 * 8 < need <= limit
    fresh = _outputs(dw)
    abi.rehydrate_batched(dw.layout, dw.descs, dw.pool_desc, dw.workspace)
    torch.cuda.synchronize()
    want = _outputs(dw)
    _restore(dw, fresh)
    abi.rehydrate_batched_noalloc(dw.layout, dw.descs, dw.pool_desc)
    torch.cuda.synchronize()
    assert _same(_outputs(dw), want)
    # one more tile does not fit: host validation rejects it, nothing runs
    big = make_workload("C2", num_layers=1, num_chunks=1, tokens=T + 16, positions=True)
    dwb = DeviceWorkload(big, device="cuda:0")
    assert abi.batch_workspace_bytes(dwb.layout, dwb.descs) > limit
    before = _outputs(dwb)
    with pytest.raises(abi.KameraError) as err:
        abi.rehydrate_batched_noalloc(dwb.layout, dwb.descs, dwb.pool_desc)
    assert err.value.name == "KAMERA_E_WORKSPACE"
    torch.cuda.synchronize()
    assert _same(_outputs(dwb), before)
    _restore(dw, fresh)
    abi.rehydrate_batched_noalloc(dw.layout, dw.descs, dw.pool_desc)
    torch.cuda.synchronize()
    assert _same(_outputs(dw), want)


def _one_chunk_batch(T):
    """(layout, [desc]) of a one-chunk re-anchored GQA batch with fake device addresses, only for sizing."""
    from position_free_kv_amd import abi
    lay = abi.make_layout(abi.GQA, abi.BF16, 1, num_kv_heads=4, head_dim=128, rope_base=1e6,
                          mrope_section=(16, 24, 24))
    fake = 1 << 36
    d = abi.ChunkDesc(num_tokens=T, delta=0, flags=abi.POSITIONS, k_src=fake, v_src=fake, k_dst=fake, v_dst=fake,
                      positions=fake)
    return lay, [d]
