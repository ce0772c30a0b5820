"""GPU checks of host-side paths: kamera_relocate on paged pools, and concurrent callers.

kamera_relocate (Kamera preprint §5: sliding-window survivors get the rotation only) is
compared with the fp64 oracle's relocation of the same pool rows, placed through the
oracle's page walk; every slot outside the relocated range must keep its bytes.

Concurrency: the library is re-entrant (thread-local error text; a per-device staging
ring under a lock). Several host threads, each with its own stream and workspace, issue
batches at the same time; each output must equal what a single-threaded run produced.
"""
import threading

import numpy as np
import pytest
import torch

import oracle.kamera_oracle as O
from oracle import tolerance as tol
from tests.gpu_util import say
from workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from position_free_kv_amd import abi
    abi.lib()   # fails loudly when the HIP library is missing
    yield


@pytest.mark.parametrize("family,slot0,table", [("gqa", 0, True), ("gqa", 11, True), ("mla", 5, True),
                                                ("gqa", 0, False)])
def test_relocate_paged_matches_oracle(family, slot0, table):
    from position_free_kv_amd import abi
    say(f"[relocate] {family} slot0={slot0} table={table}")
    P, L, num_pages, T, delta = 16, 2, 12, 100, -23456
    rng = np.random.default_rng(31 + slot0)
    if family == "gqa":
        F, lay = 512, abi.make_layout(abi.GQA, abi.BF16, L, num_kv_heads=4, head_dim=128, rope_base=1e6, page_size=P)
        okw = dict(family=O.GQA, num_kv_heads=4, head_dim=128, base=1e6)
    else:
        F, lay = 576, abi.make_layout(abi.MLA, abi.BF16, L, latent_dim=512, rope_dim=64, rope_base=1e4, page_size=P)
        okw = dict(family=O.MLA, latent_dim=512, rope_dim=64, base=1e4)
    pool_f = torch.randn(L, num_pages, P, F)
    pool = pool_f.to(torch.bfloat16).view(torch.int16).cuda()
    before = pool.cpu().numpy().view(np.uint16)
    if table:
        bt = rng.permutation(num_pages).astype(np.int32)[: -(-(slot0 + T) // P)]
    else:                                  # NULL table: slot s is pool row s
        bt = None
    spanned = -(-(slot0 % P + T) // P)    # pages the slots [slot0, slot0 + T) span, with or without a table
    ws = torch.empty(abi.workspace_bytes(1, spanned), dtype=torch.uint8, device="cuda")
    pool_v = torch.zeros_like(pool) if family == "gqa" else None   # never read or written
    abi.relocate(lay, abi.make_pool(pool, pool_v, num_pages), bt, slot0, T, delta, ws)
    torch.cuda.synchronize()
    after = pool.cpu().numpy().view(np.uint16)
    walk = np.arange(num_pages, dtype=np.int32) if bt is None else bt
    pages, offs = O.page_slots(T, walk, slot0, P)
    touched = np.zeros((num_pages, P), dtype=bool)
    touched[pages, offs] = True
    for layer in range(L):
        x = O.upcast(before[layer][pages, offs], O.BF16)
        y = O.relocate(x, delta, **okw)
        S = O.abs_terms(x, tensor=0, delta=delta, rotate_this=True,
                        bands=O.band_offsets(okw["family"], okw.get("num_kv_heads", 0), okw.get("head_dim", 0),
                                             okw.get("latent_dim", 0)),
                        d_rot=128 if family == "gqa" else 64, base=okw["base"], pairing=O.NEOX)
        res = tol.check_bf16(after[layer][pages, offs], y, O.round_to(y, O.BF16), S, 4)
        assert res["fail"] == 0, (layer, res["n"])
        assert np.array_equal(after[layer][~touched], before[layer][~touched])   # other slots: same bytes
        if family == "mla":                                                        # c_KV: same bytes
            assert np.array_equal(after[layer][pages, offs][:, :512], before[layer][pages, offs][:, :512])
    if pool_v is not None:
        assert int(pool_v.abs().sum()) == 0


def test_concurrent_callers_match_a_single_thread():
    from workloads.device import DeviceWorkload
    say("[threads] 4 host threads, own streams and workspaces")
    names = [("C2", dict(num_layers=2, num_chunks=2, tokens=300)), ("C3", dict(num_layers=2, num_chunks=2, tokens=200)),
             ("C5", dict(num_layers=2, num_chunks=6, max_tokens=300)),
             ("C2", dict(num_layers=2, num_chunks=3, tokens=150, positions=True))]
    dws = [DeviceWorkload(make_workload(n, **kw)) for n, kw in names]
    outs = lambda dw: [t.clone() for t in ([t for b in dw.dense for t in b] + (dw.pool or []))]
    # reference: one thread, one call each (in-place survivors restored from a snapshot afterwards)
    snaps = [[t.clone() for t in (dw.pool or [])] for dw in dws]
    ref = []
    for dw in dws:
        dw.run()
        torch.cuda.synchronize()
        ref.append(outs(dw))
    for dw, snap in zip(dws, snaps):
        for t, s in zip(dw.pool or [], snap):
            t.copy_(s)
    torch.cuda.synchronize()
    errors = []

    def work(dw):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(1):
                    dw.run(stream=s)
            s.synchronize()
        except Exception as e:  # noqa: BLE001
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(dw,)) for dw in dws]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for dw, r in zip(dws, ref):
        assert all(torch.equal(a, b) for a, b in zip(outs(dw), r))


def test_evicted_chunk_recalled_into_new_pages_is_byte_identical():
    """Eviction is reversible because the canonical rows are kept (Kamera preprint §5): a chunk
    rehydrated into pool pages, evicted (its pages overwritten), then recalled from its
    canonical rows into different pages gives the same bytes row for row."""
    from position_free_kv_amd import abi
    from tests.gpu_util import custom_workload, factor
    from workloads.configs import BF16, GQA, PATCH, ChunkSpec, LayoutSpec
    from workloads.device import DeviceWorkload
    say("[evict+recall]")
    P, T = 16, 150
    lay = LayoutSpec(GQA, BF16, 3, num_kv_heads=2, head_dim=128, rope_base=1e6, page_size=P)
    perm = np.random.default_rng(8).permutation(40).astype(np.int32)
    n = -(-(3 + T) // P)
    ch = ChunkSpec(index=0, num_tokens=T, delta=7777, flags=PATCH, canon_id=0,
                   factors=[factor(0, 0, 0, 0, 256, 32), factor(0, 1, 1, 0, 256, 32)],
                   block_table=perm[:n].copy(), slot0=3)
    dw = DeviceWorkload(custom_workload(lay, [ch], dense_rows=[], num_pages=40))
    dw.run()
    torch.cuda.synchronize()
    first = [[dw.out_rows(ch, layer, t) for t in (0, 1)] for layer in range(3)]
    for t in dw.pool:                       # evict: every page overwritten
        t.fill_(0x1234)
    ch2 = ChunkSpec(**{**ch.__dict__, "block_table": perm[n:2 * n].copy(), "slot0": 9})
    dw.wl.chunks = [ch2]
    abi.rehydrate_batched(dw.layout, [dw._desc(ch2)], dw.pool_desc, dw.workspace)
    torch.cuda.synchronize()
    for layer in range(3):
        for t in (0, 1):
            assert np.array_equal(dw.out_rows(ch2, layer, t), first[layer][t]), (layer, t)


def test_more_staged_calls_in_flight_than_staging_slots():
    """A paged batch is staged through a ring of 8 pinned host slots: the 9th call in flight
    waits on the host until the copy-in of the 1st has run, then reuses its slot. Twenty
    one-chunk calls on one stream, one workspace, no synchronisation in between (each call's
    copy-in runs after the previous call's kernel, in stream order): every chunk, survivors
    rotated in place and recalled chunks rehydrated into random pages, matches the oracle, and
    no slot outside the chunks' pages changes."""
    from position_free_kv_amd import abi
    from tests.gpu_util import check_all, pool_untouched_ok
    from workloads.device import DeviceWorkload
    say("[ring] 20 staged one-chunk calls on one stream")
    wl = make_workload("C5", num_layers=2, num_chunks=20, max_tokens=300)
    assert all(c.block_table is not None for c in wl.chunks)
    dw = DeviceWorkload(wl)
    stream = torch.cuda.current_stream()
    for d in dw.descs:
        abi.rehydrate_batched(dw.layout, [d], dw.pool_desc, dw.workspace, stream)
    torch.cuda.synchronize()
    tot = check_all(dw)
    say(f"  compared {tot['n']} elements: fail={tot['fail']} p2_only={tot['p2_only']}")
    assert tot["fail"] == 0, tot["bad"][:3]
    assert pool_untouched_ok(dw)


def test_stream_probes_move_what_they_say():
    """The streaming probes bench.py times beside the operator: the copy reproduces its source
    byte for byte (ragged last workgroup included), the write fills every word, and the read
    leaves its sink alone for ordinary data."""
    from position_free_kv_amd import abi
    say("[probes]")
    n = 16 * (3 * 1024 + 37)                        # three full 16 KB blocks and a ragged one
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (n // 4,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    abi.stream_probe(abi.PROBE_COPY, src, dst, n)
    abi.stream_probe(abi.PROBE_READ, src, sink, n)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    assert int(sink.abs().sum()) == 0
    abi.stream_probe(abi.PROBE_WRITE, None, dst, n - 16, 0x01020304)
    torch.cuda.synchronize()
    assert bool((dst[:-4] == 0x01020304).all()) and torch.equal(dst[-4:], src[-4:])
