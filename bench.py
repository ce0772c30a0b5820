"""Throughput of the Kamera rehydrate operator on one MI355X.

One step = one kamera_rehydrate_batched call over the whole workload (every
chunk, every layer, K and V), inputs already resident in HBM. The default
workload is the largest one that fits a single GPU: the MHA 7B reorder batch
(32 layers, 32 heads x 128, bf16, all 6 orderings of three 2048-token chunks
plus a fixed fourth, 24 rehydrations with rank-32 K and V patches; 52 GB moved
per step).

Prints one JSON line: whole-job tokens/s (rehydrated tokens per second of wall
time), the dominant kernel's roofline figures measured with HIP events on the
launch stream, and the fp64 CPU oracle's throughput on a bounded sample.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "rehydrated KV tokens/s and achieved HBM GB/s (% of MI355X peak), 1 GPU"
HBM_PEAK_GBPS = 8000.0
WORKLOADS = {
    "C1": "single-layer GQA: 2 KV heads x 64, fp32, 1 chunk of 256 tokens, delta in [0,4096], rank-8 K and V "
          "patches (0.55 MB: bound by launch latency, not by HBM)",
    "C2": "GQA VL-7B-like: 28 layers, 4 KV heads x 128, bf16, 8 chunks x 1024 tokens, "
          "per-chunk delta in [0,32768], rank-32 K and V patches",
    "C3": "MLA V2-Lite-like: 27 layers, c_KV 512 + k_rope 64, bf16, 16 chunks x 1024 tokens, "
          "rank-32 row and rope-band patches",
    "C4": "MHA 7B reorder: 32 layers, 32 heads x 128, bf16, 6 orderings x 4 chunks x 2048 tokens, rank-32",
    "C5": "GQA sliding-window deque: 36 layers, 8 KV heads x 128, bf16, 64 ragged chunks (48 in-place "
          "survivors, 16 recalled with rank-32 patches) into a 16-token paged pool",
}


def _code_only(text: str) -> str:
    """Source text without comments and blank space: what the compiled kernels depend on."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Identity of the operator kernels' code (comments excluded), to tell whether stored
    counter figures were taken on the code being run."""
    h = hashlib.sha256()
    for f in ("kamera_kernels.hip", "kamera_desc.h"):
        with open(os.path.join(ROOT, "position_free_kv_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(cfg: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{cfg}.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------- CPU oracle leg
# (chunk, layer) units timed on the oracle by default: about 10-40 CPU-s of work each
CPU_UNITS = {"C1": 32768, "C2": 448, "C3": 448, "C4": 16, "C5": 576}
CPU_PROCS_MAX = 16       # the host share of one GPU
PLAN_WARMUP = 3          # untimed launches of the uploaded plan before its timed launches
KERNEL_LAUNCHES = 100    # the kernel average covers at least this many launches
FLUSH_BYTES = 1 << 30    # written between launches to evict the 256 MB Infinity Cache
FLUSH_LAUNCHES = 50
PATTERN_WARMUP = 5


def _oracle_units(args):
    """Worker: draw its (chunk, layer) inputs first, then time only the oracle on them.
    Out-of-place GQA/MHA chunks: K and V rehydrated; MLA chunks: the 576-wide row;
    in-place survivors: R(delta) on K (the MLA rope band); each result rounded once to
    the storage dtype, and paged chunks' (page, offset) slots computed."""
    cfg, units, make_kw = args
    import torch
    from threadpoolctl import threadpool_limits
    torch.set_num_threads(1)          # one thread per worker process: no oversubscription
    threadpool_limits(1)
    import oracle.kamera_oracle as O
    from tests.expect import oracle_factors
    from workloads import make_workload
    wl = make_workload(cfg, **make_kw)
    lay = wl.layout
    prepared = []
    for ci, layer in units:
        ch = wl.chunks[ci]
        if ch.in_place:
            xs = [O.upcast(wl.pool_rows(ch, layer, 0), lay.dtype)]
        else:
            xs = [O.upcast(wl.canonical(ch.canon_id, layer, t), lay.dtype) for t in range(lay.num_tensors)]
        prepared.append((ch, xs, oracle_factors(wl, ch, layer) if ch.patched else []))
    geo = dict(num_kv_heads=lay.num_kv_heads, head_dim=lay.head_dim, latent_dim=lay.latent_dim,
               rope_dim=lay.rope_dim)
    t0 = time.perf_counter()
    tokens = 0.0
    for ch, xs, facs in prepared:
        if ch.in_place:
            ys = [O.relocate(xs[0], ch.delta, family=lay.family, base=lay.rope_base, pairing=lay.pairing, **geo)]
        elif lay.family == O.MLA:
            ys = [O.rehydrate_mla(xs[0], ch.delta, latent_dim=lay.latent_dim, rope_dim=lay.rope_dim,
                                  base=lay.rope_base, pairing=lay.pairing, factors=facs, patch=ch.patched)]
        else:
            ys = O.rehydrate_gqa(xs[0], xs[1], ch.delta, num_kv_heads=lay.num_kv_heads, head_dim=lay.head_dim,
                                 base=lay.rope_base, pairing=lay.pairing, factors=facs, patch=ch.patched)
        for y in ys:
            O.round_to(y, lay.dtype)
        if ch.block_table is not None:
            O.page_slots(ch.num_tokens, ch.block_table, ch.slot0, lay.page_size)
        tokens += ch.num_tokens / lay.num_layers   # a token is rehydrated once all its layers are done
    return time.perf_counter() - t0, len(prepared), tokens


def _cpu_share() -> int:
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count() or 1
    return max(1, min(CPU_PROCS_MAX, avail))


def cpu_baseline(cfg: str, wl, sample_units: int, make_kw: dict):
    """The fp64 oracle on a bounded sample of the workload's (chunk, layer) units, spread
    evenly over the chunks and layers: once over a pool of one process per available host
    CPU (at most the 16 that one GPU's share holds), once in a single process on one
    process's share of the sample."""
    import multiprocessing as mp
    procs = _cpu_share()
    all_units = [(ci, layer) for ci in range(len(wl.chunks)) for layer in range(wl.layout.num_layers)]
    if sample_units <= len(all_units):
        pick = [int(round(i * (len(all_units) - 1) / max(1, sample_units - 1))) for i in range(sample_units)]
        units = [all_units[i] for i in pick]
    else:
        units = [all_units[i % len(all_units)] for i in range(sample_units)]
    parts = [(cfg, units[i::procs], make_kw) for i in range(procs) if units[i::procs]]
    ctx = mp.get_context("fork")
    with ctx.Pool(len(parts)) as pool:
        res = pool.map(_oracle_units, parts)
    wall = max(r[0] for r in res)
    cpu_s = sum(r[0] for r in res)
    n_units = sum(r[1] for r in res)
    tokens = sum(r[2] for r in res)
    with ctx.Pool(1) as pool:
        one = pool.map(_oracle_units, [parts[0]])[0]
    kinds = sorted({"in-place survivors (K rotated)" if wl.chunks[ci].in_place else
                    ("MLA rows" if wl.layout.family == 1 else "K and V") for ci, _ in units})
    return {"value": tokens / wall, "unit": "tokens/s", "cores": len(parts), "kind": "oracle",
            "host_cpus": os.cpu_count(), "cpus_available": len(os.sched_getaffinity(0)),
            "one_process": {"value": one[2] / one[0], "unit": "tokens/s", "units": one[1], "wall_s": one[0]},
            "sample": f"{n_units} (chunk, layer) units ({', '.join(kinds)}; fp64, rounded to "
                      f"{'fp32' if wl.layout.dtype == 0 else 'bf16'}) of the {cfg} workload, spread evenly over "
                      f"its chunks and layers, run over {len(parts)} processes: {wall:.1f} s wall, {cpu_s:.1f} CPU-s; "
                      f"tokens = units x chunk tokens / layers; input drawing excluded; one process alone on "
                      f"{one[1]} of the units: {one[0]:.1f} s"}


# ----------------------------------------------------------------------------- patch builder
BUILDER_SHAPES = {
    # name: (layout kwargs, tokens, patched width, rank, description)
    "C2": (dict(family=0, num_kv_heads=4, head_dim=128, rope_base=1e6), 1024, 512, 32,
           "K of one C2 chunk-layer: 1024 tokens x 512 columns (4 heads x 128), bf16, rank 32"),
    "C3": (dict(family=1, latent_dim=512, rope_dim=64, rope_base=1e4), 1024, 576, 32,
           "MLA row of one C3 chunk-layer: 1024 tokens x 576 columns, bf16, rank 32"),
    "C4": (dict(family=0, num_kv_heads=32, head_dim=128, rope_base=1e4), 2048, 4096, 32,
           "K of one C4 chunk-layer: 2048 tokens x 4096 columns (32 heads x 128), bf16, rank 32"),
}


def _builder_case(cfg: str):
    from workloads.builder_inputs import BuilderCase
    from workloads.configs import BF16, LayoutSpec
    lk, T, W, m, desc = BUILDER_SHAPES[cfg]
    lay = LayoutSpec(dtype=BF16, num_layers=1, **lk)
    canon = BuilderCase(lay, tensor=0, num_tokens=T, delta=4096, col0=0, width=W, seed=7).canonical()
    cond = BuilderCase(lay, tensor=0, num_tokens=T, delta=4096, col0=0, width=W, seed=8).canonical()
    return lay, T, W, m, desc, canon, cond


def builder_cpu_baseline(cfg: str, budget_s: float = 10.0):
    """LAPACK (gesdd) truncated SVD of the fp64 deficit, the oracle of the builder, on the host."""
    import oracle.kamera_oracle as O
    from oracle.builder_oracle import deficit, truncated_svd
    lay, T, W, m, desc, canon, cond = _builder_case(cfg)
    bands = O.band_offsets(lay.family, lay.num_kv_heads, lay.head_dim, lay.latent_dim)
    d_rot = O.rotary_width(lay.family, lay.head_dim, lay.rope_dim)
    xc, xk = O.upcast(cond, lay.dtype), O.upcast(canon, lay.dtype)
    n, t0 = 0, time.perf_counter()
    while n < 200 and time.perf_counter() - t0 < budget_s:
        d = deficit(xc, xk, 4096, bands=bands, d_rot=d_rot, base=lay.rope_base, pairing=lay.pairing)[:, :W]
        truncated_svd(d, m)
        n += 1
    wall = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        threads = 1
    return {"value": n / wall, "unit": "builds/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} builds of the same deficit ({desc}): fp64 deficit and LAPACK gesdd; {wall:.1f} s wall"}


def builder_main(args) -> int:
    cpu = None if args.no_cpu else builder_cpu_baseline(args.config)
    import torch
    from position_free_kv_amd import abi
    torch.cuda.set_device(0)
    abi.lib()
    lay, T, W, m, desc, canon, cond = _builder_case(args.config)
    layout = abi.make_layout(lay.family, lay.dtype, 1, num_kv_heads=lay.num_kv_heads, head_dim=lay.head_dim,
                             latent_dim=lay.latent_dim, rope_dim=lay.rope_dim, pairing=lay.pairing,
                             rope_base=lay.rope_base)
    xk = torch.from_numpy(canon.view("int16").copy()).cuda()
    xc = torch.from_numpy(cond.view("int16").copy()).cuda()
    u = torch.empty((T, m), dtype=torch.int16, device="cuda")
    v = torch.empty((W, m), dtype=torch.int16, device="cuda")
    sig = torch.empty(m, dtype=torch.float64, device="cuda")
    ws = torch.empty(abi.build_workspace_bytes(T, W, m), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    call = lambda: abi.build_patch(layout, 0, xc, xk, T, 4096, 0, W, m, args.builder_iterations, u, v, sig, ws,
                                   stream)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    out = {
        "metric": "patch builds/s (fp64 deficit and top-m truncated SVD of one chunk-layer tensor), 1 GPU",
        "value": args.steps / wall, "unit": "builds/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f64", "data": "synthetic: two independent seeded N(0,1) bf16 row blocks (a full-rank deficit)",
        "config": {"workload": desc, "name": args.config, "tokens": T, "width": W, "rank": m,
                   "iterations": args.builder_iterations},
        "gpu_ms_per_build": ms,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


# ----------------------------------------------------------------------------- main
def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="C4", choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-units", type=int, default=None,
                    help="(chunk, layer) units timed on the CPU oracle, spread evenly over the workload "
                         "(repeated as needed); default: about 10-40 CPU-s of oracle work (%s)" %
                         ", ".join(f"{k} {v}" for k, v in CPU_UNITS.items()))
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-copy", action="store_true", help="skip the 1 GiB copy-ceiling probe")
    ap.add_argument("--rank", type=int, default=None, help="override the patch rank m of the workload")
    ap.add_argument("--chunks", type=int, default=None,
                    help="override the chunk count of the workload (C1-C3: chunks of the same shape; launch-size "
                         "studies)")
    ap.add_argument("--deep-half", action="store_true",
                    help="patch only the deeper half of the layers (every factor starts at layer L // 2)")
    ap.add_argument("--shared-basis", action="store_true",
                    help="every chunk uses the same per-layer V for a factor slot (only U differs per chunk)")
    ap.add_argument("--positions", action="store_true",
                    help="re-anchor every rehydrated chunk token by token with (t, h, w) M-RoPE ids "
                         "(64-token frames on an 8 x 8 grid at the chunk's start) instead of one delta")
    ap.add_argument("--patch-unit", choices=("auto", "mfma", "valu"), default="auto",
                    help="unit that adds the patch in the bf16 kernel: the library's choice (auto, the matrix "
                         "cores), the matrix cores, or VALU dot products (128-wide heads, rank <= 64)")
    ap.add_argument("--page-order", choices=("random", "physical"), default="random",
                    help="paged workloads: the seeded random block table (default), or the same chunks with "
                         "their pages numbered in physical order (consecutive page ids, chunk after chunk)")
    ap.add_argument("--builder", action="store_true",
                    help="time the patch builder (kamera_build_patch) on one chunk-layer of --config instead")
    ap.add_argument("--builder-iterations", type=int, default=16)
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary stderr line (the default run also times the 28-layer GQA batch's "
                         "kernel, C2, after its JSON line)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this operator runs on one GPU; chunks and layers are independent, so "
                                   "several GPUs would each rehydrate their own chunks (or layers) with no "
                                   "exchange between them; only --gpus 1 is measured"}), flush=True)
        return 2
    if args.builder:
        if args.config not in BUILDER_SHAPES:
            print(json.dumps({"error": f"no builder shape for {args.config}"}), flush=True)
            return 2
        return builder_main(args)

    from workloads import make_workload
    make_kw = dict(rank=args.rank)
    if args.chunks is not None:
        if args.config not in ("C1", "C2", "C3"):
            print(json.dumps({"error": "--chunks applies to C1, C2 and C3"}), flush=True)
            return 2
        make_kw["num_chunks"] = args.chunks
    if args.page_order != "random":
        make_kw["page_order"] = args.page_order
    wl = make_workload(args.config, **make_kw)
    variant = (args.deep_half or args.shared_basis or args.positions or args.page_order != "random"
               or args.patch_unit != "auto" or args.chunks is not None)
    if args.deep_half or args.shared_basis or args.positions:
        make_kw.update(shared_basis=args.shared_basis, positions=args.positions,
                       patch_layer0=wl.layout.num_layers // 2 if args.deep_half else None)
        wl = make_workload(args.config, **make_kw)
    # The CPU oracle leg forks worker processes, so it runs before this process
    # touches the GPU (forking a process whose HIP runtime threads are live can deadlock).
    cpu = None
    if not args.no_cpu and not variant:
        t_cpu = time.perf_counter()
        units = args.cpu_units if args.cpu_units is not None else CPU_UNITS[args.config]
        cpu = cpu_baseline(args.config, wl, units, make_kw)
        print(f"# cpu oracle leg done in {time.perf_counter() - t_cpu:.1f} s", file=sys.stderr, flush=True)

    import torch
    from position_free_kv_amd import abi
    from workloads.device import DeviceWorkload

    torch.cuda.set_device(0)
    abi.lib()
    t_stage = time.perf_counter()
    dw = DeviceWorkload(wl)
    dw.layout.patch_unit = {"auto": abi.PATCH_UNIT_AUTO, "mfma": abi.PATCH_UNIT_MFMA,
                            "valu": abi.PATCH_UNIT_VALU}[args.patch_unit]
    print(f"# staged {args.config} in {time.perf_counter() - t_stage:.1f} s", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()

    batch = dw.prepared(stream)   # arguments marshalled once; every call validates, uploads, launches
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # Collected before the warmup, not after it: a pause between the warmup and the timed
    # steps leaves the GPU idle long enough to lower its clocks, and the first timed
    # launches then run up to 12% slower (seen in kernel traces of this loop).
    gc.collect()
    gc.disable()   # no collector pauses inside the timed loops
    for _ in range(args.warmup):
        batch.call()
    print(f"# warmup issued ({args.warmup} steps)", file=sys.stderr, flush=True)

    # ---- whole calls (validation + descriptor upload + kernel): the step
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        batch.call()
    e1.record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    call_ms_gpu = e0.elapsed_time(e1) / args.steps

    # ---- the kernel alone: same batch, uploaded once, launched back to back on the
    # same stream (after untimed launches of its own), at least KERNEL_LAUNCHES times
    plan = dw.plan(stream)
    for _ in range(PLAN_WARMUP):
        abi.plan_launch(plan, stream)
    torch.cuda.synchronize()
    n_kernel = max(args.steps, KERNEL_LAUNCHES)
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e2.record(stream)
    for _ in range(n_kernel):
        abi.plan_launch(plan, stream)
    e3.record(stream)
    torch.cuda.synchronize()
    kernel_us = e2.elapsed_time(e3) / n_kernel * 1e3

    # ---- per-launch spread: each launch between its own pair of events
    n_dist = min(max(args.steps, KERNEL_LAUNCHES), 200)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_dist)]
    for ea, eb in evs:
        ea.record(stream)
        abi.plan_launch(plan, stream)
        eb.record(stream)
    torch.cuda.synchronize()
    per_launch = sorted(ea.elapsed_time(eb) * 1e3 for ea, eb in evs)
    pct = lambda q: per_launch[min(len(per_launch) - 1, int(q * len(per_launch)))]

    # ---- the same launches with the 256 MB Infinity Cache flushed before each: 1 GiB of
    # unrelated writes (the library's write probe) between launches, each launch between
    # its own event pair, so no launch can find a previous launch's factors or rows there
    flushed = None
    if not args.no_copy:
        junk = torch.empty(FLUSH_BYTES // 2, dtype=torch.int16, device="cuda")
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(FLUSH_LAUNCHES)]
        for ea, eb in fev:
            abi.stream_probe(abi.PROBE_WRITE, None, junk, FLUSH_BYTES, 0x5A5A5A5A, stream)
            ea.record(stream)
            abi.plan_launch(plan, stream)
            eb.record(stream)
        torch.cuda.synchronize()
        fl = sorted(ea.elapsed_time(eb) * 1e3 for ea, eb in fev)
        flushed = {"mean": sum(fl) / len(fl), "p50": fl[len(fl) // 2], "launches": len(fl),
                   "achieved_GBps_at_mean": dw.algorithmic_bytes() / (sum(fl) / len(fl) * 1e-6) / 1e9}
        del junk

    # ---- the same chunks at delta 0 without a patch: a plain copy through the
    # kernel's own access pattern, the practical ceiling for this workload's layout
    pattern_gbps = None
    pattern_variant = None
    cbytes = dw.copy_bytes()
    if cbytes > 0:
        cplan = abi.plan_upload(dw.layout, dw.copy_descs(), dw.pool_desc, dw.workspace, stream)
        pattern_variant = cplan.variant
        for _ in range(PATTERN_WARMUP):
            abi.plan_launch(cplan, stream)
        e6, e7 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e6.record(stream)
        for _ in range(n_dist):
            abi.plan_launch(cplan, stream)
        e7.record(stream)
        torch.cuda.synchronize()
        pattern_gbps = cbytes / (e6.elapsed_time(e7) / n_dist * 1e-3) / 1e9
    gc.enable()

    # ---- a plain device copy of known size: practical read+write ceiling, and the
    # reference kernel for scaling the HBM byte counters
    copy_gbps = None
    stream_gbps = {}
    if not args.no_copy:
        n = 1 << 30
        src = torch.empty(n // 2, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        e4, e5 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e4.record(stream)
        for _ in range(10):
            dst.copy_(src)
        e5.record(stream)
        torch.cuda.synchronize()
        copy_gbps = 2 * n / (e4.elapsed_time(e5) / 10 * 1e-3) / 1e9
        # the library's streaming probes over the same buffers: the HBM's practical rates for a
        # nontemporal copy, reads alone and writes alone (the operator mixes all three)
        sink = torch.empty(4096, dtype=torch.uint8, device="cuda")
        probes = {"copy": (abi.PROBE_COPY, src, dst, 2 * n), "read": (abi.PROBE_READ, src, sink, n),
                  "write": (abi.PROBE_WRITE, None, dst, n)}
        for name, (kind, a_, b_, moved) in probes.items():
            for _ in range(3):
                abi.stream_probe(kind, a_, b_, n, 0x3F803F80, stream)
            e4.record(stream)
            for _ in range(10):
                abi.stream_probe(kind, a_, b_, n, 0x3F803F80, stream)
            e5.record(stream)
            torch.cuda.synchronize()
            stream_gbps[name] = moved / (e4.elapsed_time(e5) / 10 * 1e-3) / 1e9
        del src, dst, sink

    ms_per_step = wall_s / args.steps * 1e3
    tokens = wl.total_tokens
    alg_bytes = dw.algorithmic_bytes()
    achieved = alg_bytes / (kernel_us * 1e-6) / 1e9
    # counters are taken on the plain workloads only
    traffic = None if variant or args.rank is not None else measured_traffic(args.config)

    out = {
        "metric": METRIC,
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl.layout.dtype == 0 else "bf16",
        "data": "synthetic: seeded N(0,1) canonical KV, orthonormal factors with geometric spectra",
        "config": {"workload": WORKLOADS[args.config] + ("" if args.rank is None else f" (rank overridden: m={args.rank})")
                   + ("" if args.chunks is None else f" (chunk count overridden: {args.chunks})")
                   + (" (deep-half patches: layers L/2..L-1 only)" if args.deep_half else "")
                   + (" (one V basis per layer shared by all chunks)" if args.shared_basis else "")
                   + (" (per-token (t, h, w) re-anchoring, M-RoPE sections %s)" % (wl.layout.mrope_section,)
                      if args.positions else "")
                   + (" (block table in physical page order)" if args.page_order == "physical" else "")
                   + (f" (patch on the {args.patch_unit.upper()})" if args.patch_unit != "auto" else ""),
                   "name": args.config, "chunks": len(wl.chunks),
                   "tokens": tokens, "layers": wl.layout.num_layers, "row_width": wl.layout.row_width},
        "roofline": dict({"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                          "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic},
                         **({"note": "the whole workload is 0.55 MB: the launch is latency-bound and the fraction "
                                     "of HBM peak is not a measure of the kernel"} if args.config == "C1" else {})),
        "kernel_us": kernel_us,
        "kernel_launches_timed": n_kernel,
        "kernel_us_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
        "kernel_us_after_cache_flush": flushed,
        # operator launches in this run, in order: whole calls, plan launches, same-pattern copy
        "launches": {"calls": args.warmup + args.steps,
                     "plan": PLAN_WARMUP + n_kernel + n_dist + (FLUSH_LAUNCHES if flushed else 0),
                     "pattern": (PATTERN_WARMUP + n_dist) if cbytes > 0 else 0,
                     "plan_variant": plan.variant, "pattern_variant": pattern_variant},
        "pattern_copy_GBps": pattern_gbps,
        "frac_of_pattern_copy": (achieved / pattern_gbps) if pattern_gbps else None,
        "call_us_gpu": call_ms_gpu * 1e3,
        "algorithmic_bytes": alg_bytes,
        "kernel_tokens_per_s": tokens / (kernel_us * 1e-6),
        "torch_copy_GBps": copy_gbps,
        "stream_probe_GBps": stream_gbps or None,
        "kernel_source_hash": kernel_source_hash(),
        "argv": sys.argv[1:],
        "cpu_baseline": cpu,
    }
    # the default run also times the 28-layer GQA batch's kernel (C2) after its own line, to stderr
    sec = None
    if args.config == "C4" and not (variant or args.rank is not None or args.no_secondary):
        sec = prepare_secondary("C2", stream)
    out["launches"].update(secondary=SECONDARY_LAUNCHES if sec else 0,
                           secondary_variant=sec[1].variant if sec else None)
    print(json.dumps(out), flush=True)
    if sec:
        secondary_kernel_line("C2", sec, stream)
    return 0


SECONDARY_LAUNCHES = PLAN_WARMUP + 10 + 200 + 200


def prepare_secondary(cfg: str, stream):
    from workloads import make_workload
    from workloads.device import DeviceWorkload
    wl = make_workload(cfg)
    dw = DeviceWorkload(wl)
    return dw, dw.plan(stream), wl


def secondary_kernel_line(cfg: str, sec, stream) -> None:
    """The kernel alone on a second workload, after the main line, to stderr: the same
    plan timing as the main line (untimed launches, then 200 back to back, then 200 each
    between its own events), so machines can be compared on a short launch too."""
    import torch
    from position_free_kv_amd import abi
    dw, plan, wl = sec
    for _ in range(PLAN_WARMUP + 10):
        abi.plan_launch(plan, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(200):
        abi.plan_launch(plan, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / 200 * 1e3
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(200)]
    for ea, eb in evs:
        ea.record(stream)
        abi.plan_launch(plan, stream)
        eb.record(stream)
    torch.cuda.synchronize()
    per = sorted(ea.elapsed_time(eb) * 1e3 for ea, eb in evs)
    alg = dw.algorithmic_bytes()
    print("# secondary " + json.dumps({"config": cfg, "workload": WORKLOADS[cfg], "kernel_us": us,
                                       "kernel_us_p10_p50_p90": [per[20], per[100], per[180]],
                                       "achieved_GBps": alg / (us * 1e-6) / 1e9,
                                       "frac": alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                                       "tokens_per_s_kernel": wl.total_tokens / (us * 1e-6)}),
          file=sys.stderr, flush=True)


if __name__ == "__main__":
    sys.exit(main())
