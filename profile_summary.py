"""Summarise rocprofv3 output of bench.py into profiles/ (kernel time and HBM bytes).

Produce the raw output with three runs of the committed bench (one for the
kernel trace, one per counter, as rocprofv3 collects counters in runs of their
own), then summarise:

    rocprofv3 --kernel-trace --stats --output-format csv -d OUT/prof_trace -o c2 -- \\
        python3 bench.py --config C2 --steps 200 --warmup 20 --no-cpu > OUT/trace.log
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/prof_fetch -o c2 -- \\
        python3 bench.py --config C2 --steps 5 --warmup 1 --no-cpu
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/prof_write -o c2 -- \\
        python3 bench.py --config C2 --steps 5 --warmup 1 --no-cpu
    python3 profile_summary.py OUT C2

(the -o prefix is the workload name in lower case; OUT/trace.log holds the traced
run's bench.py JSON line). For per-token re-anchoring, trace
`bench.py --config C2 --positions ...` the same way and summarise with
`python3 profile_summary.py OUT C2 --positions`: the summary then covers the
variant that reads the per-token cos/sin table, and counter runs are optional
(without OUT/prof_fetch and OUT/prof_write the HBM-bytes section is left out).

HBM bytes: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are each scaled by what
the same counter reads for bench.py's plain 1 GiB device copy (reads 1 GiB,
writes 1 GiB), so the figure is in bytes the memory system actually moved.
"""
from __future__ import annotations

import csv
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL = "kamera::rehydrate_mfma"
COPY_BYTES = 1 << 30


def _rows(path):
    with open(path) as fh:
        return list(csv.DictReader(fh))


def _per_kernel(rows):
    agg = defaultdict(list)
    for r in rows:
        agg[(r["Kernel_Name"], int(r["Grid_Size"]))].append(float(r["Counter_Value"]))
    return agg


def _copy_kib(agg):
    """Counter of the bench's 1 GiB copy: the copy kernel with the largest grid."""
    cands = [(g, v) for (k, g), v in agg.items() if "copyBuffer" in k or "copy" in k.lower() and "kamera" not in k]
    g, v = max(cands, key=lambda x: x[0])
    return sum(v) / len(v)


def _kernel_kib(agg):
    vals = [v for (k, g), vs in agg.items() if KERNEL in k for v in vs]
    return sum(vals) / len(vals), len(vals)


def _own_average_us(out: str, pre: str, name: str, bench: dict):
    """Average duration of the workload's own launches of `name`. bench.py launches the
    uploaded plan K + min(K, 200) times, then runs its same-pattern copy (5 + min(K, 200)
    launches of the same instantiation at delta 0 without a patch, a lighter load): the
    first K + min(K, 200) dispatches in time order are the workload's (whole calls that
    use the same instantiation come before them and are the workload's too)."""
    rows = [r for r in _rows(os.path.join(out, "prof_trace", f"{pre}_kernel_trace.csv")) if r["Kernel_Name"] == name]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    own = bench["steps"] + min(bench["steps"], 200)
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows[:own]]
    return sum(durs) / len(durs), len(durs)


def _bench_line(out: str) -> dict:
    with open(os.path.join(out, "trace.log")) as fh:
        return json.loads(next(ln for ln in fh if ln.startswith("{")))


def main(out: str, cfg: str, positions: bool = False) -> None:
    pre = cfg.lower()
    stats = _rows(os.path.join(out, "prof_trace", f"{pre}_kernel_stats.csv"))
    bench = _bench_line(out)
    # the kernel the bench line measures: with --positions, the instantiation that
    # reads per-token tables (template flag true); the same-pattern copy in that
    # run is the plain variant and is listed but not summarised
    main_row = next(r for r in stats if KERNEL in r["Name"] and (not positions or ", true>" in r["Name"]))
    avg_us, n_own = _own_average_us(out, pre, main_row["Name"], bench)
    alg = bench["algorithmic_bytes"]
    suffix = "_positions" if positions else ""
    flag = " --positions" if positions else ""
    have_pmc = all(os.path.exists(os.path.join(out, d, f"{pre}_counter_collection.csv"))
                   for d in ("prof_fetch", "prof_write"))

    lines = [
        f"# rocprofv3 summary: {KERNEL} on the {cfg} workload{' (per-token re-anchoring)' if positions else ''}",
        "",
        f"workload: {bench['config']['workload']}",
        f"kernel source hash: {bench['kernel_source_hash']}",
        "",
        "## kernel trace (rocprofv3 --kernel-trace --stats)",
        "",
        f"command: rocprofv3 --kernel-trace --stats --output-format csv -d OUT/prof_trace -o {pre} -- "
        f"python3 bench.py --config {cfg}{flag} --steps 200 --warmup 20 --no-cpu",
        "",
        "| kernel | calls | average us | min us | max us | share of GPU time |",
        "|---|---|---|---|---|---|",
    ]
    for r in stats[:6]:
        name = r["Name"].split("(")[0]
        lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} "
                     f"| {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    lines += [
        "",
        f"summarised kernel: {main_row['Name'].split('(')[0]}, averaged over the workload's own {n_own} launches "
        f"(the same-pattern copy's launches of the same instantiation excluded)",
        f"bench.py's own HIP-event figure for the same kernel in the same run: {bench['kernel_us']:.1f} us "
        f"(rocprofv3 average {avg_us:.1f} us).",
        f"algorithmic bytes per launch: {alg / 1e6:.1f} MB, {alg / (avg_us * 1e-6) / 1e9:.0f} GB/s at the rocprofv3 "
        f"average ({alg / (avg_us * 1e-6) / 8e12:.1%} of 8000 GB/s)",
    ]
    if have_pmc:
        fetch = _per_kernel(_rows(os.path.join(out, "prof_fetch", f"{pre}_counter_collection.csv")))
        write = _per_kernel(_rows(os.path.join(out, "prof_write", f"{pre}_counter_collection.csv")))
        f_copy, w_copy = _copy_kib(fetch), _copy_kib(write)
        f_scale, w_scale = (COPY_BYTES / 1024) / f_copy, (COPY_BYTES / 1024) / w_copy
        f_k, nf = _kernel_kib(fetch)
        w_k, nw = _kernel_kib(write)
        fetch_b = f_k * 1024 * f_scale
        write_b = w_k * 1024 * w_scale
        lines += [
            "",
            "## HBM bytes (rocprofv3 --pmc, one counter per run)",
            "",
            f"commands: rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE --output-format csv -d OUT/prof_fetch|prof_write "
            f"-o {pre} -- python3 bench.py --config {cfg}{flag} --steps 5 --warmup 1 --no-cpu",
            "",
            "| counter | plain 1 GiB copy (KiB/dispatch) | scale to bytes | kernel (KiB/dispatch, mean of n) "
            "| kernel bytes |",
            "|---|---|---|---|---|",
            f"| FETCH_SIZE | {f_copy:.0f} | x{f_scale:.3f} | {f_k:.0f} (n={nf}) | {fetch_b / 1e6:.1f} MB |",
            f"| WRITE_SIZE | {w_copy:.0f} | x{w_scale:.3f} | {w_k:.0f} (n={nw}) | {write_b / 1e6:.1f} MB |",
            "",
            f"measured HBM traffic per launch: {(fetch_b + write_b) / 1e6:.1f} MB; algorithmic: {alg / 1e6:.1f} MB "
            f"(ratio {(fetch_b + write_b) / alg:.3f})",
            f"measured bandwidth: {(fetch_b + write_b) / (avg_us * 1e-6) / 1e9:.0f} GB/s; algorithmic: "
            f"{alg / (avg_us * 1e-6) / 1e9:.0f} GB/s of 8000 ({alg / (avg_us * 1e-6) / 8e12:.1%})",
        ]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"rehydrate_mfma_{cfg}{suffix}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    if have_pmc and not positions:
        with open(os.path.join(ROOT, "profiles", f"traffic_{cfg}.json"), "w") as fh:
            json.dump({"kernel_source_hash": bench["kernel_source_hash"], "hbm_bytes_per_launch": fetch_b + write_b,
                       "fetch_bytes": fetch_b, "write_bytes": write_b, "fetch_scale": f_scale, "write_scale": w_scale,
                       "rocprof_avg_us": avg_us}, fh, indent=1)
    print("\n".join(lines))


if __name__ == "__main__":
    args = [a for a in sys.argv[1:] if not a.startswith("--")]
    main(args[0], args[1] if len(args) > 1 else "C2", positions="--positions" in sys.argv[1:])
