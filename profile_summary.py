"""Summarise rocprofv3 output of bench.py into profiles/ (kernel time and HBM bytes).

Produce the raw output with three runs of the committed bench (one for the
kernel trace, one per counter, as rocprofv3 collects counters in runs of their
own), then summarise:

    rocprofv3 --kernel-trace --stats --output-format csv -d OUT/prof_trace -o c4 -- \\
        python3 bench.py --config C4 --steps 50 --warmup 5 --no-cpu > OUT/trace.log
    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/prof_fetch -o c4 -- \\
        python3 bench.py --config C4 --steps 5 --warmup 1 --no-cpu > OUT/fetch.log
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/prof_write -o c4 -- \\
        python3 bench.py --config C4 --steps 5 --warmup 1 --no-cpu > OUT/write.log
    python3 profile_summary.py OUT C4

(the -o prefix is the workload name in lower case; OUT/trace.log, OUT/fetch.log and
OUT/write.log hold each run's bench.py JSON line, which counts the operator
launches of the run: whole calls, plan launches, then the same-pattern copy). For per-token re-anchoring, trace
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
import re
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL = "kamera::rehydrate_mfma"
COPY_BYTES = 1 << 30


def _rows(path):
    with open(path) as fh:
        return list(csv.DictReader(fh))


COPY_LAUNCHES = 13   # bench.py's 1 GiB device copy: 3 untimed + 10 timed


def _copy_kib(rows):
    """Counter of the bench's 1 GiB copy: the copy-kernel dispatches within 1% of the largest
    copy-kernel value of the run (host-to-device staging copies use the same kernel and grid,
    on blocks of at most tens of MB, so none comes near 1 GiB)."""
    vals = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
    top = max(vals)
    v = [x for x in vals if x >= 0.99 * top]
    if len(v) < COPY_LAUNCHES:
        raise ValueError(f"expected {COPY_LAUNCHES} dispatches of the 1 GiB copy, found {len(v)}")
    return sum(v) / len(v)


def _own(rows, bench: dict, positions: bool):
    """The workload's own dispatches of one instantiation, in dispatch order: bench.py ends
    with its same-pattern copy (the same chunks at delta 0 without a patch, a lighter load)
    and, in the default run, a secondary workload; when those run the same instantiation
    (same kernel variant), their launches at the end are not the workload's."""
    rows = sorted(rows, key=lambda r: int(r["Dispatch_Id"]))
    ln = bench["launches"]
    same = ln.get("pattern_variant", ln.get("plan_variant")) == ln.get("plan_variant")
    drop = 0 if positions or not same else ln["pattern"]
    # the default run's secondary workload comes last, through the same instantiation when its
    # variant matches
    if ln.get("secondary") and ln.get("secondary_variant") == ln.get("plan_variant"):
        drop += ln["secondary"]
    return rows[:len(rows) - drop] if drop else rows


def _kernel_kib(rows, name: str, bench: dict, positions: bool):
    own = _own([r for r in rows if r["Kernel_Name"].split("(")[0] == name.split("(")[0]], bench, positions)
    vals = [float(r["Counter_Value"]) for r in own]
    return sum(vals) / len(vals), len(vals)


def _own_average_us(out: str, pre: str, name: str, bench: dict, positions: bool):
    """Average duration of the workload's own launches of `name` (whole calls and plan
    launches through that instantiation)."""
    rows = [r for r in _rows(os.path.join(out, "prof_trace", f"{pre}_kernel_trace.csv")) if r["Kernel_Name"] == name]
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in _own(rows, bench, positions)]
    return sum(durs) / len(durs), len(durs)


def _pos_arg(name: str) -> bool:
    """The per-token-offsets template argument of an operator instantiation's name,
    kamera::rehydrate_mfma<slabs, k-steps, positions, valu>."""
    m = re.search(r"rehydrate_mfma<\s*\d+,\s*\d+,\s*(true|false)", name)
    return bool(m) and m.group(1) == "true"


def _bench_line(out: str, log: str = "trace.log") -> dict:
    with open(os.path.join(out, log)) as fh:
        return json.loads(next(ln for ln in fh if ln.startswith("{")))


def main(out: str, cfg: str, positions: bool = False) -> None:
    pre = cfg.lower()
    stats = _rows(os.path.join(out, "prof_trace", f"{pre}_kernel_stats.csv"))
    bench = _bench_line(out)
    # the kernel the bench line measures: with --positions, the instantiation that
    # reads per-token tables (template flag true); the same-pattern copy in that
    # run is the plain variant and is listed but not summarised
    main_row = next(r for r in stats if KERNEL in r["Name"] and "_inline" not in r["Name"] and _pos_arg(r["Name"]) == positions)
    avg_us, n_own = _own_average_us(out, pre, main_row["Name"], bench, positions)
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
        f"python3 bench.py --config {cfg}{flag} --steps {bench['steps']} --warmup {bench['warmup']} --no-cpu",
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
        f"(the same-pattern copy's launches of the same instantiation excluded"
        + (f"; {bench['kernel_us_after_cache_flush']['launches']} of them follow a 1 GiB cache-flushing write, "
           f"{bench['kernel_us_after_cache_flush']['mean']:.1f} us each by bench.py's events"
           if bench.get("kernel_us_after_cache_flush") else "") + ")",
        f"bench.py's own HIP-event figure for the same kernel in the same run: {bench['kernel_us']:.1f} us "
        f"(rocprofv3 average {avg_us:.1f} us).",
        f"algorithmic bytes per launch: {alg / 1e6:.1f} MB, {alg / (avg_us * 1e-6) / 1e9:.0f} GB/s at the rocprofv3 "
        f"average ({alg / (avg_us * 1e-6) / 8e12:.1%} of 8000 GB/s)",
    ]
    if have_pmc:
        fetch = _rows(os.path.join(out, "prof_fetch", f"{pre}_counter_collection.csv"))
        write = _rows(os.path.join(out, "prof_write", f"{pre}_counter_collection.csv"))
        f_copy, w_copy = _copy_kib(fetch), _copy_kib(write)
        f_scale, w_scale = (COPY_BYTES / 1024) / f_copy, (COPY_BYTES / 1024) / w_copy
        f_k, nf = _kernel_kib(fetch, main_row["Name"], _bench_line(out, "fetch.log"), positions)
        w_k, nw = _kernel_kib(write, main_row["Name"], _bench_line(out, "write.log"), positions)
        fetch_b = f_k * 1024 * f_scale
        write_b = w_k * 1024 * w_scale
        lines += [
            "",
            "## HBM bytes (rocprofv3 --pmc, one counter per run)",
            "",
            f"commands: rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE --output-format csv -d OUT/prof_fetch|prof_write "
            f"-o {pre} -- python3 bench.py --config {cfg}{flag} --steps 5 --warmup 1 --no-cpu "
            f"(the workload's own dispatches of the summarised kernel)",
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


# ----------------------------------------------------------------------------- counter comparisons
DERIVED = [
    ("UTCL1 translation miss rate", "TCP_UTCL1_TRANSLATION_MISS_sum",
     ("TCP_UTCL1_TRANSLATION_MISS_sum", "TCP_UTCL1_TRANSLATION_HIT_sum")),
    ("vector L1 -> L2 read latency (cycles per request)", "TCP_TCC_READ_REQ_LATENCY_sum", ("TCP_TCC_READ_REQ_sum",)),
    ("vector L1 -> L2 write latency (cycles per request)", "TCP_TCC_WRITE_REQ_LATENCY_sum", ("TCP_TCC_WRITE_REQ_sum",)),
    ("L2 hit rate", "TCC_HIT_sum", ("TCC_HIT_sum", "TCC_MISS_sum")),
    ("UTCL2 busy share of GPU-active cycles", "GRBM_UTCL2_BUSY", ("GRBM_GUI_ACTIVE",)),
    ("share of wave cycles waiting on instructions", "SQ_WAIT_INST_ANY", ("SQ_WAVE_CYCLES",)),
]


def counters(out: str, name: str, runs: list) -> None:
    """Per-dispatch means of rocprofv3 --pmc counters over the workload's own dispatches of the
    operator kernel, for several runs side by side. Each run is `label=dir`: dir holds pass
    subdirectories p1, p2, ... (one rocprofv3 --pmc run each, output prefix = the workload name
    in lower case) and, beside them, dir_p1.log, ... with each pass's bench.py JSON line."""
    table = {}
    cmds = []
    hashes = set()
    for spec in runs:
        label, d = spec.rsplit("=", 1)
        vals = {}
        k = 1
        while os.path.isdir(os.path.join(out, d, f"p{k}")):
            bench = _bench_line(out, f"{d}_p{k}.log")
            hashes.add(bench["kernel_source_hash"])
            pre = bench["config"]["name"].lower()
            rows = _rows(os.path.join(out, d, f"p{k}", f"{pre}_counter_collection.csv"))
            op = [r for r in rows if KERNEL in r["Kernel_Name"]]
            # the instantiation the workload runs: the one with the most dispatches
            by_name = {}
            for r in op:
                by_name.setdefault(r["Kernel_Name"].split("(")[0], set()).add(r["Dispatch_Id"])
            main_name = max(by_name, key=lambda n: len(by_name[n]))
            mine = [r for r in op if r["Kernel_Name"].split("(")[0] == main_name]
            ids = sorted({int(r["Dispatch_Id"]) for r in mine})
            drop = bench["launches"]["pattern"]
            own = set(ids[:len(ids) - drop] if drop else ids)
            per = {}
            for r in mine:
                if int(r["Dispatch_Id"]) in own:
                    per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            for cn, v in per.items():
                vals[cn] = sum(v) / len(v)
            ctrs = sorted(per)
            flags = " ".join(a for a in ("--page-order physical",) if "physical" in bench["config"]["workload"])
            cmds.append(f"rocprofv3 --pmc {' '.join(ctrs)} --output-format csv -d OUT/{d}/p{k} -o {pre} -- "
                        f"python3 bench.py --config {bench['config']['name']} {flags} --steps {bench['steps']} "
                        f"--warmup {bench['warmup']} --no-cpu --no-copy".replace("  ", " "))
            k += 1
        table[label] = vals
    labels = list(table)
    names = sorted({c for v in table.values() for c in v})
    lines = [f"# rocprofv3 counters: {KERNEL}, {name}", "",
             f"kernel source hash: {', '.join(sorted(hashes))}", "",
             "Per-dispatch means over the workload's own dispatches of the operator kernel (the same-pattern copy's "
             "dispatches excluded). Commands (one counter pass each; OUT is the output folder):", ""]
    lines += [f"    {c}" for c in cmds]
    lines += ["", "summarised with: python3 profile_summary.py " + " ".join(f'"{a}"' if " " in a else a
                                                                for a in sys.argv[1:])]
    lines += ["", "| counter | " + " | ".join(labels) + " |", "|---|" + "---|" * len(labels)]
    for c in names:
        lines.append(f"| {c} | " + " | ".join(f"{table[l][c]:.4g}" if c in table[l] else "" for l in labels) + " |")
    lines += ["", "| derived | " + " | ".join(labels) + " |", "|---|" + "---|" * len(labels)]
    for title, num, den in DERIVED:
        cells = []
        for l in labels:
            v = table[l]
            if num in v and all(x in v for x in den) and sum(v[x] for x in den) > 0:
                cells.append(f"{v[num] / sum(v[x] for x in den):.4g}")
            else:
                cells.append("")
        if any(cells):
            lines.append(f"| {title} | " + " | ".join(cells) + " |")
    with open(os.path.join(ROOT, "profiles", f"counters_{name}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ----------------------------------------------------------------------------- kernel-time sweeps
def sweep(out: str, name: str, title: str, runs: list) -> None:
    """rocprofv3 kernel-trace averages of the operator kernel over several bench runs side by side.
    Each run is `label=dir`: dir holds prof_trace/<prefix>_kernel_trace.csv of one
    `rocprofv3 --kernel-trace` run of bench.py and, beside it, dir.log with its JSON line."""
    lines = [f"# {title}", "",
             "rocprofv3 kernel-trace averages of the operator kernel over each run's own launches (whole calls and plan "
             "launches; the same-pattern copy excluded), with bench.py's HIP-event average of the same kernel in the "
             "same run. Commands (OUT is the output folder):", ""]
    rows = []
    hashes = set()
    for spec in runs:
        label, d = spec.rsplit("=", 1)
        bench = _bench_line(out, f"{d}.log")
        hashes.add(bench["kernel_source_hash"])
        pre = bench["config"]["name"].lower()
        stats = _rows(os.path.join(out, d, "prof_trace", f"{pre}_kernel_stats.csv"))
        cands = [r for r in stats if KERNEL in r["Name"] and "_inline" not in r["Name"]]
        main_row = max(cands, key=lambda r: int(r["Calls"]))
        avg, n = _own_average_us(os.path.join(out, d), pre, main_row["Name"], bench, False)
        alg = bench["algorithmic_bytes"]
        cmd_flags = " ".join(f for f in bench.get("argv", []) if f)
        lines.append(f"    rocprofv3 --kernel-trace --stats --output-format csv -d OUT/{d}/prof_trace -o {pre} -- "
                     f"python3 bench.py {cmd_flags}")
        rows.append(f"| {label} | {main_row['Name'].split('(')[0].replace('void kamera::', '')} | {n} | {avg:.1f} | "
                    f"{bench['kernel_us']:.1f} | {alg / 1e9:.4f} | {alg / (avg * 1e-6) / 1e9:.0f} | "
                    f"{alg / (avg * 1e-6) / 8e12:.1%} |")
    lines += ["", "summarised with: python3 profile_summary.py " + " ".join(f'"{a}"' if " " in a else a
                                                                for a in sys.argv[1:]),
              "", f"kernel source hash: {', '.join(sorted(hashes))}"]
    lines += ["", "| run | kernel | launches | rocprofv3 average us | bench HIP-event us | algorithmic GB | GB/s | "
              "% of 8 TB/s |", "|---|---|---|---|---|---|---|---|"] + rows
    with open(os.path.join(ROOT, "profiles", f"{name}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    if sys.argv[1:2] == ["--sweep"]:
        # profile_summary.py --sweep OUT NAME TITLE label=dir [label=dir ...]
        sweep(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5:])
        sys.exit(0)
    if sys.argv[1:2] == ["--counters"]:
        # profile_summary.py --counters OUT NAME label=dir [label=dir ...]
        counters(sys.argv[2], sys.argv[3], sys.argv[4:])
        sys.exit(0)
    args = [a for a in sys.argv[1:] if not a.startswith("--")]
    main(args[0], args[1] if len(args) > 1 else "C2", positions="--positions" in sys.argv[1:])
