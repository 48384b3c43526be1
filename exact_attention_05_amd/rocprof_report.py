"""Summaries of rocprofv3 output for the attention kernels.

Turns the CSV files that ``rocprofv3 --kernel-trace --stats`` and
``rocprofv3 --pmc ...`` write into short Markdown tables, and derives

* per-kernel achieved TFLOP/s or GB/s against MI355X's peaks, from the
  algorithmic work per launch and the kernel's average duration;
* HBM traffic per launch from ``FETCH_SIZE`` / ``WRITE_SIZE`` (KiB per
  dispatch), each scaled by what the same counter reads for a plain device
  copy of known size in the same run;
* instruction mix (VALU, transcendental, MFMA, LDS) from the SQ counters;
* the shader clock under load from ``SQ_BUSY_CU_CYCLES`` and the dispatch
  durations.

Only parsing happens here; the profiler itself runs as its own command with
the program after ``--``.  Usage::

    python -m exact_attention_05_amd.rocprof_report stats DIR --title T --cmd C
    python -m exact_attention_05_amd.rocprof_report traffic --fetch DIR --write DIR \
        --kernel REGEX --calib-mib 256 --key NAME --sources fwd.hip,common.h --cmd C
    python -m exact_attention_05_amd.rocprof_report counters DIR --kernel REGEX
    python -m exact_attention_05_amd.rocprof_report clock DIR --kernel REGEX --key NAME --sources fwd.hip,common.h --cmd C
    python -m exact_attention_05_amd.rocprof_report cycles --run LABEL=DIR:TILES ... --kernel REGEX --title T --cmd C ...
    python -m exact_attention_05_amd.rocprof_report utilisation --a DIR --b DIR --kernel LABEL=REGEX ... --title T --cmd C ...
"""

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")

PEAK_BF16_TFLOPS = 2516.6
PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS  # dense E4M3 MFMA
PEAK_HBM_GBPS = 8000.0
COPY_KERNEL = r"copyBuffer"


def short_name(n):
    """Readable name of a mangled attention kernel (template arguments kept)."""
    n = n.replace("_ZN4attn12_GLOBAL__N_1", "")
    m = re.match(r"(\d+)", n)
    if m:
        ln = int(m.group(1))
        start = len(m.group(1))
        base = n[start:start + ln]
        rest = n[start + ln:]
        args = [a or ("true" if b == "1" else "false") for a, b in re.findall(r"Li(\d+)E|Lb(\d)E", rest)]
        return f"{base}<{','.join(args)}>" if args else base
    n = n.replace("(anonymous namespace)::", "").split("(")[0]
    return re.sub(r"^void |attn::", "", n)


def _find(d, suffix):
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def kernel_stats(d):
    """[(name, calls, avg_ns, min_ns, max_ns, pct)] from the --stats CSV."""
    rows = []
    with open(_find(d, "kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]),
                         float(r["MaxNs"]), float(r["Percentage"])))
    return rows


def counter_values(d):
    """{(kernel_name, counter): [value per dispatch]} from a --pmc run."""
    out = collections.defaultdict(list)
    with open(_find(d, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            out[(r["Kernel_Name"], r["Counter_Name"])].append(float(r["Counter_Value"]))
    return out


def _match(vals, kernel_re, counter):
    hits = [v for (k, c), v in vals.items() if c == counter and re.search(kernel_re, k)]
    if not hits:
        raise KeyError(f"no {counter} values for kernels matching {kernel_re!r}")
    flat = [x for h in hits for x in h]
    return sum(flat) / len(flat), len(flat)


def _largest(vals, kernel_re, counter):
    hits = [x for (k, c), v in vals.items() if c == counter and re.search(kernel_re, k) for x in v]
    if not hits:
        raise KeyError(f"no {counter} values for kernels matching {kernel_re!r}")
    return max(hits)


def src_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_dispatch_stats(d):
    """[(name, grid, calls, avg_ns, min_ns, max_ns, pct)] from the --kernel-trace
    CSV, one row per kernel and grid size (one kernel can serve several
    workloads in one run), or None when the directory holds no trace."""
    try:
        path = _find(d, "kernel_trace.csv")
    except FileNotFoundError:
        return None
    groups = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            groups[(r["Kernel_Name"], grid)].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    total = sum(sum(v) for v in groups.values()) or 1
    rows = [(name, grid, len(v), sum(v) / len(v), min(v), max(v), 100.0 * sum(v) / total)
            for (name, grid), v in groups.items()]
    rows.sort(key=lambda r: -r[2] * r[3])
    return rows


def cmd_stats(a):
    rows = kernel_dispatch_stats(a.dir)
    if rows is None:
        rows = [(name, None, calls, avg, mn, mx, pct) for name, calls, avg, mn, mx, pct in kernel_stats(a.dir)]
    work = []
    for spec in a.work or []:
        # REGEX[@GRID]=AMOUNT:UNIT with UNIT in {flop, flop8, byte} (flop8: FP8
        # products); GRID (work-items per launch) picks one workload of a kernel
        rx, rest = spec.rsplit("=", 1)
        grid = None
        if "@" in rx:
            rx, g = rx.rsplit("@", 1)
            grid = int(g)
        amt, unit = rest.split(":")
        work.append((rx, grid, float(amt), unit))
    lines = [f"# {a.title}", "", "Command (MI355X host, repository root):", "", "```", a.cmd, "```", ""]
    lines.append("| kernel | grid (work-items) | calls | average (us) | min (us) | max (us) | share | achieved vs peak |")
    lines.append("|---|---|---|---|---|---|---|---|")
    for name, grid, calls, avg, mn, mx, pct in rows:
        ach = ""
        for rx, wgrid, amt, unit in work:
            if re.search(rx, name) and (wgrid is None or wgrid == grid):
                if unit in ("flop", "flop8"):
                    t = amt / (avg * 1e-9) / 1e12
                    peak, kind = (PEAK_FP8_TFLOPS, "FP8") if unit == "flop8" else (PEAK_BF16_TFLOPS, "bf16")
                    ach = f"{t:.1f} TFLOP/s = {100 * t / peak:.1f}% of {kind} MFMA"
                else:
                    g = amt / (avg * 1e-9) / 1e9
                    ach = f"{g:.1f} GB/s = {100 * g / PEAK_HBM_GBPS:.1f}% of HBM"
        gtxt = "" if grid is None else str(grid)
        lines.append(f"| `{short_name(name)}` | {gtxt} | {calls} | {avg / 1e3:.1f} | {mn / 1e3:.1f} | {mx / 1e3:.1f} | "
                     f"{pct:.1f}% | {ach} |")
    text = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text)


def cmd_traffic(a):
    fv = counter_values(a.fetch)
    wv = counter_values(a.write)
    calib = a.calib_mib * 2 ** 20
    # the calibration copy is the largest copy dispatch of the run (input
    # uploads may add small ones)
    f_copy = _largest(fv, COPY_KERNEL, "FETCH_SIZE")
    w_copy = _largest(wv, COPY_KERNEL, "WRITE_SIZE")
    f_scale = calib / (f_copy * 1024.0)
    w_scale = calib / (w_copy * 1024.0)
    f_k, nf = _match(fv, a.kernel, "FETCH_SIZE")
    w_k, nw = _match(wv, a.kernel, "WRITE_SIZE")
    fetch_b = f_k * 1024.0 * f_scale
    write_b = w_k * 1024.0 * w_scale
    total = fetch_b + write_b
    path = os.path.join(ROOT, "profiles", "traffic.json")
    tab = {}
    if os.path.exists(path):
        with open(path) as f:
            tab = json.load(f)
    srcs = a.sources.split(",")
    tab[a.key] = {
        "bytes_per_launch": round(total),
        "fetch_bytes": round(fetch_b),
        "write_bytes": round(write_b),
        "fetch_scale": round(f_scale, 4),
        "write_scale": round(w_scale, 4),
        "kernel_regex": a.kernel,
        "sources": srcs,
        "source_sha": src_sha(srcs),
    }
    with open(path, "w") as f:
        json.dump(tab, f, indent=1, sort_keys=True)
        f.write("\n")
    lines = [
        f"# HBM traffic of `{a.kernel}` ({a.key})", "", "Commands (MI355X host, repository root):", "", "```", a.cmd, "```", "",
        f"Calibration: a device copy of {a.calib_mib} MiB reads FETCH_SIZE = {f_copy:.1f} KiB and "
        f"WRITE_SIZE = {w_copy:.1f} KiB, so the counters are scaled by {f_scale:.4f} (fetch) and "
        f"{w_scale:.4f} (write).", "",
        "| counter | raw KiB per dispatch | dispatches | scaled bytes per launch |",
        "|---|---|---|---|",
        f"| FETCH_SIZE | {f_k:.1f} | {nf} | {fetch_b:.0f} |",
        f"| WRITE_SIZE | {w_k:.1f} | {nw} | {write_b:.0f} |",
        f"| total | | | {total:.0f} |",
    ]
    if a.algorithmic:
        lines.append("")
        lines.append(f"Algorithmic bytes per launch: {a.algorithmic:.0f}; measured / algorithmic = "
                     f"{total / a.algorithmic:.3f}.")
    text = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text)


def cmd_counters(a):
    vals = counter_values(a.dir)
    names = sorted({c for (k, c) in vals if re.search(a.kernel, k)})
    print(f"| counter | mean per dispatch |\n|---|---|")
    got = {}
    for c in names:
        v, _ = _match(vals, a.kernel, c)
        got[c] = v
        print(f"| {c} | {v:.1f} |")
    if "SQ_INSTS_MFMA" in got and "SQ_INSTS_VALU" in got:
        print(f"\nVALU instructions per MFMA instruction: {got['SQ_INSTS_VALU'] / got['SQ_INSTS_MFMA']:.2f}")


def cmd_clock(a):
    """Average shader clock of a kernel under load: SQ_BUSY_CU_CYCLES per
    dispatch over the 256 CUs, divided by the dispatch's duration (both from
    the same --pmc run's counter CSV)."""
    rows = []
    with open(_find(a.dir, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == "SQ_BUSY_CU_CYCLES" and re.search(a.kernel, r["Kernel_Name"]):
                ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                rows.append((float(r["Counter_Value"]) / a.cus, ns))
    if not rows:
        raise KeyError(f"no SQ_BUSY_CU_CYCLES values for kernels matching {a.kernel!r}")
    cyc = sum(c for c, _ in rows) / len(rows)
    ns = sum(n for _, n in rows) / len(rows)
    ghz = cyc / ns
    path = os.path.join(ROOT, "profiles", "clock.json")
    tab = {}
    if os.path.exists(path):
        with open(path) as f:
            tab = json.load(f)
    srcs = a.sources.split(",")
    tab[a.key] = {"clock_ghz": round(ghz, 4), "busy_cycles_per_cu": round(cyc), "avg_ns": round(ns),
                  "dispatches": len(rows), "kernel_regex": a.kernel, "sources": srcs, "source_sha": src_sha(srcs)}
    with open(path, "w") as f:
        json.dump(tab, f, indent=1, sort_keys=True)
        f.write("\n")
    lines = [
        f"# Shader clock under load of `{a.kernel}` ({a.key})", "", "Command (MI355X host, repository root):", "",
        "```", a.cmd, "```", "",
        "| dispatches | SQ_BUSY_CU_CYCLES / CU | duration (ns) | clock (GHz) |", "|---|---|---|---|",
        f"| {len(rows)} | {cyc:.0f} | {ns:.0f} | {ghz:.3f} |", "",
        f"At this clock the dense bf16 MFMA peak is 256 CU x 4 SIMD x 1024 FLOP/clk x {ghz:.3f} GHz = "
        f"{256 * 4 * 1024 * ghz / 1e3:.1f} TFLOP/s ({100 * ghz / 2.4:.1f}% of the 2.4 GHz figure).",
    ]
    text = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text)


def cmd_cycles(a):
    """Instructions and cycles of one kernel across runs (different sizes or
    inputs): per-wavefront instruction counts, busy cycles per CU, duration and
    clock of each run, and the per-tile increments between the first two runs
    (the loop's cost, free of the per-wavefront prologue and epilogue)."""
    want = ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_SALU",
            "SQ_BUSY_CU_CYCLES"]
    runs = []
    for spec in a.run:
        label, rest = spec.rsplit("=", 1)
        d, tiles = rest.rsplit(":", 1)
        per = collections.defaultdict(dict)  # dispatch -> counter -> value, plus its duration
        with open(_find(d, "counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                if re.search(a.kernel, r["Kernel_Name"]):
                    e = per[r["Dispatch_Id"]]
                    e[r["Counter_Name"]] = float(r["Counter_Value"])
                    e["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if not per:
            raise KeyError(f"no dispatches of kernels matching {a.kernel!r} in {d}")
        mean = {c: sum(e[c] for e in per.values()) / len(per) for c in want + ["ns"]}
        runs.append((label, int(tiles), len(per), mean))
    lines = [f"# Instructions and cycles of `{a.kernel}` ({a.title})", "", "Commands (MI355X host, repository root):",
             "", "```", *a.cmd, "```", "",
             "| run | dispatches | waves | tiles per wave | VALU / wave | MFMA / wave | transcendental / wave | "
             "SALU / wave | busy cycles / CU | duration (us) | clock (GHz) |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for label, tiles, n, m in runs:
        w = m["SQ_WAVES"]
        cyc = m["SQ_BUSY_CU_CYCLES"] / a.cus
        lines.append(f"| {label} | {n} | {w:.0f} | {tiles} | {m['SQ_INSTS_VALU'] / w:.1f} | {m['SQ_INSTS_MFMA'] / w:.1f} | "
                     f"{m['SQ_INSTS_VALU_TRANS_F32'] / w:.1f} | {m['SQ_INSTS_SALU'] / w:.1f} | {cyc:.0f} | "
                     f"{m['ns'] / 1e3:.1f} | {cyc / m['ns']:.3f} |")
    if len(runs) >= 2:
        (la, ta, _, ma), (lb, tb, _, mb) = runs[0], runs[1]
        dt = tb - ta
        inc = {c: (mb[c] / mb["SQ_WAVES"] - ma[c] / ma["SQ_WAVES"]) / dt for c in want[1:5]}
        fixed = ma["SQ_INSTS_VALU"] / ma["SQ_WAVES"] - inc["SQ_INSTS_VALU"] * ta
        lines += ["", f"Per tile and wavefront (from {la} and {lb}): {inc['SQ_INSTS_VALU']:.1f} VALU instructions, of "
                  f"which {inc['SQ_INSTS_MFMA']:.1f} MFMA (SQ_INSTS_VALU counts them) and "
                  f"{inc['SQ_INSTS_VALU_TRANS_F32']:.1f} transcendental, so "
                  f"{inc['SQ_INSTS_VALU'] - inc['SQ_INSTS_MFMA'] - inc['SQ_INSTS_VALU_TRANS_F32']:.1f} "
                  f"other vector instructions; "
                  f"{inc['SQ_INSTS_SALU']:.1f} scalar. Per wavefront outside the loop: {fixed:.0f} VALU instructions."]
    text = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text)


def cmd_utilisation(a):
    """Per-SIMD split of a kernel's cycles from the two --pmc passes: matrix
    unit busy (SQ_VALU_MFMA_BUSY_CYCLES), VALU issuing (SQ_ACTIVE_INST_VALU,
    4-cycle units), both at once (SQ_VALU_MFMA_COEXEC_CYCLES) and neither,
    against the launch's cycles (SQ_BUSY_CU_CYCLES per CU); the raw means
    follow."""
    simds = 4 * a.cus
    lines = [f"# {a.title}", "", "Commands (MI355X host, repository root):", "", "```", *a.cmd, "```", "",
             "Per SIMD: SQ_ACTIVE_INST_VALU x 4 / SIMDs (4-cycle units), SQ_VALU_MFMA_BUSY_CYCLES and "
             "SQ_VALU_MFMA_COEXEC_CYCLES / SIMDs, SQ_BUSY_CU_CYCLES / CUs = the cycles of the launch "
             f"({a.cus} CUs, {simds} SIMDs).", "",
             "| kernel | cycles | MFMA busy | VALU issuing | both at once | neither |", "|---|---|---|---|---|---|"]
    raw = []
    for spec in a.kernel:
        label, regex = spec.split("=", 1)
        va, vb = counter_values(a.a), counter_values(a.b)
        cyc = _match(va, regex, "SQ_BUSY_CU_CYCLES")[0] / a.cus
        valu = _match(va, regex, "SQ_ACTIVE_INST_VALU")[0] * 4 / simds
        mfma = _match(vb, regex, "SQ_VALU_MFMA_BUSY_CYCLES")[0] / simds
        both = _match(vb, regex, "SQ_VALU_MFMA_COEXEC_CYCLES")[0] / simds
        neither = cyc - (mfma + valu - both)
        pct = lambda x: f"{100 * x / cyc:.0f}%"
        lines.append(f"| {label} | {cyc / 1e3:.0f} k | {pct(mfma)} | {pct(valu)} | {pct(both)} | {pct(neither)} |")
        raw.append((label, regex, va, vb))
    for label, regex, va, vb in raw:
        lines += ["", f"## {label}", "", "| counter | mean per dispatch |", "|---|---|"]
        for vals in (va, vb):
            for c in sorted({c for (k, c) in vals if re.search(regex, k)}):
                lines.append(f"| {c} | {_match(vals, regex, c)[0]:.1f} |")
    text = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--title", required=True)
    s.add_argument("--cmd", required=True)
    s.add_argument("--out")
    s.add_argument("--work", action="append", help="REGEX[@GRID]=AMOUNT:flop|flop8|byte per launch")
    s.set_defaults(fn=cmd_stats)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--calib-mib", type=int, required=True)
    t.add_argument("--key", required=True)
    t.add_argument("--sources", required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--algorithmic", type=float, default=0.0)
    t.add_argument("--out")
    t.set_defaults(fn=cmd_traffic)
    k = sub.add_parser("clock")
    k.add_argument("dir")
    k.add_argument("--kernel", required=True)
    k.add_argument("--key", required=True)
    k.add_argument("--sources", required=True)
    k.add_argument("--cmd", required=True)
    k.add_argument("--cus", type=int, default=256)
    k.add_argument("--out")
    k.set_defaults(fn=cmd_clock)
    y = sub.add_parser("cycles")
    y.add_argument("--run", action="append", required=True, help="LABEL=DIR:TILES_PER_WAVE (a --pmc run)")
    y.add_argument("--kernel", required=True)
    y.add_argument("--title", required=True)
    y.add_argument("--cmd", action="append", required=True)
    y.add_argument("--cus", type=int, default=256)
    y.add_argument("--out")
    y.set_defaults(fn=cmd_cycles)
    w = sub.add_parser("utilisation")
    w.add_argument("--a", required=True, help="pass with SQ_ACTIVE_INST_VALU and SQ_BUSY_CU_CYCLES")
    w.add_argument("--b", required=True, help="pass with SQ_VALU_MFMA_BUSY_CYCLES and SQ_VALU_MFMA_COEXEC_CYCLES")
    w.add_argument("--kernel", action="append", required=True, help="LABEL=REGEX")
    w.add_argument("--title", required=True)
    w.add_argument("--cmd", action="append", required=True)
    w.add_argument("--cus", type=int, default=256)
    w.add_argument("--out")
    w.set_defaults(fn=cmd_utilisation)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--kernel", required=True)
    c.set_defaults(fn=cmd_counters)
    a = ap.parse_args(argv)
    a.fn(a)


if __name__ == "__main__":
    sys.exit(main())
