"""Summarise rocprofv3 CSV output into the short text kept under profiles/.

    python -m mixture_experts_ffn_05_amd.prof_summary trace <kernel_stats.csv> <kernel_substr> <out.md> <command...>
    python -m mixture_experts_ffn_05_amd.prof_summary pmc <fetch_dir> <write_dir> <copy_mib> <kernel_substr> \
        <out.md> <command...>

`trace` writes per-kernel call counts and average durations, and the summed
average duration of the kernels whose name contains <kernel_substr> (the
launches of one timed call; '|' separates alternatives).  `replay` tabulates route-trace replay results (per-stage GPU times and the
shared-vs-routed split); `marker` counts the roctx stage ranges of a
rocprofv3 marker trace.

`sq` tabulates SQ/TA/TD counter runs per kernel (MFMA busy share, waiting
shares, texture-data unit busy and stalled shares, implied clock).

`bandwidth` reads the kernel trace of a bench run with --copy-reference-mb and
reports the copy, read (the cache-eviction reduction) and fill bandwidths.

`pmc` reads two counter-collection runs
(FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), calibrates both against the
device copy of <copy_mib> MiB that the profiled command performed first (its
counters should read copy_mib*1024 KiB each), and writes the calibrated HBM
bytes per dispatch of every kernel, plus a JSON line, read by bench.py for the
roofline object's `traffic` field, with the bytes of one timed call: the sum
over the kernels whose name contains <kernel_substr> (each launched once per
call).  The JSON line records a hash of the kernel sources, so a later change
of a kernel voids the figure.
"""

from __future__ import annotations

import collections
import csv
import glob
import hashlib
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))


def _code_only(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed (string literals
    are kept as they are; none of the kernel sources puts comment markers in one)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


# Sources of every kernel a counter record can name (the grouped GEMMs, the
# combine, the backward kernels) and the header they share.
RECORDED_SOURCES = ("moe_gemm.hip", "moe_combine.hip", "moe_backward.hip", "moe_common.h")


def kernel_source_hash() -> str:
    """Hash of the code of the recorded kernels' sources (comments and layout
    ignored): a change to any of those kernels voids a recorded figure; an
    edited comment, or a change to the routing and scatter kernels, does not."""
    h = hashlib.sha256()
    for name in sorted(RECORDED_SOURCES):
        with open(os.path.join(PKG, "csrc", name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def matches(name: str, kernel_substr: str) -> bool:
    """True if any '|'-separated alternative of kernel_substr occurs in name."""
    name = name.replace("moe::(anonymous namespace)::", "")
    return any(alt and alt in name for alt in kernel_substr.split("|"))


def short(name: str) -> str:
    name = name.replace("moe::(anonymous namespace)::", "")
    return name if len(name) < 110 else name[:107] + "..."


def trace(stats_csv: str, kernel_substr: str, out_md: str, command: str) -> None:
    rows = list(csv.DictReader(open(stats_csv)))
    lines = ["# rocprofv3 kernel trace", "", f"Command: `{command}`", "",
             "| kernel | calls | avg us | total share % |", "|---|---|---|---|"]
    matched = 0.0
    names = []
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
        if matches(r["Name"], kernel_substr):
            matched += float(r["AverageNs"]) / 1e3
            names.append(short(r["Name"]))
    lines += ["", f"Timed call (kernels containing `{kernel_substr}`: {'; '.join(names)}): "
                  f"summed average duration {matched:.2f} us", "",
              "Machine-readable record for the timed call (read by bench.py for the profile-based roofline "
              "fraction):", "",
              "TRACE_JSON " + json.dumps({"kernels": names, "avg_us_per_call": matched,
                                          "gemm_source_hash": kernel_source_hash()})]
    open(out_md, "w").write("\n".join(lines) + "\n")


def _per_dispatch(run_dir: str, counter: str):
    path = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)[0]
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return per


def pmc(fetch_dir: str, write_dir: str, copy_mib: float, kernel_substr: str, out_md: str, command: str) -> None:
    fetch = _per_dispatch(fetch_dir, "FETCH_SIZE")
    write = _per_dispatch(write_dir, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0
    fcopy = [v for k, vs in fetch.items() if "copyBuffer" in k for v in vs if v > 0.5 * copy_kib]
    wcopy = [v for k, vs in write.items() if "copyBuffer" in k for v in vs if v > 0.5 * copy_kib]
    f_scale = copy_kib / max(fcopy) if fcopy else None
    w_scale = copy_kib / max(wcopy) if wcopy else None
    lines = ["# rocprofv3 HBM counters (FETCH_SIZE, WRITE_SIZE)", "",
             f"Command (run once with `--pmc FETCH_SIZE`, once with `--pmc WRITE_SIZE`): `{command}`", "",
             f"Calibration: a device copy of {copy_mib:.0f} MiB reads FETCH_SIZE "
             f"{max(fcopy) if fcopy else float('nan'):.0f} KiB and WRITE_SIZE "
             f"{max(wcopy) if wcopy else float('nan'):.0f} KiB; scale factors "
             f"{f_scale if f_scale else float('nan'):.4f} (fetch) and {w_scale if w_scale else float('nan'):.4f} (write).",
             "", "| kernel | dispatches | FETCH KiB/dispatch | WRITE KiB/dispatch | calibrated HBM MB/dispatch |",
             "|---|---|---|---|---|"]
    record = None
    for k in sorted(set(fetch) | set(write)):
        if "moe::" not in k:
            continue
        fv, wv = fetch.get(k, []), write.get(k, [])
        fa = sum(fv) / len(fv) if fv else 0.0
        wa = sum(wv) / len(wv) if wv else 0.0
        hbm = (fa * (f_scale or 1.0) + wa * (w_scale or 1.0)) * 1024 / 1e6
        lines.append(f"| {short(k)} | {len(fv)} | {fa:.0f} | {wa:.0f} | {hbm:.1f} |")
        if matches(k, kernel_substr):
            if record is None:
                record = {"kernels": [], "fetch_kib": 0.0, "write_kib": 0.0, "fetch_scale": f_scale,
                          "write_scale": w_scale, "hbm_bytes_per_call": 0.0, "gemm_source_hash": kernel_source_hash()}
            record["kernels"].append(short(k))
            record["fetch_kib"] += fa
            record["write_kib"] += wa
            record["hbm_bytes_per_call"] += hbm * 1e6
    lines += ["", f"Machine-readable record for the timed call (kernels containing `{kernel_substr}`; read by "
                  "bench.py):", "",
              "TRAFFIC_JSON " + json.dumps(record)]
    open(out_md, "w").write("\n".join(lines) + "\n")


def sq(out_md: str, command: str, dirs: list, cus: int = 256, xcds: int = 8) -> None:
    """Per-kernel averages of the SQ/TA/TD counters of several counter runs (one
    directory each), with ratios that need no unit assumptions (waiting shares of
    the wave cycles) and ratios that take GRBM_GUI_ACTIVE as the sum over the XCDs
    of the kernel's clock cycles (MFMA busy per SIMD cycle, TD busy per CU cycle,
    and the clock implied by the dispatch duration)."""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    dur = collections.defaultdict(list)
    for d in dirs:
        for path in glob.glob(os.path.join(d, "*counter_collection.csv")):
            for r in csv.DictReader(open(path)):
                k = r["Kernel_Name"]
                if "moe::" not in k:
                    continue
                vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
                if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                    dur[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    avg = lambda xs: sum(xs) / len(xs) if xs else float("nan")
    lines = ["# rocprofv3 SQ / TA / TD counters per kernel", "",
             f"Command (one run per counter set): `{command}`", "",
             "Ratios: *wait* = SQ_WAIT_ANY / SQ_WAVE_CYCLES (share of resident wave time spent in s_waitcnt); "
             "*LDS wait* = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES; *MFMA busy* = SQ_VALU_MFMA_BUSY_CYCLES / "
             f"({cus * 4} SIMDs x cycles); *TD busy*, *TD stalled on TC* = TD_TD_BUSY, TD_TC_STALL / ({cus} CUs x "
             f"cycles); cycles = GRBM_GUI_ACTIVE / {xcds} (taken as summed over the XCDs); *clock* = cycles / the "
             "dispatch's duration under counter collection. For short kernels the counter window outlasts the dispatch "
             "(implied clocks above the 2.4 GHz maximum); the clock and the cycle-based shares are meaningful only for "
             "the long GEMM launches.", "",
             "| kernel | dispatches | MFMA insts | MFMA busy | wait | LDS wait | LDS bank conflicts | TD busy | "
             "TD stalled on TC | clock GHz |", "|---|---|---|---|---|---|---|---|---|---|"]
    for k in sorted(vals):
        v = {c: avg(x) for c, x in vals[k].items()}
        cyc = v.get("GRBM_GUI_ACTIVE", float("nan")) / xcds
        wc = v.get("SQ_WAVE_CYCLES", float("nan"))
        pct = lambda a, b: f"{100.0 * a / b:.0f}%" if b == b and b > 0 and a == a else "n/a"
        lines.append(
            f"| {short(k)} | {len(vals[k].get('SQ_WAVES', []))} | {v.get('SQ_INSTS_MFMA', float('nan')):.4g} | "
            f"{pct(v.get('SQ_VALU_MFMA_BUSY_CYCLES', float('nan')), cus * 4 * cyc)} | "
            f"{pct(v.get('SQ_WAIT_ANY', float('nan')), wc)} | {pct(v.get('SQ_WAIT_INST_LDS', float('nan')), wc)} | "
            f"{v.get('SQ_LDS_BANK_CONFLICT', float('nan')):.4g} | {pct(v.get('TD_TD_BUSY', float('nan')), cus * cyc)} | "
            f"{pct(v.get('TD_TC_STALL', float('nan')), cus * cyc)} | {cyc / avg(dur[k]) / 1e9:.2f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def bandwidth(trace_csv: str, out_md: str, command: str, mib: float = 1024.0) -> None:
    """Reference bandwidths from one kernel trace of a bench run with --copy-reference-mb: the
    device copy of `mib` MiB (read + write), and the cache-eviction pass's 1 GiB reduction (read)
    and 1 GiB fill (write) that the bench runs."""
    rows = list(csv.DictReader(open(trace_csv)))
    nbytes = mib * 2 ** 20

    def durs(pred, min_us):
        out = []
        for r in rows:
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            if pred(r["Kernel_Name"]) and d >= min_us:
                out.append(d)
        return out

    copy = durs(lambda n: "copyBuffer" in n, 100.0)
    read = durs(lambda n: "reduce_kernel" in n, 50.0)
    fill = durs(lambda n: "FillFunctor" in n, 50.0)
    med = lambda xs: sorted(xs)[len(xs) // 2] if xs else float("nan")
    lines = ["# Reference bandwidths on the box", "", f"Command: `{command}`", "",
             f"Each kernel moves {nbytes / 1e9:.3f} GB of payload (1 GiB); GB/s = bytes moved / median duration.", "",
             "| kernel | what it moves | dispatches | median us | GB/s |", "|---|---|---|---|---|"]
    for name, what, xs, factor in (("device copy (copyBuffer)", "1 GiB read + 1 GiB written", copy, 2.0),
                                   ("reduction (torch sum, the cache eviction)", "1 GiB read", read, 1.0),
                                   ("fill (torch ones)", "1 GiB written", fill, 1.0)):
        m = med(xs)
        lines.append(f"| {name} | {what} | {len(xs)} | {m:.1f} | {factor * nbytes / (m * 1e-6) / 1e9:.0f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def replay(out_md: str, command: str, results: list) -> None:
    lines = ["# Route-trace replay: per-stage GPU time", "", f"Command (per trace): `{command}`", "",
             "Times are means over the repeats of HIP-event intervals around each libmoe call, in microseconds; "
             "shared and routed leave out gather / scatter_combine / accumulator_init.", "",
             "| trace | T | total us | router_topk | gather | expert_projection | scatter_combine | shared expert "
             "| shared us | routed us | excluded us | shared fraction | gates |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for path in results:
        r = json.load(open(path))
        st = {k: v["wall_ns"] / 1e3 for k, v in r["stages"].items()}
        shared = sum(v for k, v in st.items() if k.startswith("shared_expert"))
        sp = r["shared_vs_routed"]
        tr = r["trace"]
        lines.append(f"| {tr['model']['name']} ({tr['source']}) | {tr['tokens']} | {r['total_profiled_ns'] / 1e3:.1f} "
                     f"| {st.get('router_topk', 0):.1f} | {st.get('gather', 0):.1f} "
                     f"| {st.get('expert_projection', 0):.1f} | {st.get('scatter_combine', 0):.1f} | {shared:.1f} "
                     f"| {sp['shared_ns'] / 1e3:.1f} | {sp['routed_ns'] / 1e3:.1f} | {sp['excluded_ns'] / 1e3:.1f} "
                     f"| {sp['shared_fraction']:.3f} | {'pass' if r['gates_pass'] else 'FAIL'} |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def marker(marker_csv: str, kernel_csv: str, out_md: str, command: str) -> None:
    """Counts of the roctx ranges (stage names) and of the kernels in one marker + kernel trace."""
    ranges = collections.Counter(r.get("Function") or r.get("Message") for r in csv.DictReader(open(marker_csv))
                                 if "RANGE" in r.get("Domain", ""))
    kernels = collections.Counter(short(r["Kernel_Name"]) for r in csv.DictReader(open(kernel_csv)))
    lines = ["# rocprofv3 marker trace of a route-trace replay", "", f"Command: `{command}`", "",
             "| roctx range (stage) | count |", "|---|---|"]
    lines += [f"| {k} | {v} |" for k, v in sorted(ranges.items())]
    lines += ["", "| kernel | dispatches |", "|---|---|"]
    lines += [f"| {k} | {v} |" for k, v in sorted(kernels.items()) if "at::" not in k]
    open(out_md, "w").write("\n".join(lines) + "\n")


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "replay":
        replay(sys.argv[2], sys.argv[3], sys.argv[4:])
        sys.exit(0)
    if mode == "marker":
        marker(sys.argv[2], sys.argv[3], sys.argv[4], " ".join(sys.argv[5:]))
        sys.exit(0)
    if mode == "sq":  # sq <out.md> <dir> [<dir> ...] -- <command...>
        cut = sys.argv.index("--")
        sq(sys.argv[2], " ".join(sys.argv[cut + 1:]), sys.argv[3:cut])
        sys.exit(0)
    if mode == "bandwidth":  # bandwidth <kernel_trace.csv> <out.md> <command...>
        bandwidth(sys.argv[2], sys.argv[3], " ".join(sys.argv[4:]))
        sys.exit(0)
    if mode == "trace":
        trace(sys.argv[2], sys.argv[3], sys.argv[4], " ".join(sys.argv[5:]))
    elif mode == "pmc":
        pmc(sys.argv[2], sys.argv[3], float(sys.argv[4]), sys.argv[5], sys.argv[6], " ".join(sys.argv[7:]))
    else:
        raise SystemExit(__doc__)
