"""Summaries of rocprofv3 output for the profiles/ folder.

    python -m hgemm_strassen_type_amd.prof_summary stats <kernel_stats.csv> <out.md> "<command>"
        [<kernel_trace.csv> "<kernel substring>" <warmup dispatches> <bench stdout log>]
    python -m hgemm_strassen_type_amd.prof_summary traffic <fetch.csv> <write.csv> <out.json>
        "<kernel substring>" "<command>"

    python -m hgemm_strassen_type_amd.prof_summary clock <pmc.csv> <out.md> "<command>"
        "<kernel substring>" <FLOP per launch>
    python -m hgemm_strassen_type_amd.prof_summary adds <kernel_trace.csv> <fetch.csv>
        <write.csv> <bench stdout log> <out.md> "<commands>"
    python -m hgemm_strassen_type_amd.prof_summary timeline <kernel_trace.csv> <out.md>
        "<command>" "<first kernel substring>" "<title>" [<its launches per call>]
    python -m hgemm_strassen_type_amd.prof_summary stalls <pmc1.csv,pmc2.csv,...> <out.md>
        "<commands joined by ' && '>" "<kernel substring>" <FLOP per launch> [<phases a wave>
        [<FLOP per clock per CU at the MFMA's full rate: 4096 for 16-bit, 16384 for 4-bit>]]

`stats` keeps the per-kernel call count and average/min/max duration of a
`--kernel-trace --stats` run.  `traffic` turns two `--pmc FETCH_SIZE` /
`--pmc WRITE_SIZE` runs (KiB per dispatch) into HBM bytes per launch of the
named kernel, each scaled by what the same counter reads for the 1 GiB device
copy that `bench.py --copy-calib` runs in the same process (read 1 GiB, write
1 GiB), and records the GEMM kernel sources' hash so a stale record is ignored.
`adds` does the same for the Strassen add kernels of `bench.py --only-adds` (and
for the decode kernel of `bench.py --only-decode`, whose JSON line has the same keys): per
kernel, the average duration of the timed dispatches, the algorithmic bytes that
bench.py states, the GB/s they make against the 8 TB/s HBM peak, and the
counters' bytes per launch next to the algorithmic ones.  `timeline` lists the
kernels of the last call of a trace (start, end, queue, workgroups), which shows
what runs concurrently on two streams.  `stalls` splits a GEMM kernel's wave cycles
into issuing, ready-but-not-issued and waiting, from SQ counters taken in several
--pmc runs of one command, with LDS occupancy and the instruction mix.
"""
from __future__ import annotations

import csv
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GIB = 1024 ** 3


def _short(name: str, width: int = 120) -> str:
    return name if len(name) <= width else name[:width - 3] + "..."


def stats(csv_path: str, out_md: str, command: str, trace_csv: str | None = None,
          kernel: str | None = None, skip: int = 0, bench_log: str | None = None) -> None:
    rows = list(csv.DictReader(open(csv_path)))
    lines = ["# rocprofv3 kernel statistics", "", "Command:", "", "```", command, "```", "",
             "| kernel | calls | avg us | min us | max us | share % |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    if trace_csv and kernel:
        # the launches of bench.py's timed region: all dispatches after the warmup ones
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
             for r in csv.DictReader(open(trace_csv)) if kernel in r["Kernel_Name"]]
        timed = d[skip:]
        lines += ["", f"Timed region ({len(timed)} dispatches after {skip} warmup ones) of "
                      f"`{kernel}`: average {statistics.mean(timed):.2f} us "
                      f"(min {min(timed):.2f}, max {max(timed):.2f})."]
        if bench_log:
            for line in open(bench_log):
                if line.startswith("{"):
                    ms = json.loads(line)["ms_per_step"]
                    lines.append(f"bench.py's own HIP-event timing of the same launches in that "
                                 f"run: {ms * 1e3:.2f} us per step.")
    open(out_md, "w").write("\n".join(lines) + "\n")


def _per_kernel(csv_path: str, counter: str):
    vals = {}
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


def _kernel_hash() -> str:
    sys.path.insert(0, ROOT)
    import bench  # noqa: E402  (the hash bench.py compares against)
    return bench.kernel_hash()


def traffic(fetch_csv: str, write_csv: str, out_json: str, kernel: str, command: str) -> None:
    fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
    write = _per_kernel(write_csv, "WRITE_SIZE")

    def pick(d, sub):
        keys = [k for k in d if sub in k]
        if not keys:
            raise SystemExit(f"no kernel matching {sub!r}")
        return statistics.mean(d[keys[0]]), keys[0]

    f_k, name = pick(fetch, kernel)
    w_k, _ = pick(write, kernel)
    f_c, _ = pick(fetch, "copyBuffer")
    w_c, _ = pick(write, "copyBuffer")
    f_scale = GIB / (f_c * 1024.0)   # true bytes per counted byte
    w_scale = GIB / (w_c * 1024.0)
    rec = {"kernel": name, "kernel_hash": _kernel_hash(),
           "fetch_kib_raw": f_k, "write_kib_raw": w_k,
           "copy_fetch_kib_raw": f_c, "copy_write_kib_raw": w_c,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "fetch_bytes": f_k * 1024.0 * f_scale, "write_bytes": w_k * 1024.0 * w_scale,
           "command": command}
    rec["bytes_per_launch"] = rec["fetch_bytes"] + rec["write_bytes"]
    json.dump(rec, open(out_json, "w"), indent=1)
    md = os.path.splitext(out_json)[0] + ".md"
    open(md, "w").write(
        "# HBM traffic of the GEMM kernel (rocprofv3 --pmc)\n\n"
        f"Kernel: `{_short(name)}`\n\nCommands:\n\n```\n{command}\n```\n\n"
        "| counter | kernel KiB/launch (raw) | 1 GiB copy KiB (raw) | scale | bytes/launch |\n"
        "|---|---|---|---|---|\n"
        f"| FETCH_SIZE | {f_k:.0f} | {f_c:.0f} | {f_scale:.3f} | {rec['fetch_bytes']:.4g} |\n"
        f"| WRITE_SIZE | {w_k:.0f} | {w_c:.0f} | {w_scale:.3f} | {rec['write_bytes']:.4g} |\n\n"
        f"Total HBM bytes per launch: {rec['bytes_per_launch']:.4g}\n")


def adds(trace_csv: str, fetch_csv: str, write_csv: str, bench_log: str, out_md: str,
         command: str, peak_gbps: float = 8000.0,
         title: str = "the Strassen add kernels") -> None:
    info = None
    for line in open(bench_log):
        if line.startswith("{"):
            info = json.loads(line)
    if info is None:
        raise SystemExit("no JSON line in " + bench_log)
    fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
    write = _per_kernel(write_csv, "WRITE_SIZE")

    def mean_of(d, sub):
        keys = [k for k in d if sub in k]
        if not keys:
            raise SystemExit(f"no kernel matching {sub!r}")
        return statistics.mean(v for k in keys for v in d[k])

    f_scale = GIB / (mean_of(fetch, "copyBuffer") * 1024.0)
    w_scale = GIB / (mean_of(write, "copyBuffer") * 1024.0)
    trace = list(csv.DictReader(open(trace_csv)))
    lines = [f"# HBM rate of {title} (rocprofv3)", "",
             f"Workload: {info['workload']}; {info['steps']} timed steps after "
             f"{info['warmup']} warmup ones, {info['ms_per_step']} ms per step "
             f"({info['effective_tflops']} effective TFLOP/s).", "", "Commands:", "", "```",
             command, "```", "",
             "| kernel | timed launches | avg us | algorithmic bytes | GB/s | of 8 TB/s "
             "| counter bytes/launch | counter / algorithmic |",
             "|---|---|---|---|---|---|---|---|"]
    for k, alg in info["alg_bytes_per_launch"].items():
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
             for r in trace if k in r["Kernel_Name"]]
        timed = d[info["warmup"] * info["launches_per_step"][k]:]
        us = statistics.mean(timed)
        gbps = alg / (us * 1e-6) / 1e9
        hbm = mean_of(fetch, k) * 1024.0 * f_scale + mean_of(write, k) * 1024.0 * w_scale
        lines.append(f"| `{k.rstrip(',')}` | {len(timed)} | {us:.2f} | {alg:.4g} | {gbps:.0f} | "
                     f"{gbps / peak_gbps:.3f} | {hbm:.4g} | {hbm / alg:.3f} |")
    lines += ["", f"Counter scale from the 1 GiB copy in the same process: FETCH_SIZE x{f_scale:.3f}, "
                  f"WRITE_SIZE x{w_scale:.3f}. Both counter runs average over every dispatch of a "
                  "kernel" + (" (the two pre-add launches move the same bytes on this square shape)."
                              if "preadd_kernel" in info["alg_bytes_per_launch"] else ".")]
    # the copy's own rate in the counter runs (2 GiB moved per launch), where timed
    copy_us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
               for path in (fetch_csv, write_csv) for r in csv.DictReader(open(path))
               if "copyBuffer" in r["Kernel_Name"] and r.get("Start_Timestamp")]
    if copy_us:
        rates = [2 * GIB / (u * 1e-6) / 1e12 for u in copy_us]
        lines += ["", f"For comparison, the runtime's 1 GiB device copy (2 GiB moved per launch) in "
                      f"the same counter runs: {min(copy_us):.0f}-{max(copy_us):.0f} us, "
                      f"{min(rates):.1f}-{max(rates):.1f} TB/s."]
    open(out_md, "w").write("\n".join(lines) + "\n")


def clock(pmc_csv: str, out_md: str, command: str, kernel: str, flops: float, cus: int = 256,
          xcds: int = 8, flop_per_clk_cu: float = 4096.0) -> None:
    """Clock held and MFMA occupancy of a GEMM kernel from GRBM_GUI_ACTIVE (GPU cycles
    while busy, summed over the XCDs): per dispatch, cycles per XCD / duration is the
    clock; the cycles the MFMA work needs at full rate (flops / (cus * flop_per_clk_cu))
    over the cycles taken is the fraction of cycles the MFMA pipes had work."""
    per = {}
    for r in csv.DictReader(open(pmc_csv)):
        if kernel not in r["Kernel_Name"]:
            continue
        d = per.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"]})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    if not per:
        raise SystemExit(f"no kernel matching {kernel!r}")
    need = flops / (cus * flop_per_clk_cu)
    name = next(iter(per.values()))["name"]
    lines = ["# Clock and MFMA occupancy of the GEMM kernel (rocprofv3 --pmc)", "",
             f"Kernel: `{_short(name)}`", "", "Command:", "", "```", command, "```", "",
             f"MFMA work per launch: {flops:.4g} FLOP = {need / 1e6:.3f} M cycles per CU at "
             f"{flop_per_clk_cu:.0f} FLOP/clock/CU (dense 16-bit) on {cus} CUs.", "",
             "| dispatch | us | GRBM_GUI_ACTIVE (sum of XCDs) | cycles per XCD | clock GHz "
             "| MFMA busy | TFLOP/s |", "|---|---|---|---|---|---|---|"]
    for k in sorted(per, key=int):
        d = per[k]
        cyc = d["GRBM_GUI_ACTIVE"] / xcds
        lines.append(f"| {k} | {d['us']:.1f} | {d['GRBM_GUI_ACTIVE']:.4g} | {cyc / 1e6:.3f} M | "
                     f"{cyc / (d['us'] * 1e3):.2f} | {need / cyc:.3f} | "
                     f"{flops / (d['us'] * 1e-6) / 1e12:.0f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def _mops_flops(d: dict):
    """FLOP of a dispatch from whichever SQ_INSTS_VALU_MFMA_MOPS_* counters it holds
    (each counts FLOP / 512), or None."""
    v = [x for n, x in d.items() if n.startswith("SQ_INSTS_VALU_MFMA_MOPS_")]
    return 512.0 * sum(v) if v else None


def _steady_medians(pmc_csv: str, kernel: str, flops: float | None = None) -> dict:
    """Median over the dispatches of `kernel` in one --pmc run, the first one left
    out (it starts from an idle chip at a higher clock), of every counter.  With
    `flops`, dispatches whose MOPS counters show other MFMA work (another shape of the
    same kernel) are left out too."""
    per = {}
    for r in csv.DictReader(open(pmc_csv)):
        if kernel not in r["Kernel_Name"]:
            continue
        d = per.setdefault(int(r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if flops:
        per = {i: d for i, d in per.items()
               if _mops_flops(d) is None or abs(_mops_flops(d) - flops) <= 0.01 * flops}
    if not per:
        raise SystemExit(f"no kernel matching {kernel!r} in {pmc_csv}")
    ids = sorted(per)[1:] or sorted(per)
    names = set().union(*(per[i] for i in ids))
    return {n: statistics.median(per[i][n] for i in ids if n in per[i]) for n in names}


def stalls(pmc_csvs: list, out_md: str, command: str, kernel: str, flops: float,
           phases_per_wave: int = 0, cus: int = 256, xcds: int = 8,
           flop_per_clk_cu: float = 4096.0) -> None:
    """Where a GEMM kernel's wave cycles go, from --pmc runs of the same command
    (each run one counter set; every set holds GRBM_GUI_ACTIVE).  The SQ wave
    counters count quad-cycles summed over all waves: SQ_WAVE_CYCLES is the waves'
    lifetime, split into SQ_ACTIVE_INST_ANY (issuing), SQ_WAIT_INST_ANY (an
    instruction ready but not issued, e.g. behind the SIMD's other wave on the MFMA
    pipe) and SQ_WAIT_ANY (waiting on a counter or the barrier).  A run's wave-cycle
    counters are scaled to the first run by the ratio of GRBM_GUI_ACTIVE.  MFMA busy
    is the cycles the MFMA work needs at full rate over the cycles taken, as in
    `clock`; LDS busy is SQ_LDS_IDX_ACTIVE per CU over the cycles taken.  Dispatches
    whose SQ_INSTS_VALU_MFMA_MOPS_* counters show other work than `flops` (another
    shape of the same kernel in the run) are left out."""
    runs = [_steady_medians(p, kernel, flops) for p in pmc_csvs]
    base = runs[0]
    if "SQ_WAVE_CYCLES" not in base:
        raise SystemExit("the first run must hold SQ_WAVE_CYCLES")
    c = {}
    for r in runs:
        scale = base["GRBM_GUI_ACTIVE"] / r["GRBM_GUI_ACTIVE"]
        for n, v in r.items():
            if n != "GRBM_GUI_ACTIVE" and n not in c:
                c[n] = (v, scale)
    cyc = base["GRBM_GUI_ACTIVE"] / xcds
    waves = c["SQ_WAVES"][0] if "SQ_WAVES" in c else None
    wave_cycles = 4.0 * base["SQ_WAVE_CYCLES"]

    def frac(n):
        v, s = c[n]
        return 4.0 * v * s / wave_cycles

    lines = ["# Where the GEMM kernel's wave cycles go (rocprofv3 --pmc)", "",
             f"Kernel filter: `{kernel}`; medians over each run's dispatches but the first.", "",
             "Commands (one counter set a run):", "", "```", *command.split(" && "), "```", "",
             "| counter | median per dispatch |", "|---|---|"]
    for n in sorted(c):
        lines.append(f"| {n} | {c[n][0]:.4g} |")
    need = flops / (cus * flop_per_clk_cu)
    lines += ["", f"GRBM_GUI_ACTIVE (first run): {base['GRBM_GUI_ACTIVE']:.4g}, {cyc / 1e6:.3f} M "
              f"cycles per XCD; MFMA work {flops:.4g} FLOP needs {need / 1e6:.3f} M cycles per CU at "
              f"{flop_per_clk_cu:.0f} FLOP/clock/CU: **MFMA busy {need / cyc:.3f}**.", ""]
    for n in sorted(c):
        if n.startswith("SQ_INSTS_VALU_MFMA_MOPS_"):
            lines.append(f"MFMA work counted by {n} × 512: {c[n][0] * 512:.4g} FLOP.")
            lines.append("")
    lines += ["| share of the waves' cycles | fraction |", "|---|---|"]
    for n, label in (("SQ_ACTIVE_INST_ANY", "issuing (SQ_ACTIVE_INST_ANY)"),
                     ("SQ_WAIT_INST_ANY", "ready, not issued (SQ_WAIT_INST_ANY)"),
                     ("SQ_WAIT_ANY", "waiting on a counter or the barrier (SQ_WAIT_ANY)"),
                     ("SQ_ACTIVE_INST_LDS", "  of which LDS instructions issuing (SQ_ACTIVE_INST_LDS)"),
                     ("SQ_WAIT_INST_LDS", "  LDS instruction ready, not issued (SQ_WAIT_INST_LDS)"),
                     ("SQ_ACTIVE_INST_VALU", "  VALU and MFMA instructions issuing (SQ_ACTIVE_INST_VALU)"),
                     ("SQ_ACTIVE_INST_SCA", "  scalar instructions issuing (SQ_ACTIVE_INST_SCA)")):
        if n in c:
            lines.append(f"| {label} | {frac(n):.3f} |")
    if waves and "SQ_WAVE_CYCLES" in base:
        lines += ["", f"Waves: {waves:.0f}; lifetime {wave_cycles / waves / 1e6:.3f} M cycles a wave "
                  f"against {cyc / 1e6:.3f} M for the launch."]
    if "SQ_LDS_IDX_ACTIVE" in c:
        lds = c["SQ_LDS_IDX_ACTIVE"][0] * c["SQ_LDS_IDX_ACTIVE"][1] / cus
        lines.append(f"LDS busy (SQ_LDS_IDX_ACTIVE per CU over the launch's cycles): {lds / cyc:.3f}; "
                     f"bank-conflict cycles: {c.get('SQ_LDS_BANK_CONFLICT', (0.0, 1.0))[0]:.4g}.")
    if waves:
        per = [("SQ_INSTS_MFMA", "MFMA"), ("SQ_INSTS_LDS", "LDS"), ("SQ_INSTS_VALU", "VALU (MFMA included)"),
               ("SQ_INSTS_SALU", "SALU"), ("SQ_INSTS_VMEM", "vector memory")]
        have = [(n, l) for n, l in per if n in c]
        if have:
            unit = f"a wave a phase ({phases_per_wave} phases a wave)" if phases_per_wave else "a wave"
            lines += ["", f"| instructions | {unit} |", "|---|---|"]
            for n, l in have:
                v = c[n][0] / waves / (phases_per_wave or 1)
                lines.append(f"| {l} | {v:.1f} |")
    open(out_md, "w").write("\n".join(lines) + "\n")


def timeline(trace_csv: str, out_md: str, command: str, first: str, title: str,
             per_call: int = 1) -> None:
    """The kernels of the last call in a `--kernel-trace` run, in start order, from
    the `per_call`-th last dispatch whose name contains `first` (the call's first
    kernel, which a call launches `per_call` times; kernels
    of that call already running on another queue are included from the latest
    start before it that overlaps it): start and end relative to that dispatch,
    duration, hardware queue and workgroup count."""
    rows = list(csv.DictReader(open(trace_csv)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    marks = [i for i, r in enumerate(rows) if first in r["Kernel_Name"]]
    if not marks:
        raise SystemExit(f"no kernel matching {first!r}")
    i0 = marks[-per_call]
    t0 = int(rows[i0]["Start_Timestamp"])
    # launches of the same call issued on another queue just before it, still running at t0
    lo = i0
    while lo > 0 and int(rows[lo - 1]["End_Timestamp"]) > t0 and \
            rows[lo - 1]["Queue_Id"] != rows[i0]["Queue_Id"]:
        lo -= 1
    lines = [f"# Timeline of one call: {title} (rocprofv3 --kernel-trace)", "", "Command:", "",
             "```", command, "```", "",
             "| start us | end us | us | queue | workgroups | kernel |", "|---|---|---|---|---|---|"]
    end = 0.0
    for r in rows[lo:]:
        s_us = (int(r["Start_Timestamp"]) - t0) / 1e3
        e_us = (int(r["End_Timestamp"]) - t0) / 1e3
        end = max(end, e_us)
        wgs = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
        wgs *= int(r.get("Grid_Size_Y") or 1) // max(1, int(r.get("Workgroup_Size_Y") or 1))
        lines.append(f"| {s_us:.1f} | {e_us:.1f} | {e_us - s_us:.1f} | {r['Queue_Id']} | {wgs} | "
                     f"`{_short(r['Kernel_Name'], 100)}` |")
    first_start = (int(rows[lo]["Start_Timestamp"]) - t0) / 1e3
    lines += ["", f"Call span: {end - first_start:.1f} us from the first start to the last end."]
    open(out_md, "w").write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        extra = sys.argv[5:]
        stats(sys.argv[2], sys.argv[3], sys.argv[4], *(extra[:2]),
              *([int(extra[2])] if len(extra) > 2 else []), *(extra[3:4]))
    elif sys.argv[1] == "traffic":
        traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6])
    elif sys.argv[1] == "clock":
        clock(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], float(sys.argv[6]))
    elif sys.argv[1] == "adds":
        adds(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6], sys.argv[7],
             title=sys.argv[8] if len(sys.argv) > 8 else "the Strassen add kernels")
    elif sys.argv[1] == "stalls":
        stalls(sys.argv[2].split(","), sys.argv[3], sys.argv[4], sys.argv[5], float(sys.argv[6]),
               int(sys.argv[7]) if len(sys.argv) > 7 else 0,
               flop_per_clk_cu=float(sys.argv[8]) if len(sys.argv) > 8 else 4096.0)
    elif sys.argv[1] == "timeline":
        timeline(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6],
                 int(sys.argv[7]) if len(sys.argv) > 7 else 1)
    else:
        raise SystemExit(__doc__)
