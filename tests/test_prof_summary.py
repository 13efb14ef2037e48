"""Host logic of the rocprofv3 summarizer on small hand-made CSV files: durations
of the timed dispatches, counter scaling by the 1 GiB copy, and the add kernels'
GB/s against their algorithmic bytes."""
import csv
import json

import pytest

from hgemm_strassen_type_amd import prof_summary

GIB = 1024 ** 3


def write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def trace_rows(spec):
    """spec: list of (kernel name, duration in ns); consecutive timestamps."""
    rows, t = [], 1000
    for name, ns in spec:
        rows.append([name, t, t + ns])
        t += ns + 100
    return rows


def counter_rows(counter, spec):
    return [[name, counter, v] for name, v in spec]


def test_adds_summary(tmp_path):
    # 2 warmup steps + 2 timed steps; per step: two pre-adds, one post-add
    spec = []
    for step, (pre_ns, post_ns) in enumerate([(9e6, 9e6), (9e6, 9e6), (250e3, 500e3),
                                             (270e3, 500e3)]):
        spec += [("preadd_kernel(x)", int(pre_ns)), ("preadd_kernel(x)", int(pre_ns)),
                 ("gemm_mfma_kernel<...>", 5000000), ("postadd_kernel(y)", int(post_ns))]
    write_csv(tmp_path / "trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
              trace_rows(spec))
    # the copy reads half its bytes per counted byte (scale 2) and writes 1:1
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    write_csv(tmp_path / "fetch.csv", hdr, counter_rows("FETCH_SIZE", [
        ("__amd_rocclr_copyBuffer", GIB / 1024 / 2), ("preadd_kernel(x)", 200000.0),
        ("preadd_kernel(x)", 200000.0), ("postadd_kernel(y)", 700000.0)]))
    write_csv(tmp_path / "write.csv", hdr, counter_rows("WRITE_SIZE", [
        ("__amd_rocclr_copyBuffer", GIB / 1024), ("preadd_kernel(x)", 100000.0),
        ("preadd_kernel(x)", 100000.0), ("postadd_kernel(y)", 200000.0)]))
    info = {"workload": "w", "steps": 2, "warmup": 2, "ms_per_step": 1.0,
            "effective_tflops": 1.0, "launches_per_step": {"preadd_kernel": 2, "postadd_kernel": 1},
            "alg_bytes_per_launch": {"preadd_kernel": 512000000, "postadd_kernel": 1638400000}}
    (tmp_path / "bench.log").write_text("[bench] x\n" + json.dumps(info) + "\n")
    out = tmp_path / "out.md"
    prof_summary.adds(str(tmp_path / "trace.csv"), str(tmp_path / "fetch.csv"),
                      str(tmp_path / "write.csv"), str(tmp_path / "bench.log"), str(out), "cmd")
    rows = {line.split("|")[1].strip(): [c.strip() for c in line.split("|")[2:-1]]
            for line in out.read_text().splitlines() if line.startswith("| `")}
    pre, post = rows["`preadd_kernel`"], rows["`postadd_kernel`"]
    # timed pre-adds: 250, 250, 270, 270 us -> 260 us; 512 MB / 260 us = 1969 GB/s
    assert pre[0] == "4" and float(pre[1]) == pytest.approx(260.0)
    assert float(pre[3]) == pytest.approx(512e6 / 260e-6 / 1e9, abs=1)
    assert float(post[1]) == pytest.approx(500.0) and float(post[3]) == pytest.approx(3277, abs=1)
    # counters: pre-add 2*200000 KiB read + 100000 KiB written = 500000 KiB
    assert float(pre[5]) == pytest.approx(500000 * 1024, rel=1e-3)
    assert float(post[5]) == pytest.approx(1600000 * 1024, rel=1e-3)
    assert float(post[6]) == pytest.approx(1600000 * 1024 / 1638400000, abs=1e-3)


def test_traffic_record(tmp_path):
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    write_csv(tmp_path / "fetch.csv", hdr, counter_rows("FETCH_SIZE", [
        ("__amd_rocclr_copyBuffer", GIB / 1024 / 2), ("gemm_mfma_kernel<A>", 1000.0),
        ("gemm_mfma_kernel<A>", 3000.0)]))
    write_csv(tmp_path / "write.csv", hdr, counter_rows("WRITE_SIZE", [
        ("__amd_rocclr_copyBuffer", GIB / 1024), ("gemm_mfma_kernel<A>", 500.0)]))
    out = tmp_path / "t.json"
    prof_summary.traffic(str(tmp_path / "fetch.csv"), str(tmp_path / "write.csv"), str(out),
                         "gemm_mfma_kernel", "cmd")
    rec = json.loads(out.read_text())
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["bytes_per_launch"] == pytest.approx(2000 * 1024 * 2 + 500 * 1024)
    assert len(rec["kernel_hash"]) == 16


def test_clock_summary(tmp_path):
    # 8 XCDs summing 8 * 1.5e6 cycles over 1000 us: 1.5 GHz; 1.05e12 FLOP on 256 CUs at
    # 4096 FLOP/clock/CU needs ~1.0014e6 cycles, so the MFMA pipes are busy ~0.668
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
           "End_Timestamp"]
    rows = [["7", "gemm_mfma_kernel<TileCfg<256, 256,...>", "GRBM_GUI_ACTIVE", 12.0e6, 1000, 1001000],
            ["7", "gemm_mfma_kernel<TileCfg<256, 256,...>", "SQ_WAVES", 2048, 1000, 1001000],
            ["8", "other_kernel", "GRBM_GUI_ACTIVE", 1.0, 0, 10]]
    write_csv(tmp_path / "pmc.csv", hdr, rows)
    out = tmp_path / "c.md"
    prof_summary.clock(str(tmp_path / "pmc.csv"), str(out), "cmd", "TileCfg<256, 256", 1.05e12)
    line = [l for l in out.read_text().splitlines() if l.startswith("| 7 |")][0]
    cells = [c.strip() for c in line.split("|")[1:-1]]
    assert float(cells[1]) == pytest.approx(1000.0)
    assert float(cells[4]) == pytest.approx(1.5)
    assert float(cells[5]) == pytest.approx(1.05e12 / (256 * 4096) / 1.5e6, abs=1e-3)
    assert float(cells[6]) == pytest.approx(1050, abs=1)
    assert "| 8 |" not in out.read_text()


def test_timeline_of_the_last_call(tmp_path):
    """Two calls on two queues: the second call's kernels, with the product batch that
    started on the other queue just before its first kernel, at times relative to
    that kernel; workgroups from the grid and workgroup sizes."""
    header = ["Kernel_Name", "Queue_Id", "Start_Timestamp", "End_Timestamp", "Grid_Size_X",
              "Workgroup_Size_X", "Grid_Size_Y", "Workgroup_Size_Y"]
    rows = []
    for base in (0, 100000):
        rows += [["gemm_mfma_kernel<P1P2>", 2, base + 9000, base + 40000, 224 * 512, 512, 1, 1],
                 ["maxabs_kernel(a)", 1, base + 10000, base + 13000, 8 * 256, 256, 4, 1],
                 ["preadd_kernel(a)", 1, base + 13000, base + 30000, 4 * 256, 256, 8192, 1],
                 ["gemm_mfma_kernel<P3P7>", 2, base + 41000, base + 90000, 256 * 512, 512, 1, 1],
                 ["postadd_kernel(c)", 2, base + 90000, base + 95000, 32 * 256, 256, 8192, 1]]
    write_csv(tmp_path / "t.csv", header, rows)
    out = tmp_path / "t.md"
    prof_summary.timeline(str(tmp_path / "t.csv"), str(out), "cmd", "maxabs", "test")
    text = out.read_text()
    body = [l for l in text.splitlines() if l.startswith("| ") and not l.startswith("| start")]
    assert len(body) == 5
    assert body[0].startswith("| -1.0 | 30.0 | 31.0 | 2 | 224 | `gemm_mfma_kernel<P1P2>`")
    assert body[1].startswith("| 0.0 | 3.0 | 3.0 | 1 | 32 |")
    assert body[4].startswith("| 80.0 | 85.0 | 5.0 | 2 | 262144 |")
    assert "Call span: 86.0 us" in text
    # a first kernel launched twice per call: the earlier of the last call's two
    rows2 = [r for r in rows]
    rows2.insert(2, ["maxabs_kernel(b)", 1, 100000 + 13000, 100000 + 13000, 8 * 256, 256, 4, 1])
    write_csv(tmp_path / "t2.csv", header, rows2)
    prof_summary.timeline(str(tmp_path / "t2.csv"), str(out), "cmd", "maxabs", "test", per_call=2)
    assert "| 0.0 | 3.0 | 3.0 | 1 | 32 |" in out.read_text()


def test_stall_breakdown(tmp_path):
    # two --pmc runs of one command; the first dispatch of each is left out.  Run 1:
    # 2048 waves living 1.0e6 cycles each (SQ_WAVE_CYCLES in quad-cycles), 30 % of
    # them issuing, 50 % ready but not issued, 20 % waiting; 8 XCDs at 1.5e6 cycles.
    # Run 2 took 1.2x the cycles, so its wave-cycle counters are scaled by 1/1.2.
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    k = "gemm_mfma_kernel<TileCfg<256, 256,...>"
    wc = 2048 * 1.0e6 / 4
    run1 = []
    for d, f in (("1", 3.0), ("2", 1.0), ("3", 1.0)):      # dispatch 1: a different state
        run1 += [[d, k, "GRBM_GUI_ACTIVE", 8 * 1.5e6 * f], [d, k, "SQ_WAVE_CYCLES", wc * f],
                 [d, k, "SQ_ACTIVE_INST_ANY", 0.3 * wc * f], [d, k, "SQ_WAIT_INST_ANY", 0.5 * wc * f],
                 [d, k, "SQ_WAIT_ANY", 0.2 * wc * f], [d, k, "SQ_INSTS_MFMA", 2048 * 6400.0]]
    run1.append(["4", "other_kernel", "SQ_WAVE_CYCLES", 1.0])
    run2 = []
    for d in ("5", "6"):
        run2 += [[d, k, "GRBM_GUI_ACTIVE", 1.2 * 8 * 1.5e6], [d, k, "SQ_WAVES", 2048],
                 [d, k, "SQ_WAIT_INST_LDS", 1.2 * 0.05 * wc], [d, k, "SQ_INSTS_LDS", 2048 * 4000.0],
                 [d, k, "SQ_LDS_IDX_ACTIVE", 256 * 0.25 * 1.2 * 1.5e6],
                 [d, k, "SQ_LDS_BANK_CONFLICT", 0]]
    write_csv(tmp_path / "a.csv", hdr, run1)
    write_csv(tmp_path / "b.csv", hdr, run2)
    out = tmp_path / "s.md"
    flops = 0.7 * 1.5e6 * 256 * 4096
    prof_summary.stalls([str(tmp_path / "a.csv"), str(tmp_path / "b.csv")], str(out),
                        "cmd1 && cmd2", "TileCfg<256, 256", flops, phases_per_wave=100)
    text = out.read_text()

    def row(label):
        line = [l for l in text.splitlines() if l.startswith(f"| {label}")][0]
        return float(line.split("|")[-2])
    assert "**MFMA busy 0.700**" in text
    assert row("issuing (SQ_ACTIVE_INST_ANY)") == pytest.approx(0.3)
    assert row("ready, not issued (SQ_WAIT_INST_ANY)") == pytest.approx(0.5)
    assert row("waiting on a counter or the barrier") == pytest.approx(0.2)
    assert row("  LDS instruction ready, not issued") == pytest.approx(0.05)
    assert "LDS busy (SQ_LDS_IDX_ACTIVE per CU over the launch's cycles): 0.250" in text
    assert row("MFMA |") == pytest.approx(64.0)
    assert row("LDS |") == pytest.approx(40.0)
    assert "cmd2" in text


def test_stall_breakdown_picks_one_shape(tmp_path):
    # one kernel run at two shapes: the MOPS counter tells them apart, so the
    # medians come from the 1e12-FLOP launches only (the first of them left out)
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    k = "gemm_mfma_kernel<TileCfg<256, 256, 2, 2, 64, 2, 1, 32>, 12, true>"
    rows = []
    for d, fl, cyc in (("1", 1e12, 9e6), ("2", 1e12, 8e6), ("3", 1e12, 8e6), ("4", 5e11, 4e6),
                       ("5", 5e11, 4e6)):
        rows += [[d, k, "GRBM_GUI_ACTIVE", cyc], [d, k, "SQ_WAVE_CYCLES", cyc / 4],
                 [d, k, "SQ_WAIT_ANY", 0.25 * cyc / 4], [d, k, "SQ_WAVES", 1024],
                 [d, k, "SQ_INSTS_VALU_MFMA_MOPS_F6F4", fl / 512]]
    write_csv(tmp_path / "a.csv", hdr, rows)
    out = tmp_path / "s.md"
    prof_summary.stalls([str(tmp_path / "a.csv")], str(out), "cmd", ", 12, true", 1e12,
                        flop_per_clk_cu=16384.0)
    text = out.read_text()
    # 1e12 FLOP at 16384 FLOP/clock on 256 CUs over 1e6 cycles per XCD
    assert f"**MFMA busy {1e12 / (256 * 16384) / 1e6:.3f}**" in text
    assert "SQ_INSTS_VALU_MFMA_MOPS_F6F4 × 512: 1e+12 FLOP" in text
    assert "| waiting on a counter or the barrier (SQ_WAIT_ANY) | 0.250 |" in text
