"""The rocprofv3 summary tool (profiles/ are made with it, and bench.py reads
the short-window kernel's HBM bytes back from its output): duration
clustering, the HBM bytes derived from the per-size request counters, and the
kernel-source hash check.  Synthetic CSV files, no GPU."""
import csv

import pytest

from hyper_connection_residual_amd import rocprof_summary as rs


def _write_trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"])
        t = 0
        for name, wgs, us in rows:
            w.writerow([name, wgs * 256, 256, t, t + int(us * 1000)])
            t += 100000


def _table(md):
    return [r for r in md.splitlines() if r.startswith("| hc::")]


def test_trace_keeps_a_single_outlier_in_its_group(tmp_path):
    p = tmp_path / "trace.csv"
    _write_trace(p, [("void hc::(anonymous namespace)::decode_kernel<8>(int)", 256, us)
                     for us in (9.0, 9.2, 9.1, 9.3, 27.5)])
    rows = _table(rs.trace(str(p)))
    assert len(rows) == 1
    cells = [c.strip() for c in rows[0].split("|")]
    assert cells[1] == "hc::decode_kernel<8>" and cells[3] == "5"
    assert float(cells[5]) == pytest.approx(9.2)   # median
    assert float(cells[9]) == pytest.approx(27.5)  # max


def test_trace_splits_a_kernel_run_at_two_sizes(tmp_path):
    p = tmp_path / "trace.csv"
    _write_trace(p, [("hc::prefill_upmix3<false>", 256, us) for us in (44.0, 45.0, 44.5, 170.0, 172.0, 171.0)])
    rows = _table(rs.trace(str(p)))
    assert len(rows) == 2
    assert any("(size 1 of 2)" in r and "| 3 |" in r for r in rows)
    assert any("(size 2 of 2)" in r and "| 3 |" in r for r in rows)


def _write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name", "Counter_Value"])
        for d, name, counters in rows:
            for c, v in counters.items():
                w.writerow([d, name, 256 * 512, 512, c, v])


def test_counters_derive_bytes_and_report_the_sweep_with_its_hash(tmp_path):
    log = tmp_path / "run.log"
    log.write_text("# kernel source hash: 0123456789abcdef\n")
    p = tmp_path / "pmc.csv"
    rd = {"TCC_EA0_RDREQ_32B_sum": 10, "TCC_EA0_RDREQ_64B_sum": 20, "TCC_EA0_RDREQ_128B_sum": 1000}
    wr = {"TCC_EA0_WRREQ_sum": 30, "TCC_EA0_WRREQ_64B_sum": 10}
    _write_counters(p, [(1, "hc::decode_kernel<1>", {**rd, **wr}), (2, "hc::decode_kernel<1>", {**rd, **wr})])
    md = rs.counters([str(log)], [str(p)])
    read = 32 * 10 + 64 * 20 + 128 * 1000
    written = 64 * 10 + 32 * (30 - 10)
    assert "read %.3f MB" % (read / 1e6) in md
    assert "written %.3f MB" % (written / 1e6) in md
    out = tmp_path / "counters.md"
    out.write_text(md)
    assert rs.read_traffic(str(out)) == (read + written, "0123456789abcdef")


def test_counters_refuse_runs_of_different_sources(tmp_path):
    a, b = tmp_path / "a.log", tmp_path / "b.log"
    a.write_text("# kernel source hash: 1111111111111111\n")
    b.write_text("# kernel source hash: 2222222222222222\n")
    p = tmp_path / "pmc.csv"
    _write_counters(p, [(1, "hc::decode_kernel<1>", {"TCC_EA0_RDREQ_sum": 1})])
    with pytest.raises(SystemExit):
        rs.counters([str(a), str(b)], [str(p)])
