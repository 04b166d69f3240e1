"""The rocprofv3 summaries behind profiles/ (block_dequant_gemv_amd.prof), on
small hand-written CSV files in rocprofv3's column layout (no GPU needed)."""
import os

from block_dequant_gemv_amd import prof


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write(",".join(header) + "\n")
        for r in rows:
            f.write(",".join(str(v) for v in r) + "\n")


def test_trace_summary_groups_by_launch_shape_and_skips_warmup(tmp_path):
    hdr = ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"]
    rows = []
    # kernel A, 100 workgroups of 256: durations 10, 20 (warm-up) then 5 x 1 us
    for i, d in enumerate([10, 20, 1, 1, 1, 1, 1]):
        rows.append(["void qgk::a<1>(int)", 25600, 256, 1000 * i, 1000 * i + 1000 * d])
    # the same kernel on another grid is its own row
    rows.append(["void qgk::a<1>(int)", 512, 256, 50000, 52000])
    _write(str(tmp_path / "t" / "run_kernel_trace.csv"), hdr, rows)
    full = prof.trace_summary(str(tmp_path / "t"))
    assert "qgk::a<1>" in full and "(int)" not in full
    line = [ln for ln in full.splitlines() if " 100 " in ln][0].split()
    assert line[3] == "7" and abs(float(line[4]) - 35 / 7) < 0.01
    skipped = prof.trace_summary(str(tmp_path / "t"), skip=2)
    line = [ln for ln in skipped.splitlines() if " 100 " in ln][0].split()
    assert line[3] == "5" and float(line[4]) == 1.0 and float(line[5]) == 1.0
    assert not [ln for ln in skipped.splitlines() if ln.split()[1:2] == ["2"]]   # 1 dispatch, skipped
    # the last 3 dispatches of every shape: A's 1 us launches, and the other grid's single one
    tail = prof.trace_summary(str(tmp_path / "t"), tail=3)
    line = [ln for ln in tail.splitlines() if " 100 " in ln][0].split()
    assert line[3] == "3" and float(line[4]) == 1.0
    line = [ln for ln in tail.splitlines() if ln.split()[1:3] == ["2", "256"]][0].split()
    assert line[3] == "1" and float(line[4]) == 2.0


def test_counter_summary_derives_clock_and_valu_per_wave(tmp_path):
    hdr = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name", "Counter_Value",
           "Start_Timestamp", "End_Timestamp"]
    rows = []
    for did in (1, 2):
        for c, v in (("GRBM_GUI_ACTIVE", 200000), ("SQ_WAVES", 4000), ("SQ_INSTS_VALU", 1200000)):
            rows.append([did, "qgk::k", 256000, 256, c, v, 0, 100000])   # 100 us each
    _write(str(tmp_path / "c" / "run_counter_collection.csv"), hdr, rows)
    text = prof.counter_summary(str(tmp_path / "c"))
    line = [ln for ln in text.splitlines() if ln.startswith("qgk::k")][0].split()
    # wgs 1000, wg 256, n 2, 100 us; clock 200000 / 8 XCDs / 100 = 250 (cycles per us); 1200000 / 4000 = 300
    # waves' instructions; VALU busy 1200000 * 4 / (1024 * 25000) = 0.1875
    assert line[1:5] == ["1000", "256", "2", "100.00"]
    assert float(line[-3]) == 250.0 and float(line[-2]) == 300.0 and abs(float(line[-1]) - 0.1875) < 1e-3


def test_counter_summary_adds_hbm_rate_from_traffic(tmp_path):
    # the same counter run as above, with the traffic run's 8 MB per dispatch of that
    # launch shape (and an entry for a shape this run does not have)
    hdr = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name", "Counter_Value",
           "Start_Timestamp", "End_Timestamp"]
    rows = []
    for did in (1, 2):
        for c, v in (("GRBM_GUI_ACTIVE", 200000), ("SQ_WAVES", 4000), ("SQ_INSTS_VALU", 1200000)):
            rows.append([did, "qgk::k", 256000, 256, c, v, 0, 100000])   # 100 us each
    rows.append([3, "qgk::other", 2560, 256, "GRBM_GUI_ACTIVE", 80000, 0, 10000])
    _write(str(tmp_path / "c" / "run_counter_collection.csv"), hdr, rows)
    traffic = {"kernels": {"qgk::k|1000x256": {"fetch_bytes": 7.5e6, "write_bytes": 0.5e6},
                           "qgk::absent|4x64": {"fetch_bytes": 1.0, "write_bytes": 0.0}}}
    hbm = prof.shape_bytes(traffic)
    assert hbm == {("qgk::k", 1000, 256): 8.0e6, ("qgk::absent", 4, 64): 1.0}
    text = prof.counter_summary(str(tmp_path / "c"), hbm)
    assert "hbm_B_per_clk" in text
    line = [ln for ln in text.splitlines() if ln.startswith("qgk::k")][0].split()
    # 8 MB in 100 us = 80 GB/s; 8e6 bytes over 200000 / 8 = 25000 clocks = 320 bytes per clock
    assert float(line[-2]) == 80.0 and float(line[-1]) == 320.0
    other = [ln for ln in text.splitlines() if ln.startswith("qgk::other")][0].split()
    assert other[-2:] == ["-", "-"]
    # without traffic data the columns are not there
    assert "hbm_GBps" not in prof.counter_summary(str(tmp_path / "c"))
