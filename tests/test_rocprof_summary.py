"""Host logic of the profile summaries (block_diffusion_draft_amd.rocprof_summary) on
small hand-made rocprofv3 CSV files: per-launch HBM traffic scaled by a copy kernel,
and matrix-core use from MFMA busy cycles over SIMD cycles."""
import csv
import io
import os

import pytest

from block_diffusion_draft_amd import rocprof_summary as rs

FIELDS = ["Correlation_Id", "Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_counters(d, name, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, name + "_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (disp, grid, kern, cname, val) in enumerate(rows):
            w.writerow(dict(Correlation_Id=i, Dispatch_Id=disp, Grid_Size=grid, Kernel_Name=kern,
                            Counter_Name=cname, Counter_Value=val))


def test_traffic_scales_by_copy_kernel(tmp_path):
    # copy of 1 MiB: FETCH_SIZE reads 512 KiB (scale 2), WRITE_SIZE 1024 KiB (scale 1)
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    write_counters(fetch, "fetch", [
        (1, 64, "k_head_stream(args)", "FETCH_SIZE", 100.0),
        (2, 64, "k_head_stream(args)", "FETCH_SIZE", 300.0),
        (3, 8, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 512.0)])
    write_counters(write, "write", [
        (1, 64, "k_head_stream(args)", "WRITE_SIZE", 10.0),
        (2, 64, "k_head_stream(args)", "WRITE_SIZE", 30.0),
        (3, 8, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024.0)])
    r = rs.traffic(fetch, write, "k_head_stream", 1 << 20, copies=1)
    assert r["FETCH_SIZE"]["scale"] == pytest.approx(2.0)
    assert r["WRITE_SIZE"]["scale"] == pytest.approx(1.0)
    # mean fetch 200 KiB x 2 + mean write 20 KiB x 1
    assert r["hbm_bytes_per_launch"] == pytest.approx((400 + 20) * 1024)


def test_mfma_busy_fraction(tmp_path):
    # 1024 SIMDs busy 1/4 of 1000 cycles (GRBM_GUI_ACTIVE summed over 8 XCDs)
    d = str(tmp_path / "m")
    write_counters(d, "mfma", [
        (7, 131072, "void k_gemm_big_dma<256, 256>(BigGemmArgs)", "SQ_VALU_MFMA_BUSY_CYCLES", 256000.0),
        (7, 131072, "void k_gemm_big_dma<256, 256>(BigGemmArgs)", "GRBM_GUI_ACTIVE", 8000.0)])
    out = io.StringIO()
    rs.mfma(d, out=out)
    line = [l for l in out.getvalue().splitlines() if "k_gemm_big_dma" in l][0].split()
    assert float(line[-3]) == pytest.approx(0.25)
    assert float(line[-1]) == pytest.approx(1000.0)


def write_trace(d, rows):
    """rows: (dispatch, kernel, grid x, grid y, start ns, end ns)."""
    os.makedirs(d, exist_ok=True)
    fields = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp",
              "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    with open(os.path.join(d, "t_kernel_trace.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for disp, kern, gx, gy, t0, t1 in rows:
            w.writerow(dict(Kind="KERNEL_DISPATCH", Dispatch_Id=disp, Kernel_Name=kern,
                            Start_Timestamp=t0, End_Timestamp=t1, Grid_Size_X=gx,
                            Grid_Size_Y=gy, Grid_Size_Z=1))


def test_launches_keep_equal_sized_grids_of_different_shape_apart(tmp_path):
    # two launches of one kernel with the same total grid (26112 x 5 = 7680 x 17 = 130560
    # threads) but different shapes; the trace's dispatch ids give each its shape
    k = "void k_q4k_stream<8, 32>(Q4kFusedArgs)"
    fetch, write, sq, tr = (str(tmp_path / x) for x in "fwst")
    write_counters(fetch, "f", [(1, 130560, k, "FETCH_SIZE", 1000.0), (2, 130560, k, "FETCH_SIZE", 500.0),
                                (3, 8, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 512.0)])
    write_counters(write, "w", [(1, 130560, k, "WRITE_SIZE", 0.0), (2, 130560, k, "WRITE_SIZE", 0.0),
                                (3, 8, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024.0)])
    write_counters(sq, "s", [(1, 130560, k, "SQ_WAVES", 2048.0), (2, 130560, k, "SQ_WAVES", 2048.0),
                             (1, 130560, k, "GRBM_GUI_ACTIVE", 8000.0),
                             (2, 130560, k, "GRBM_GUI_ACTIVE", 8000.0)])
    write_trace(tr, [(1, k, 26112, 5, 0, 20000), (2, k, 7680, 17, 30000, 40000),
                     (3, "__amd_rocclr_copyBuffer", 8, 1, 50000, 51000)])
    out = io.StringIO()
    rs.launches(fetch, write, sq, tr, "k_q4k_stream", 1 << 20, copies=1, out=out)
    # columns after the kernel name (which holds spaces): grid, us, hbm_MB, then 6 more
    lines = {l.split()[-9]: l.split()[-9:] for l in out.getvalue().splitlines()[1:]}
    assert set(lines) == {"26112x5", "7680x17"}
    assert float(lines["26112x5"][1]) == pytest.approx(20.0)          # us
    assert float(lines["7680x17"][1]) == pytest.approx(10.0)
    # FETCH_SIZE scaled x 2: 1000 KiB -> 2.048 MB, 500 KiB -> 1.024 MB
    assert float(lines["26112x5"][2]) == pytest.approx(2.048, abs=0.006)
    assert float(lines["7680x17"][2]) == pytest.approx(1.024, abs=0.006)


def test_hbm_lists_every_kernel_by_shape(tmp_path):
    k = "void k_q4k_stream<8, 32>(Q4kFusedArgs)"
    fetch, write, tr = (str(tmp_path / x) for x in "fwt")
    write_counters(fetch, "f", [(1, 130560, k, "FETCH_SIZE", 1000.0), (2, 130560, k, "FETCH_SIZE", 500.0),
                                (3, 8, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 512.0)])
    write_counters(write, "w", [(1, 130560, k, "WRITE_SIZE", 100.0), (2, 130560, k, "WRITE_SIZE", 0.0),
                                (3, 8, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024.0)])
    write_trace(tr, [(1, k, 26112, 5, 0, 20000), (2, k, 7680, 17, 30000, 40000),
                     (3, "__amd_rocclr_copyBuffer", 8, 1, 50000, 51000)])
    out = io.StringIO()
    rs.hbm(fetch, write, tr, "", 1 << 20, copies=1, out=out)
    rows = {l.split()[-6]: l.split()[-6:] for l in out.getvalue().splitlines()[1:]}
    assert set(rows) == {"26112x5x1", "7680x17x1", "8x1x1"}
    # grid, launches, us, fetch MB (x 2), write MB (x 1), GB/s
    assert rows["26112x5x1"][1:5] == ["1", "20.0", "2.05", "0.10"]
    assert rows["7680x17x1"][1:5] == ["1", "10.0", "1.02", "0.00"]
