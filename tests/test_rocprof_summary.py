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
