"""Host tests of the rocprofv3 summary helpers on small synthetic CSV files."""
import json
import sys

import pytest

from binary_basis_lut_amd import rocprof_summary as RS

HDR = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id","Grid_Size","Kernel_Id",'
       '"Kernel_Name","Workgroup_Size","LDS_Block_Size","Scratch_Size","VGPR_Count","Accum_VGPR_Count","SGPR_Count",'
       '"Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"\n')


def pmc_dir(tmp_path, name, rows):
    d = tmp_path / name
    d.mkdir()
    lines = [HDR]
    for disp, kernel, counter, value in rows:
        lines.append(f'{disp},{disp},"Agent 1",1,1,1,64,1,"{kernel}",64,0,0,8,0,16,"{counter}",{value},0,1\n')
    (d / "c_counter_collection.csv").write_text("".join(lines))
    return str(d)


def test_pmc_medians_sum_instances_then_take_the_median(tmp_path):
    # dispatch 1: two instances 10 + 20, dispatch 2: 40, dispatch 3: 5 + 5; another kernel ignored
    d = pmc_dir(tmp_path, "a", [(1, "lut_gemv<4>", "FETCH_SIZE", 10), (1, "lut_gemv<4>", "FETCH_SIZE", 20),
                                (2, "lut_gemv<4>", "FETCH_SIZE", 40), (3, "lut_gemv<4>", "FETCH_SIZE", 5),
                                (3, "lut_gemv<4>", "FETCH_SIZE", 5), (4, "other", "FETCH_SIZE", 1000)])
    med, n, name = RS.pmc_medians(d, "lut_gemv")
    assert n == 3 and name == "lut_gemv<4>" and med["FETCH_SIZE"] == 30
    with pytest.raises(SystemExit):
        RS.pmc_medians(d, "nothing_like_this")


def test_traffic_scales_each_counter_by_the_copy_calibration(tmp_path, monkeypatch):
    k = "lut_gemv<4>"
    fetch = pmc_dir(tmp_path, "f", [(1, k, "FETCH_SIZE", 100)])
    write = pmc_dir(tmp_path, "w", [(1, k, "WRITE_SIZE", 8)])
    # a 1 MiB copy that reads as 512 KiB fetched (scale 2) and 1024 KiB written (scale 1)
    cf = pmc_dir(tmp_path, "cf", [(1, "copyBuffer", "FETCH_SIZE", 512)])
    cw = pmc_dir(tmp_path, "cw", [(1, "copyBuffer", "WRITE_SIZE", 1024)])
    out = tmp_path / "t.json"
    monkeypatch.setattr(sys, "argv", ["x", "traffic", "--fetch", fetch, "--write", write, "--copy-fetch", cf,
                                     "--copy-write", cw, "--copy-bytes", str(1 << 20), "--kernel", "lut_gemv",
                                     "--algorithmic-bytes", "200000", "--workload", "w", "--out", str(out)])
    assert RS.main() == 0
    d = json.loads(out.read_text())
    assert d["fetch_scale_from_copy"] == 2.0 and d["write_scale_from_copy"] == 1.0
    assert d["hbm_bytes_per_launch"] == 100 * 1024 * 2 + 8 * 1024
    assert d["kernel_source_hash"] == RS.kernel_source_hash() and len(d["kernel_source_hash"]) == 16
    assert d["traffic_over_algorithmic"] == round((100 * 2048 + 8192) / 200000, 4)


def test_trace_table_lists_the_kernels(tmp_path):
    d = tmp_path / "t"
    d.mkdir()
    (d / "t_kernel_stats.csv").write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"void fluxbin::lut_gemv_kernel<4, 1, 8, 4, 0, 0>(fluxbin::GemvArgs)",4,100,25.0,50.0,20,30,1.0\n'
        '"copyBuffer",2,100,50.0,50.0,50,50,0.0\n')
    rows = RS.trace_rows(str(d))
    assert rows[0][1:] == (4, 25.0, 20.0, 30.0) and rows[1][0] == "copyBuffer"


def test_trace_by_grid_keeps_the_shapes_apart(tmp_path, capsys, monkeypatch):
    d = tmp_path / "g"
    d.mkdir()
    hdr = ('"Kind","Agent_Id","Queue_Id","Stream_Id","Thread_Id","Dispatch_Id","Kernel_Id","Kernel_Name",'
           '"Correlation_Id","Start_Timestamp","End_Timestamp","LDS_Block_Size","Scratch_Size","VGPR_Count",'
           '"Accum_VGPR_Count","SGPR_Count","Workgroup_Size_X","Workgroup_Size_Y","Workgroup_Size_Z","Grid_Size_X",'
           '"Grid_Size_Y","Grid_Size_Z"\n')
    k = "void fluxbin::lut_gemv_kernel<4, 1, 8, 2, 0, 0>(fluxbin::GemvArgs)"
    rows = [(k, 100, 130, 112, 17), (k, 200, 220, 112, 17), (k, 300, 400, 112, 17), (k, 400, 410, 16, 57)]
    lines = [hdr] + [f'"KERNEL_DISPATCH","Agent 1",1,0,1,{i},1,"{n}",{i},{s},{e},0,0,60,0,40,512,1,1,{gx * 512},{gy},1\n'
                     for i, (n, s, e, gx, gy) in enumerate(rows)]
    (d / "b_kernel_trace.csv").write_text("".join(lines))
    out = {(key[1] // key[3], key[2]): (calls, avg, med, p10, p90)
           for key, calls, avg, med, p10, p90, mn, mx in RS.trace_by_grid(str(d))}
    # durations 30, 20, 100: percentiles linear between closest ranks (numpy's default): 22 and 86
    assert out == {(112, 17): (3, 50, 30, 22, 86), (16, 57): (1, 10, 10, 10, 10)}
    assert [RS.percentile([20, 30, 100], q) for q in (0, 10, 50, 90, 100)] == [20, 22, 30, 86, 100]
    monkeypatch.setattr(sys, "argv", ["x", "trace", str(d), "--by-grid", "--kernel", "lut_gemv"])
    assert RS.main() == 0
    text = capsys.readouterr().out
    assert "| 112 x 17 | 3 | 50 | 30 | 22 | 86 | 20 | 100 |" in text
    assert "| 16 x 57 | 1 | 10 | 10 | 10 | 10 | 10 | 10 |" in text
