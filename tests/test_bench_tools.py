"""Host-side checks of the benchmark's measurement plumbing (no GPU): the
rocprofv3 counter summary scales FETCH_SIZE / WRITE_SIZE by the plain copy's
reading, the traffic recorded under profiles/ is used only while the kernel
source is unchanged, and a multi-GPU request is refused."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

HDR = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id","Grid_Size","Kernel_Id",'
       '"Kernel_Name","Workgroup_Size","LDS_Block_Size","Scratch_Size","VGPR_Count","Accum_VGPR_Count","SGPR_Count",'
       '"Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"\n')


def _counter_csv(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w") as fh:
        fh.write(HDR)
        for i, (kernel, value) in enumerate(rows):
            fh.write(f'{i},{i},1,1,1,1,1,1,"{kernel}",256,0,0,8,0,16,"{counter}",{value},0,1\n')


def test_counter_summary_scales_by_the_copy(tmp_path, capsys):
    gib_kib = bench.COPY_CAL_BYTES // 1024
    k = "void qmm::gemv_stream_kernel<2, 1, false, 8>(...)"
    _counter_csv(tmp_path / "f", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", gib_kib // 2), (k, 1000), (k, 3000)])
    _counter_csv(tmp_path / "w", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", gib_kib), (k, 10), (k, 30)])
    bench.summarize_counters([str(tmp_path / "f"), str(tmp_path / "w")])
    out = capsys.readouterr().out
    line = [l for l in out.splitlines() if l.startswith("TRAFFIC gemv_stream_kernel")][0]
    # FETCH counted half of the copy's bytes (factor 2), WRITE all of them (factor 1)
    assert int(line.split()[3]) == 2 * 2000 * 1024 + 20 * 1024
    assert f"source_sha256 {bench.source_hash('gemv_stream_kernel')}" in line


def test_traffic_is_used_only_for_the_profiled_source(tmp_path, monkeypatch):
    h = bench.source_hash("gemm_kernel")
    (tmp_path / "a.txt").write_text(f"x\nTRAFFIC gemm_kernel bytes_per_launch 12345 source_sha256 {h}\n")
    (tmp_path / "b.txt").write_text("TRAFFIC gemv_stream_kernel bytes_per_launch 99 source_sha256 0000000000000000\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.traffic_from_profiles("gemm_kernel", "a.txt") == 12345
    assert bench.traffic_from_profiles("gemm_kernel", "b.txt") is None     # only the named profile is read
    assert bench.traffic_from_profiles("gemv_stream_kernel", "b.txt") is None  # another source's figure
    assert bench.traffic_from_profiles("gemm_kernel", "missing.txt") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
