"""Host-side logic of bench.py (no GPU): the HBM-traffic summary of two rocprofv3
--pmc runs, the algorithmic byte counts it is compared with, and the traffic records'
source hashes."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _write_counters(path, counter, rows):
    """rows: (dispatch id, kernel name as rocprofv3 prints it, grid, per-instance values)"""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for did, name, grid, vals in rows:
            for v in vals:
                w.writerow(dict(Dispatch_Id=did, Kernel_Name=name, Grid_Size=grid, Counter_Name=counter,
                                Counter_Value=v))


def test_summarize_pmc_scales_by_the_calibration_copy(tmp_path, capsys):
    n_kib = (256 << 20) / 1024
    copy = "__amd_rocclr_copyBuffer"
    gemv = "void nvq::gemv_nvfp4_kernel<0, false, 8, 5>(unsigned char const*, long, int, signed char const*)"
    gemm = "void nvq::gemm_nvfp4_kernel<nvq::(anonymous namespace)::NvCfg<1, 8, 8, 1>, false>(unsigned char const*)"
    red = "void nvq::ksplit_reduce_kernel<nvq::(anonymous namespace)::NvCfg<1, 8, 8, 1> >(float const*, long)"
    q4 = "void nvq::gemm_q4x_i8_kernel<nvq::(anonymous namespace)::QI8Cfg<2, 4, 2, 1>, 1, false>(unsigned char const*)"
    q4red = "void nvq::ksplit_reduce_kernel<nvq::(anonymous namespace)::QI8Cfg<2, 4, 2, 1> >(float const*, long)"
    # FETCH_SIZE reads half the copied bytes (factor 2), WRITE_SIZE all of them; counter
    # values are split over instances (summed per dispatch)
    fetch = [("1", copy, "131072", [n_kib / 4, n_kib / 4]),
             ("2", gemv, "1114112", [100.0, 200.0]), ("3", gemv, "1114112", [150.0, 150.0]),
             ("4", gemm, "393216", [1000.0]), ("5", red, "262144", [10.0]),
             ("6", q4, "131072", [40.0]), ("7", q4red, "262144", [4.0])]
    write = [("1", copy, "131072", [n_kib / 2, n_kib / 2]),
             ("2", gemv, "1114112", [1.0]), ("3", gemv, "1114112", [3.0]),
             ("4", gemm, "393216", [500.0]), ("5", red, "262144", [5.0]),
             ("6", q4, "131072", [20.0]), ("7", q4red, "262144", [2.0])]
    fp, wp = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _write_counters(fp, "FETCH_SIZE", fetch)
    _write_counters(wp, "WRITE_SIZE", write)
    bench.summarize_pmc(str(fp), str(wp))
    res = json.loads(capsys.readouterr().out)

    assert res["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert res["calibration"]["write_factor"] == pytest.approx(1.0)
    g = res["gemv_nvfp4_gate_up"]
    assert g["kernel"] == "gemv_nvfp4_kernel<0, false, 8, 5>" and g["dispatches"] == 2
    assert g["bytes_per_launch"] == pytest.approx((300.0 * 2 + 2.0) * 1024)  # mean fetch 300 KiB x 2, write 2 KiB
    assert g["alg_bytes_per_launch"] == bench.gemv_alg_bytes(1, 34816, 5120)
    m = res["gemm_nvfp4_m2048"]
    assert m["parts"]["main"]["kernel"] == "gemm_nvfp4_kernel<NvCfg<1, 8, 8, 1>, false>"
    assert m["parts"]["reduce"]["kernel"] == "ksplit_reduce_kernel<NvCfg<1, 8, 8, 1> >"
    assert m["bytes_per_launch"] == pytest.approx((1000.0 * 2 + 500.0 + 10.0 * 2 + 5.0) * 1024)
    q = res["gemm_q4_1_m512"]
    assert q["parts"]["reduce"]["kernel"] == "ksplit_reduce_kernel<QI8Cfg<2, 4, 2, 1> >"
    assert q["bytes_per_launch"] == pytest.approx((40.0 * 2 + 20.0 + 4.0 * 2 + 2.0) * 1024)
    # the fused kernel ran in neither file: no record
    assert "gemv_nvfp4_fused_gate_up" not in res


def test_gemm_alg_bytes():
    # NVFP4: 9/16 B per weight (codes + one UE4M3 byte per 16); Q4_1: 5/8 B (codes + fp16 d, m per 32)
    assert bench.gemm_alg_bytes("nvfp4", 2048, 17408, 5120) == (
        17408 * 5120 // 2 + 17408 * 5120 // 16 + 2048 * 5120 + 2048 * 160 * 2 + 4 * 2048 * 17408)
    assert bench.gemm_alg_bytes("q4_1", 512, 4096, 4096) == (
        4096 * 4096 // 2 + 4096 * 128 * 4 + 512 * 4096 + 512 * 128 * 2 + 4 * 512 * 4096)


def test_traffic_records_match_the_current_sources():
    """profiles/traffic.json is keyed by a hash of the kernels' sources: bench reports a
    record only while it matches, and every committed record names its kernel."""
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        t = json.load(f)
    for key in bench.KERNEL_SOURCES:
        assert key in t, key
        assert t[key]["src_hash"] == bench.kernel_src_hash(key), key
        assert bench.load_traffic(key) == pytest.approx(t[key]["bytes_per_launch"])
        assert t[key]["bytes_per_launch"] >= t[key]["alg_bytes_per_launch"] * 0.99


def test_src_hash_ignores_comments():
    a = "int f(int x) { // one\n  return x + 1; /* two */ }\n"
    b = "int f(int x) {\n  return x + 1; }  // changed comment\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(a.replace("+ 1", "+ 2"))


@pytest.mark.parametrize("argv, env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    """Only one GPU is measured: asking for more exits with status 2 and says why,
    before anything touches a device."""
    import subprocess

    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env=e, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
