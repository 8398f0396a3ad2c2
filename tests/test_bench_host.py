"""Host logic of bench.py that runs without a GPU: the counter-CSV reduction behind
profiles/traffic.json, the median and bootstrap interval of the timed rounds, and the
multi-GPU refusal."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write_csv(path, dispatches, counter):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, v) in enumerate(dispatches, start=1):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_from_scales_by_copy_and_sums_each_call(tmp_path):
    mark = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<short>>(int)"
    copy = "void at::native::vectorized_elementwise_kernel<4, neg>(int)"
    gemm, red = "void w4::gemm_dma_kernel(GemmArgs)", "void w4::splitk_reduce_kernel(float*)"
    man = {"reps": 2, "groups": [
        {"key": "copy", "read_bytes": 2048 * 1024, "write_bytes": 1024 * 1024, "source": None},
        {"key": "gemm_f16_1570_2048_11008", "bytes": 1000, "flops": 1, "source": "gemm.hip", "source_sha": "x"}]}
    # the counters read half (fetch) and a quarter (write) of the true bytes
    setup = [("void setup_kernel()", 99.0)]
    fetch = setup + [(mark, 0.0), (copy, 1024.0), (copy, 1024.0), (mark, 0.0),
                     (gemm, 2.0), (red, 1.0), (gemm, 2.0), (red, 1.0), (mark, 0.0)]
    write = setup + [(mark, 0.0), (copy, 256.0), (copy, 256.0), (mark, 0.0),
                     (gemm, 0.5), (red, 0.25), (gemm, 0.5), (red, 0.25), (mark, 0.0)]
    _write_csv(tmp_path / "f.csv", fetch, "FETCH_SIZE")
    _write_csv(tmp_path / "w.csv", write, "WRITE_SIZE")
    (tmp_path / "m.json").write_text(json.dumps(man))
    out = tmp_path / "traffic.json"
    bench.traffic_from(str(tmp_path / "m.json"), str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(out))
    t = json.loads(out.read_text())
    assert t["copy_calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert t["copy_calibration"]["write_factor"] == pytest.approx(4.0)
    k = t["kernels"]["gemm_f16_1570_2048_11008"]
    assert k["hbm_read_bytes"] == pytest.approx(3 * 1024 * 2.0)   # 3 KiB per call (gemm + reduce) x 2
    assert k["hbm_write_bytes"] == pytest.approx(0.75 * 1024 * 4.0)
    assert k["source_sha"] == "x"
    assert t["kernels"]["gemm_f16_prefill"]["hbm_bytes_per_launch"] == pytest.approx(k["hbm_bytes_per_launch"])


def test_traffic_from_rejects_a_plan_mismatch(tmp_path):
    mark = "FillFunctor<short>"
    man = {"reps": 1, "groups": [{"key": "copy", "read_bytes": 1, "write_bytes": 1}, {"key": "a", "bytes": 1}]}
    _write_csv(tmp_path / "f.csv", [(mark, 0), ("c", 1), (mark, 0)], "FETCH_SIZE")
    _write_csv(tmp_path / "w.csv", [(mark, 0), ("c", 1), (mark, 0)], "WRITE_SIZE")
    (tmp_path / "m.json").write_text(json.dumps(man))
    with pytest.raises(SystemExit):
        bench.traffic_from(str(tmp_path / "m.json"), str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                           str(tmp_path / "t.json"))


def test_util_from_averages_each_kernel_per_dispatch(tmp_path):
    mark = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<short>>(int)"
    copy = "void at::native::vectorized_elementwise_kernel<4, neg>(int)"
    gemm, red = "void w4::gemm_dma_kernel(GemmArgs)", "void w4::splitk_reduce_kernel(float*)"
    man = {"reps": 2, "groups": [
        {"key": "copy", "read_bytes": 1, "write_bytes": 1, "source": None},
        {"key": "gemm_f16_1570_2048_11008", "bytes": 1000, "flops": 1, "source": "gemm.hip", "source_sha": "x"}]}
    seq = [("void setup()", 50.0, 50.0), (mark, 0, 0), (copy, 1.0, 0), (copy, 1.0, 0), (mark, 0, 0),
           (gemm, 10.0, 40.0), (red, 6.0, 0.0), (gemm, 12.0, 36.0), (red, 4.0, 0.0), (mark, 0, 0)]
    with open(tmp_path / "u.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, valu, mfma) in enumerate(seq, start=1):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": "VALUBusy", "Counter_Value": valu})
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": "MfmaUtil", "Counter_Value": mfma})
    (tmp_path / "m.json").write_text(json.dumps(man))
    out = tmp_path / "u.json"
    bench.util_from(str(tmp_path / "m.json"), str(tmp_path / "u.csv"), str(out))
    k = json.loads(out.read_text())["kernels"]["gemm_f16_1570_2048_11008"]
    assert k["source_sha"] == "x"
    g, r = k["by_kernel"]["void w4::gemm_dma_kernel"], k["by_kernel"]["void w4::splitk_reduce_kernel"]
    assert (g["VALUBusy"], g["MfmaUtil"], g["launches"]) == (pytest.approx(11.0), pytest.approx(38.0), 2)
    assert (r["VALUBusy"], r["MfmaUtil"], r["launches"]) == (pytest.approx(5.0), pytest.approx(0.0), 2)


def test_multi_gpu_request_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_median_ci_bootstrap_interval():
    import numpy as np
    const = bench.median_ci(np, [5.0] * 20)
    assert const == {"median": 5.0, "ci95": [5.0, 5.0], "rounds": 20}
    x = list(np.random.default_rng(3).normal(100.0, 2.0, 20))
    r = bench.median_ci(np, x)
    assert r["median"] == round(float(np.median(x)), 3)
    assert r["ci95"][0] <= r["median"] <= r["ci95"][1]
    assert r["ci95"][1] - r["ci95"][0] < 4.0  # the median of 20 N(100, 2) draws is tight
    assert bench.median_ci(np, x) == r  # fixed seed: the same interval every time
    # one slow outlier round moves neither the median nor the interval much
    y = x[:-1] + [1000.0]
    assert abs(bench.median_ci(np, y)["median"] - r["median"]) < 1.0
