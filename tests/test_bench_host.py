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


def _write_csv(path, dispatches, counters):
    """dispatches: (kernel name, {counter: value}) in dispatch order."""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, vals) in enumerate(dispatches, start=1):
            for c in counters:
                w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": c, "Counter_Value": vals.get(c, 0)})


def _rd(n32=0, n64=0, n128=0):
    return {"TCC_EA0_RDREQ_sum": n32 + n64 + n128, "TCC_EA0_RDREQ_32B_sum": n32, "TCC_EA0_RDREQ_64B_sum": n64,
            "TCC_EA0_RDREQ_128B_sum": n128}


def _wr(n32=0, n64=0):
    return {"TCC_EA0_WRREQ_sum": n32 + n64, "TCC_EA0_WRREQ_64B_sum": n64}


def test_traffic_from_counts_bytes_by_request_size_and_sums_each_call(tmp_path):
    mark = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<short>>(int)"
    copy = "void at::native::vectorized_elementwise_kernel<4, neg>(int)"
    gemm, red = "void w4::gemm_dma_kernel(GemmArgs)", "void w4::splitk_reduce_kernel(float*)"
    man = {"reps": 2, "groups": [
        {"key": "copy", "kind": "validation", "read_bytes": 128 * 100, "write_bytes": 64 * 200, "source": None},
        {"key": "gemm_f16_1570_2048_11008", "bytes": 1000, "flops": 1, "source": "gemm.hip", "source_sha": "x"}]}
    setup = [("void setup_kernel()", _rd(n128=99))]
    # each copy call: 100 reads of 128 B; each GEMM call: the GEMM reads 10 x 64 B + 4 x 32 B, the
    # reduce 2 x 128 B
    reads = setup + [(mark, {}), (copy, _rd(n128=100)), (copy, _rd(n128=100)), (mark, {}),
                     (gemm, _rd(n32=4, n64=10)), (red, _rd(n128=2)), (gemm, _rd(n32=4, n64=10)), (red, _rd(n128=2)),
                     (mark, {})]
    writes = setup + [(mark, {}), (copy, _wr(n64=200)), (copy, _wr(n64=200)), (mark, {}),
                      (gemm, _wr(n32=6, n64=1)), (red, _wr(n64=3)), (gemm, _wr(n32=6, n64=1)), (red, _wr(n64=3)),
                      (mark, {})]
    _write_csv(tmp_path / "r.csv", reads, bench.READ_COUNTERS)
    _write_csv(tmp_path / "w.csv", writes, bench.WRITE_COUNTERS)
    (tmp_path / "m.json").write_text(json.dumps(man))
    out = tmp_path / "traffic.json"
    bench.traffic_from(str(tmp_path / "m.json"), str(tmp_path / "r.csv"), str(tmp_path / "w.csv"), str(out))
    t = json.loads(out.read_text())
    v = t["validation"]["copy"]
    assert v["read_over_touched"] == pytest.approx(1.0) and v["write_over_touched"] == pytest.approx(1.0)
    k = t["kernels"]["gemm_f16_1570_2048_11008"]
    assert k["hbm_read_bytes"] == pytest.approx(10 * 64 + 4 * 32 + 2 * 128)
    assert k["hbm_write_bytes"] == pytest.approx(6 * 32 + 64 + 3 * 64)
    assert k["source_sha"] == "x"
    assert k["read_requests_by_size_over_all"] == pytest.approx(1.0)
    assert t["kernels"]["gemm_f16_prefill"]["hbm_bytes_per_launch"] == pytest.approx(k["hbm_bytes_per_launch"])


def test_traffic_from_rejects_a_plan_mismatch(tmp_path):
    mark = "FillFunctor<short>"
    man = {"reps": 1, "groups": [{"key": "copy", "kind": "validation", "read_bytes": 1, "write_bytes": 1},
                                 {"key": "a", "bytes": 1}]}
    _write_csv(tmp_path / "r.csv", [(mark, {}), ("c", _rd(1)), (mark, {})], bench.READ_COUNTERS)
    _write_csv(tmp_path / "w.csv", [(mark, {}), ("c", _wr(1)), (mark, {})], bench.WRITE_COUNTERS)
    (tmp_path / "m.json").write_text(json.dumps(man))
    with pytest.raises(SystemExit):
        bench.traffic_from(str(tmp_path / "m.json"), str(tmp_path / "r.csv"), str(tmp_path / "w.csv"),
                           str(tmp_path / "t.json"))


def test_util_from_averages_each_kernel_per_dispatch(tmp_path):
    mark = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<short>>(int)"
    copy = "void at::native::vectorized_elementwise_kernel<4, neg>(int)"
    gemm, red = "void w4::gemm_dma_kernel(GemmArgs)", "void w4::splitk_reduce_kernel(float*)"
    man = {"reps": 2, "groups": [
        {"key": "copy", "kind": "validation", "read_bytes": 1, "write_bytes": 1, "source": None},
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


def test_trace_from_takes_each_shape_between_markers(tmp_path):
    mark = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<short>>(int)"
    gemv = "void w4::(anonymous namespace)::gemv1s_kernel<3, 1, false, false, 1>(unsigned int const*)"
    gemm, red = "void w4::(anonymous namespace)::gemm_dma_kernel<8>(GemmArgs)", "w4::(anonymous namespace)::splitk_reduce_kernel(float*)"
    kernels = {"w4_gemv/1/22016/2048": {"launches": 3, "avg_us": 6.0},
               "gemm_f16/1570/2048/11008": {"launches": 2, "avg_us": 100.0}}
    (tmp_path / "b.json").write_text("[bench] log line\n" + json.dumps({"kernels": kernels}) + "\n")
    fields = ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Workgroup_Size_X"]
    seq = [(gemv, 0, 9000), (mark, 0, 1), (gemv, 0, 6000), (gemv, 0, 7000), (gemv, 0, 6500), (mark, 0, 1),
           (gemm, 0, 80000), (red, 0, 14000), (gemm, 0, 82000), (red, 0, 16000), (mark, 0, 1), (gemv, 0, 1)]
    with open(tmp_path / "t.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        t = 1000
        for i, (name, a, b) in enumerate(seq, start=1):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Start_Timestamp": t + a, "End_Timestamp": t + b,
                        "Grid_Size_X": 1835 * 256 if "gemv" in name else 240 * 512, "Workgroup_Size_X": 256 if "gemv" in name else 512})
            t += 100000
    out = tmp_path / "kt.json"
    bench.trace_from(str(tmp_path / "b.json"), str(tmp_path / "t.csv"), out_path=str(out))
    k = json.loads(out.read_text())["kernels"]
    g = k["w4_gemv/1/22016/2048"]
    assert g["dispatches"] == 3 and g["mean_us"] == pytest.approx(6.5) and g["median_us"] == pytest.approx(6.5)
    assert g["mean_over_bench"] == pytest.approx(6.5 / 6.0)
    assert g["kernels"] == ["gemv1s_kernel<3, 1, false, false, 1>[1835]"]
    m = k["gemm_f16/1570/2048/11008"]
    assert m["kernels_per_launch"] == 2 and m["mean_us"] == pytest.approx(96.0)


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
