"""Host logic of bench.py that needs no GPU: the one-GPU guard and the
attribution of counter readings to library calls."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_counters(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for i, (name, kib) in enumerate(rows, start=1):
            wr.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib})


def test_record_traffic_attributes_kernels_to_calls(tmp_path, monkeypatch):
    calib_kib = bench.COPY_CALIB_BYTES / 1024
    step = [("void moe::(anonymous namespace)::route_list_kernel<16, 8, 8, true>(float const*)", 10.0),
            ("void moe::(anonymous namespace)::rank_count_kernel<ExpertBucket>(x)", 6.0),
            ("moe::(anonymous namespace)::permute_fused_kernel(x)", 100.0),
            ("moe::(anonymous namespace)::build_tiles_kernel(x)", 0.5),
            ("void moe::(anonymous namespace)::grouped_gemm_bf16_kernel<Cfg<...> >(x)", 1000.0),
            ("void moe::(anonymous namespace)::grouped_gemm_bf16_kernel<Cfg<...> >(y)", 500.0),
            ("void moe::(anonymous namespace)::combine_kernel<unsigned short>(x)", 50.0)]
    head = [("at::native::FillFunctor", 7.0), ("__amd_rocclr_copyBuffer", 12345.0)]
    # FETCH_SIZE reads half of the calibration copy, WRITE_SIZE all of it
    fetch = head + [("__amd_rocclr_copyBuffer", calib_kib / 2)] + step + step
    write = head + [("__amd_rocclr_copyBuffer", calib_kib)] + [(n, v / 10) for n, v in step] * 2
    _write_counters(tmp_path / "f", "FETCH_SIZE", fetch)
    _write_counters(tmp_path / "w", "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "mid_bf16", "--record-traffic", str(tmp_path / "f"),
                                      str(tmp_path / "w")])
    bench.record_traffic(bench.parse())
    e = json.load(open(out))["mid_bf16"]
    assert e["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert e["calibration"]["write_factor"] == pytest.approx(1.0)
    c = e["calls"]
    assert c["route"]["read_bytes"] == int(10.0 * 1024 * 2)
    assert c["permute"]["read_bytes"] == int(106.0 * 1024 * 2)        # rank passes belong to the permute
    assert c["swiglu"]["read_bytes"] == int(1500.5 * 1024 * 2)
    assert c["combine"]["write_bytes"] == int(5.0 * 1024)
    assert all(v["launches"] == 2 for v in c.values())
    # recorded figures are used only while the sources match
    w = bench.W.WORKLOADS["mid_bf16"]
    assert bench.recorded_traffic(w, "swiglu") == int(1500.5 * 1024 * 2) + int(150.05 * 1024)
    data = json.load(open(out))
    data["mid_bf16"]["calls"]["swiglu"]["sources_sha256"] = "0" * 64
    json.dump(data, open(out, "w"))
    assert bench.recorded_traffic(w, "swiglu") is None


def test_record_traffic_splits_a_training_step(tmp_path, monkeypatch):
    """Forward and backward kernels share names (tile tables, GEMMs, the
    combine): the backward GEMMs are told apart by their last two tile
    parameters (SwiGLU-backward epilogue, K-major B), tile tables go to the
    call of the next dispatch, and the fp32 combine is the token-gradient pass."""
    calib_kib = bench.COPY_CALIB_BYTES / 1024
    ns = "moe::(anonymous namespace)::"
    # tile arguments as the library names them: ..., EPI, BT, A stages, fragment distances, swapped layout
    gemm = ("void " + ns + "grouped_gemm_bf16_kernel<" + ns +
            "Cfg<128, 256, 2, 4, 3, {}, {}, false, 64, 1, 2, 8, false, {}, {}, 2, 1, 1, false>, false>(x)")
    step = [("void " + ns + "route_list_kernel<16, 8, 8, true>(float const*)", 1.0),
            ("void " + ns + "rank_count_kernel<ExpertBucket>(x)", 1.0),
            (ns + "scatter_rows_kernel(x)", 10.0),
            (ns + "build_tiles_kernel(x)", 0.5),
            (gemm.format("true", "false", 0, "false"), 100.0),
            (gemm.format("false", "false", 0, "false"), 50.0),
            ("void " + ns + "combine_kernel<unsigned short>(x)", 5.0),
            ("void " + ns + "combine_backward_kernel<unsigned short, unsigned short>(x)", 7.0),
            (ns + "build_tiles_kernel(x)", 0.25),
            (ns + "build_tiles_kernel(x)", 0.25),
            (gemm.format("false", "false", 0, "true"), 40.0),
            (gemm.format("true", "false", 1, "false"), 60.0),
            (gemm.format("false", "true", 0, "true"), 80.0)]
    step += [("void " + ns + "grouped_wgrad_kernel<" + ns + "WgCfg<128, 256, 2, 4, 3, 1> >(x)", 206.0)] * 2
    step += [("void " + ns + "combine_kernel<float>(x)", 9.0)]
    head = [("__amd_rocclr_copyBuffer", 99.0)]
    fetch = head + [("__amd_rocclr_copyBuffer", calib_kib / 2)] + step * 3
    write = head + [("__amd_rocclr_copyBuffer", calib_kib)] + step * 3
    _write_counters(tmp_path / "f", "FETCH_SIZE", fetch)
    _write_counters(tmp_path / "w", "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "mid_bf16_train", "--record-traffic",
                                      str(tmp_path / "f"), str(tmp_path / "w")])
    bench.record_traffic(bench.parse())
    c = json.load(open(out))["mid_bf16_train"]["calls"]
    assert set(c) == {"route", "permute", "swiglu", "combine", "combine_bwd", "swiglu_bwd", "dx_combine"}
    assert all(v["launches"] == 3 for v in c.values())
    assert c["swiglu"]["write_bytes"] == int(150.5 * 1024)
    assert c["swiglu_bwd"]["write_bytes"] == int((0.5 + 180.0 + 412.0) * 1024)
    assert c["combine"]["write_bytes"] == int(5.0 * 1024) and c["dx_combine"]["write_bytes"] == int(9.0 * 1024)
    assert c["combine_bwd"]["read_bytes"] == int(7.0 * 1024 * 2)
    # from saved activations: a row pass forms dG | dU in place of the gate/up GEMM
    saved = [e if e[0] != gemm.format("true", "false", 1, "false") else (ns + "swiglu_bwd_rows_kernel(x)", 20.0)
             for e in step]
    _write_counters(tmp_path / "f", "FETCH_SIZE", head + [("__amd_rocclr_copyBuffer", calib_kib / 2)] + saved * 2)
    _write_counters(tmp_path / "w", "WRITE_SIZE", head + [("__amd_rocclr_copyBuffer", calib_kib)] + saved * 2)
    bench.record_traffic(bench.parse())
    c = json.load(open(out))["mid_bf16_train"]["calls"]
    assert all(v["launches"] == 2 for v in c.values())
    assert c["swiglu_bwd"]["write_bytes"] == int((0.5 + 140.0 + 412.0) * 1024)


def test_record_mfma_busy_fraction(tmp_path, monkeypatch):
    """Busy fraction = MFMA busy cycles over (GUI-active cycles per XCD x CUs x
    4 SIMDs), cycle-weighted per call, set-up dispatches excluded."""
    d = tmp_path / "m"
    os.makedirs(d)
    with open(d / "run_agent_info.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Agent_Type", "Cu_Count", "Num_Xcc", "Simd_Per_Cu"])
        wr.writeheader()
        wr.writerow({"Agent_Type": "CPU", "Cu_Count": 0, "Num_Xcc": 1, "Simd_Per_Cu": 0})
        wr.writerow({"Agent_Type": "GPU", "Cu_Count": 256, "Num_Xcc": 8, "Simd_Per_Cu": 4})
    gu = "void moe::(anonymous namespace)::grouped_gemm_bf16_kernel<moe::(anonymous namespace)::Cfg<256, 256, 4, " \
         "2, 2, true, false, false, 64, 1, 4, 8, true, 0, false> >(x)"
    dn = gu.replace("2, 2, true, false, false", "2, 2, false, true, false")
    disp = [(gu, 1e9, 8e6)]                       # set-up call before the first library call: excluded
    disp += [("moe::(anonymous namespace)::compact_rows_kernel(x)", 0.0, 1e6), (gu, 0.5 * 1e6 * 1024, 8e6),
             (dn, 0.25 * 1e6 * 1024, 8e6)]
    fields = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=fields)
        wr.writeheader()
        for i, (name, busy, gui) in enumerate(disp, start=1):
            for c, v in (("SQ_VALU_MFMA_BUSY_CYCLES", busy), ("GRBM_GUI_ACTIVE", gui)):
                wr.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": c, "Counter_Value": v,
                             "Start_Timestamp": 0, "End_Timestamp": 1000})
    out = tmp_path / "mfma.json"
    monkeypatch.setattr(bench, "MFMA_FILE", str(out))
    monkeypatch.setattr(sys, "argv", ["bench.py", "--workload", "recv_share_bf16", "--record-mfma", str(d)])
    bench.record_mfma(bench.parse())
    c = json.load(open(out))["recv_share_bf16"]["calls"]
    # per XCD 1e6 GUI cycles, 1024 SIMDs: busy 0.5 for gate/up, 0.25 for down, 0.375 together
    assert c["swiglu:gate_up"]["mfma_busy"] == pytest.approx(0.5)
    assert c["swiglu:down_or_other"]["mfma_busy"] == pytest.approx(0.25)
    assert c["swiglu"]["mfma_busy"] == pytest.approx(0.375)
    assert c["swiglu"]["dispatches"] == 2
    monkeypatch.setattr(bench, "MFMA_FILE", str(out))
    assert bench.recorded_mfma(bench.W.WORKLOADS["recv_share_bf16"], "swiglu") == pytest.approx(0.375)


def test_nearest_rank_and_input_hash():
    import numpy as np
    v = [5.0, 1.0, 4.0, 2.0, 3.0]
    assert bench.nearest_rank(v, 50) == 3.0
    assert bench.nearest_rank(v, 95) == 5.0
    assert bench.nearest_rank(list(range(1, 101)), 95) == 95
    a = {"x": np.arange(6, dtype=np.uint16).reshape(2, 3), "p": [np.zeros(3, np.float32), np.ones(2, np.float32)]}
    h1 = bench.input_sha256(a)
    a["p"][1][0] = 2.0
    assert bench.input_sha256(a) != h1
    info = bench.cpu_host_info()
    assert set(info) == {"cpu_model", "host_cpus", "blas"}
