"""bench.py host logic: the one-GPU guard, the algorithmic counts it prices the roofline
with, and the counter calibration behind `traffic`. No GPU is used."""
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
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_flops_per_chunk_head():
    # per chunk-head at C = 64, d_k = d_v = 128: A_kk 516,096, A_qk 532,480, W and U
    # 524,288 each, the solve 83,328, three state contractions 6,291,456, A_qk E 532,480,
    # decay 16,384 (triangles counted as triangles)
    assert bench.prefill_flops(64, 1, 128, 128) == 9_020_800
    assert bench.prefill_flops(8192, 64, 128, 128) == 9_020_800 * 64 * 128


def test_compulsory_bytes_main_and_decode():
    # main prefill, bf16 q, k, v, beta, fp32 g: 810,549,248 B with a bf16 o; bench.py
    # writes o in fp32 (134,217,728 B more)
    assert bench.prefill_bytes(8192, 64, 128, 128, 2, 2, 1) == 810_549_248
    assert bench.prefill_bytes(8192, 64, 128, 128, 2, 4, 1) == 810_549_248 + 134_217_728
    # decode step, N256 H64: 2,172,682,240 B with a bf16 o; fp32 o adds 4,194,304
    assert bench.decode_bytes(256, 64, 128, 128, 2, 2) == 2_172_682_240
    assert bench.decode_bytes(256, 64, 128, 128, 2, 4) == 2_172_682_240 + 4_194_304


def test_code_hash_ignores_comments_and_spacing():
    a = "int f(int x) {\n  return x + 1; // one\n}\n/* block\n comment */"
    b = "int f(int x) { return x + 1; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only("return x + 1;") != bench._code_only("return x + 2;")


def _write_csv(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_traffic_summary_calibration(tmp_path):
    KiB = 1024.0
    copy_kib = bench.COPY_BYTES / KiB
    # the copy reads half of its bytes in FETCH_SIZE units and all of them in WRITE_SIZE
    _write_csv(tmp_path / "cf.csv", [{"Dispatch_Id": 1, "Kernel_Name": "copyBuffer",
                                      "Counter_Name": "FETCH_SIZE",
                                      "Counter_Value": copy_kib / 2}])
    _write_csv(tmp_path / "cw.csv", [{"Dispatch_Id": 1, "Kernel_Name": "copyBuffer",
                                      "Counter_Name": "WRITE_SIZE", "Counter_Value": copy_kib}])
    # two prep dispatches, each counted on two instances (summed per dispatch)
    fetch = [{"Dispatch_Id": d, "Kernel_Name": "kda::prep_kernel<...>", "Counter_Name": "FETCH_SIZE",
              "Counter_Value": 1000.0} for d in (1, 2) for _ in range(2)]
    fetch += [{"Dispatch_Id": 3, "Kernel_Name": "kda::state_kernel<...>",
               "Counter_Name": "FETCH_SIZE", "Counter_Value": 500.0}]
    write = [{"Dispatch_Id": d, "Kernel_Name": "kda::prep_kernel<...>", "Counter_Name": "WRITE_SIZE",
              "Counter_Value": 3000.0} for d in (1, 2)]
    write += [{"Dispatch_Id": 3, "Kernel_Name": "kda::state_kernel<...>",
               "Counter_Name": "WRITE_SIZE", "Counter_Value": 100.0}]
    # Gated DeltaNet and Gated DeltaNet-2 dispatches are not part of the KDA figures
    fetch += [{"Dispatch_Id": 4, "Kernel_Name": "void kda::prep_kernel<__hip_bfloat16, 128, 128, true>(...)",
               "Counter_Name": "FETCH_SIZE", "Counter_Value": 9.0e6},
              {"Dispatch_Id": 5, "Kernel_Name": "_ZN3kda11prep_kernelIDF16bLi128ELi128ELb1ELb0EEEvPKT_",
               "Counter_Name": "FETCH_SIZE", "Counter_Value": 7.0e6},
              {"Dispatch_Id": 6, "Kernel_Name": "_ZN3kda11prep_kernelIDF16bLi128ELi128ELb0ELb1EEEvPKT_",
               "Counter_Name": "FETCH_SIZE", "Counter_Value": 5.0e6},
              {"Dispatch_Id": 7, "Kernel_Name": "void kda::decode_kernel<__bf16, float, 128, 128, false, true>(...)",
               "Counter_Name": "FETCH_SIZE", "Counter_Value": 3.0e6},
              # the raw-input and gated modes of the bf16 prep kernel
              {"Dispatch_Id": 8, "Kernel_Name": "void kda::prep_fast_kernel<1>(...)",
               "Counter_Name": "FETCH_SIZE", "Counter_Value": 2.0e6},
              {"Dispatch_Id": 9, "Kernel_Name": "void kda::prep_fast_kernel<2>(...)",
               "Counter_Name": "FETCH_SIZE", "Counter_Value": 2.0e6}]

    _write_csv(tmp_path / "f.csv", fetch)
    _write_csv(tmp_path / "w.csv", write)
    out_file = str(tmp_path / "traffic.json")
    out = bench.traffic_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"),
                                out_file=out_file)
    assert out["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert out["calibration"]["write_factor"] == pytest.approx(1.0)
    prep = out["per_kernel"]["prep_kernel"]
    assert prep["dispatches"] == 2
    assert prep["fetch_bytes"] == pytest.approx(2000.0 * KiB * 2.0)
    assert prep["write_bytes"] == pytest.approx(3000.0 * KiB)
    state = out["per_kernel"]["state_kernel"]
    assert out["prefill_call_bytes"] == pytest.approx(
        prep["fetch_bytes"] + prep["write_bytes"] + state["fetch_bytes"] + state["write_bytes"])
    assert out["decode_bytes"] is None
    assert set(out["per_kernel"]) == {"prep_kernel", "state_kernel"}
    # figures are used only while the kernel sources hash to the recorded value
    assert bench.load_traffic(out_file)[0] == pytest.approx(out["prefill_call_bytes"])
    d = json.load(open(out_file))
    d["kernels_source_sha256"] = "0" * 64
    json.dump(d, open(out_file, "w"))
    assert bench.load_traffic(out_file) == (None, None)


def test_code_hash_ignores_python_comments():
    assert bench._code_only("x = 1  # one\n# two\n", python=True) == bench._code_only("x = 1", python=True)


def test_kernel_names_of_the_kda_figures():
    """The bf16 prep kernel's KDA mode counts as the prep kernel (demangled or mangled); its
    raw-input and gated modes and the gate variants of the other kernels do not."""
    assert bench._short("void kda::prep_fast_kernel<0>(bf16 const*, ...)") == "prep_kernel"
    assert bench._short("_ZN3kda16prep_fast_kernelILi0EEEvPKDF16b") == "prep_kernel"
    assert bench._short("void kda::prep_fast_kernel<1>(bf16 const*, ...)") is None
    assert bench._short("_ZN3kda16prep_fast_kernelILi2EEEvPKDF16b") is None
    assert bench._short("void kda::state_kernel<bf16, float, 128, 128, 32>(...)") == "state_kernel"
    assert bench._short("void kda::decode_kernel<bf16, float, 128, 128, true, false>(...)") is None
