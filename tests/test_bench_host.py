"""Host logic of bench.py, on the CPU: the one-GPU guard, the kernel-name
classes its profile summaries rely on, the rocprofv3 summary arithmetic (clock,
MFMA busy, calibrated traffic) and the algorithmic flop and byte counts."""
import csv
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


NS = "void matopt::(anonymous namespace)::"


@pytest.mark.parametrize("name,cls", [
    (NS + "ns_gemm_bf16_kernel<0, 0, 8, false>(matopt::GemmParams)", "gram"),
    (NS + "ns_gemm_bf16_kernel<1, 0, 8, false>(matopt::GemmParams)", "poly"),
    (NS + "ns_gemm_bf16_kernel<1, 0, 8, true>(matopt::GemmParams)", "poly"),
    (NS + "ns_gemm_bf16_kernel<2, 0, 8, false>(matopt::GemmParams)", "apply"),
    (NS + "ns_gemm_bf16_kernel<2, 1, 8, false>(matopt::GemmParams)", "apply_final"),
    (NS + "ns_gemm_bf16_kernel<2, 2, 8, false>(matopt::GemmParams)", "apply_final"),
    (NS + "ns_gemm_bf16_kernel<0, 0, 8>(matopt::GemmParams)", "gram"),
    (NS + "ns_apply_persist_kernel<8>(matopt::GemmParams)", "apply"),
    (NS + "prep_kernel<unsigned short>(matopt::PrepParams)", "prep"),
    (NS + "prep_t_kernel(matopt::PrepParams)", "prep"),
    (NS + "rmnp_kernel<unsigned short, 1, 4>(matopt::RmnpParams)", "rmnp"),
    (NS + "bind_kernel(matopt::BindArgs)", "bind"),
    ("__amd_rocclr_copyBuffer", "copy"),
    ("at::native::vectorized_elementwise_kernel<4, ...>", None),
])
def test_kernel_classes(name, cls):
    assert bench.kernel_class(name) == cls


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)


def test_profile_summary_arithmetic(tmp_path):
    gram = NS + "ns_gemm_bf16_kernel<0, 0, 8, false>(matopt::GemmParams)"
    # two Gram launches of 1000 and 3000 ns, one small and one large copy
    trace = [{"Kernel_Name": gram, "Start_Timestamp": 0, "End_Timestamp": 1000},
             {"Kernel_Name": gram, "Start_Timestamp": 5000, "End_Timestamp": 8000},
             {"Kernel_Name": "__amd_rocclr_copyBuffer", "Start_Timestamp": 9000,
              "End_Timestamp": 9100}]
    _write_csv(tmp_path / "x_kernel_trace.csv", trace)
    # GRBM_GUI_ACTIVE sums 8 XCDs: 8 * 2000 cycles over a 2000 ns average is 1 GHz;
    # MFMA busy is summed over 1024 SIMDs
    cnt = [{"Kernel_Name": gram, "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": 16000},
           {"Kernel_Name": gram, "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": 16000},
           {"Kernel_Name": gram, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES",
            "Counter_Value": 1024 * 1000},
           {"Kernel_Name": gram, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES",
            "Counter_Value": 1024 * 1000},
           {"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE",
            "Counter_Value": 2},
           {"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE",
            "Counter_Value": 524288}]
    _write_csv(tmp_path / "x_counter_collection.csv", cnt)
    out = bench.summarize_profile(str(tmp_path))
    g = out["gram"]
    assert g["launches"] == 2
    assert g["avg_us"] == pytest.approx(2.0)
    assert g["clock_GHz"] == pytest.approx(1.0)
    # the calibration reads the largest copy launch, not the mean over all
    assert out["copy"]["FETCH_SIZE_max"] == 524288
    assert out["copy"]["FETCH_SIZE_avg"] == pytest.approx((2 + 524288) / 2)


def test_algorithmic_counts():
    # one 256 x 512 and one 512 x 256 matrix (transposed: same m, n)
    m, n = 256, 512
    per_it = m * (m + 1) * n + m * m * (m + 1) + 2 * m * m * n
    assert bench.ns_alg_flops([(256, 512), (512, 256)], 5) == 2 * 5 * per_it
    # bf16 X0 read in place for a wide matrix with tile-multiple sides only
    assert bench.prep_alg_bytes([(256, 512)], "bf16") == 3 * 2 * 256 * 512
    assert bench.prep_alg_bytes([(512, 256)], "bf16") == 4 * 2 * 256 * 512
    assert bench.prep_alg_bytes([(300, 512)], "bf16") == 4 * 2 * 300 * 512
    assert bench.prep_alg_bytes([(256, 512)], "f32") == 4 * 4 * 256 * 512
