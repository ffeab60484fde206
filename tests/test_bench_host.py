"""Host-side logic of bench.py that needs no GPU."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def test_byte_counts_of_the_formats():
    # FP8: one byte a code + an FP32 scale per 128x128 block
    assert bench.weight_bytes("fp8", 17408, 5120) == 17408 * 5120 + 4 * 136 * 40
    # nibbles: half a byte a code, 16 B of FP16 scales per row and 8 K blocks, 16 B of map
    assert bench.weight_bytes("lut3", 28672, 8192) == 28672 * 8192 // 2 + 16 * 28672 * 8 + 16
    assert bench.weight_bytes("lut3d", 28672, 8192) == 28672 * 8192 * 3 // 8 + 16 * 28672 * 8 + 16
    assert bench.algorithmic_bytes("fp8", 17408, 5120, 16) == 89_871_616


def test_sysfs_gpu_state_reads_marked_level_and_sensors(tmp_path):
    node = tmp_path / "0000:05:00.0"
    (node / "hwmon" / "hwmon3").mkdir(parents=True)
    (node / "pp_dpm_sclk").write_text("0: 500Mhz\n1: 1800Mhz *\n2: 2400Mhz\n")
    hw = node / "hwmon" / "hwmon3"
    (hw / "temp1_input").write_text("45000\n")
    (hw / "temp1_label").write_text("edge\n")
    (hw / "temp2_input").write_text("61500\n")
    (hw / "freq1_input").write_text("2100000000\n")
    (hw / "freq1_label").write_text("sclk\n")
    st = bench.sysfs_gpu_state(str(node))
    assert st == {"sclk_level": "1800Mhz", "temp_edge_C": 45.0, "temp_temp2_C": 61.5, "sclk_MHz": 2100}


def test_sysfs_gpu_state_absent_node(tmp_path):
    assert bench.sysfs_gpu_state(str(tmp_path / "missing")) == {}


def test_more_than_one_gpu_is_refused():
    import subprocess
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr + r.stdout


def test_cpu_baseline_grades_the_gpu_output():
    """The CPU-baseline leg grades the timed workload's output against the
    oracle's: the oracle's own RNE result passes with 0 ULP, and one output
    moved far beyond both criteria fails (tiny config, no GPU needed)."""
    import numpy as np
    import oracle
    import synth
    fmt, N, K, Ms = synth.CONFIGS["tiny"]
    M = Ms[0]
    codes, scales = synth.fp8_weights(N, K, synth.SEEDS["tiny"])
    x = synth.x_bf16(M, K, synth.SEEDS["tiny"] + 100)
    good = oracle.bf16_rne(oracle.gemm_fp8(x, codes, scales))
    r = bench.cpu_baseline("tiny", M, min_seconds=0.0, gpu_bits=good)
    assert r["kind"] == "oracle" and r["parity"]["ok"] and r["parity"]["max_ulp"] == 0
    assert r["parity"]["n"] == M * N and r["parity"]["fail"] == 0
    bad = good.copy()
    moved = float(oracle.bf16_value(good[:1, 7:8])[0, 0]) + 100.0
    bad[0, 7] = oracle.bf16_rne(np.array([[moved]]))[0, 0]
    r = bench.cpu_baseline("tiny", M, min_seconds=0.0, gpu_bits=bad)
    assert not r["parity"]["ok"] and r["parity"]["fail"] == 1
