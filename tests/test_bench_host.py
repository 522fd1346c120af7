"""Host-side logic of bench.py, on the CPU: the algorithmic byte counts its roofline
fractions divide by, the check that a committed profile was taken on the current sources,
the refusal of more than one GPU, and the CPU baseline's one-core leg on a tiny workload."""
import hashlib
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes_llama_up_bf16_2_4():
    # 11008 x 4096 bf16, 2:4 (2-bit fields), T = 2048, bf16 out
    R, K, T = 11008, 4096, 2048
    ab = bench.algorithmic_bytes(R, K, T, 2, 4, 2, 2)
    e = R * K
    meta = R * (K // 4 * 2 * 2 // 32) * 4        # 2048 fields of 2 bits per row: 128 words
    assert meta == R * 512
    assert ab["mask"] == 3 * e                    # W in, one mask byte out
    assert ab["compress"] == 2 * e + e + meta     # W in; half the values out; metadata
    assert ab["mask_compress"] == 2 * e + e + e + meta
    assert ab["decompress"] == e + meta + 2 * e
    assert ab["spmm"] == e + meta + K * T * 2 + R * T * 2
    # the figure the bench prints as the product's algorithmic bytes per launch
    assert ab["spmm"] == 112590848


def test_algorithmic_bytes_meta_rounds_rows_to_words():
    # 4:8 (3-bit fields): K = 104 gives 52 fields = 156 bits, 5 words per row
    ab = bench.algorithmic_bytes(3, 104, 1, 4, 8, 2, 2)
    assert ab["compress"] == 3 * 104 * 2 + 3 * 52 * 2 + 3 * 5 * 4
    assert ab["spmm"] == 3 * 52 * 2 + 3 * 5 * 4 + 104 * 1 * 2 + 3 * 1 * 2


def write_profile(tmp, name, sources, per):
    prof = {"sources_sha256": sources, "per_dispatch_bytes": per,
            "kernel": "gains_kernel<2, 4>", "valu_insts_per_dispatch": {"m": 7.0}}
    (tmp / "profiles").mkdir(exist_ok=True)
    (tmp / "profiles" / name).write_text(json.dumps(prof))


def test_profiles_are_used_only_on_the_sources_they_were_taken_on(tmp_path, monkeypatch):
    csrc = tmp_path / "masking_sparse_gemm_amd" / "csrc"
    csrc.mkdir(parents=True)
    files = {"nm_spmm.hip": b"a", "nm_spmm_sk.hip": b"b", "nm_mfma.h": b"c", "nm_perm.hip": b"d"}
    for n, b in files.items():
        (csrc / n).write_bytes(b)
    sha = {n: hashlib.sha256(b).hexdigest() for n, b in files.items()}
    per = {"smfmac_ws_spmm_kernel<x> [grid=1]": {"read_bytes": 100.0, "write_bytes": 20.0},
           "smfmac_ws_spmm_kernel<x> [grid=2]": {"read_bytes": 300.0, "write_bytes": 20.0},
           "other_kernel [grid=3]": {"read_bytes": 5.0, "write_bytes": 5.0}}
    write_profile(tmp_path, "w_traffic.json", sha, per)
    write_profile(tmp_path, "w_valu.json", sha, {})
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # mean over the matching dispatches' read + write bytes
    assert bench.profiled_traffic("w") == pytest.approx(220.0)
    assert bench.profiled_traffic("w", "other_kernel") == pytest.approx(10.0)
    assert bench.profiled_traffic("w", "absent") is None
    assert bench.profiled_valu("w") == {"m": 7.0}
    assert bench.profiled_traffic("missing") is None
    # any listed source changed since the profile: no figure
    (csrc / "nm_spmm_sk.hip").write_bytes(b"changed")
    assert bench.profiled_traffic("w") is None
    assert bench.profiled_valu("w") == {"m": 7.0}        # its own source did not change
    (csrc / "nm_perm.hip").write_bytes(b"changed")
    assert bench.profiled_valu("w") == {}


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode != 0
    assert "one GPU" in (res.stdout + res.stderr)


def test_cpu_one_core_leg_on_a_tiny_workload():
    import synth

    w = synth.WORKLOADS["toy_f32"]
    mats = [{"name": "toy", "R": w.R, "K": w.K, "T": w.T, "W": w.W(), "X": w.X(), "dtype": "f32",
             "s": 4, "ys": 4}]
    r = bench.cpu_one_core(mats, 2, 4, rows=8)
    assert r["cores"] == 1 and r["value"] > 0 and np.isfinite(r["value"])
    assert r["phases"]["mask_compress_gbps"] > 0 and r["phases"]["product_TFLOP_per_s"] > 0
    # 8 of 64 rows timed: the whole-workload step is 8x the sample's time
    assert r["extrapolated_step_s"] == pytest.approx(8 * r["seconds"], abs=0.1)


def test_cpu_baseline_all_cores_on_a_tiny_workload():
    import synth

    w = synth.WORKLOADS["toy_f32"]
    mats = [{"name": "toy", "R": w.R, "K": w.K, "T": w.T, "W": w.W(), "X": w.X(), "dtype": "f32",
             "s": 4, "ys": 4}]
    r = bench.cpu_baseline(mats, 2, 4, threads=2, budget_s=0.0)
    assert r["cores"] == 2 and r["kind"] == "oracle" and r["value"] > 0
    assert "rows 0..8 of 64" in r["sample"]            # one round: 4 rows per thread
    ph = r["phases"]
    assert ph["mask_compress_gbps"] > 0 and ph["decompress_gbps"] > 0
    assert ph["product_TFLOP_per_s"] > 0
