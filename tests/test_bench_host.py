"""Host-side pieces of bench.py (no GPU): the one-GPU contract, the
algorithmic byte and op counts behind roofline.achieved, and the handling
of committed counter records."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert out.returncode == 2
    assert "one GPU" in out.stderr
    assert out.stdout.strip() == ""


@pytest.mark.parametrize("M,N,K,R", [(700, 3072, 1024, 32), (1, 14336, 4096, 32), (17, 48, 128, 0)])
def test_algorithmic_counts_closed_form(M, N, K, R):
    """Counts written out from the layer's definition: the int4 product is
    2MNK ops, LoRA 2MR(K+N); the GEMM moves the packed activation (half a
    byte per code plus one fp16 scale per 64 codes, rows padded to 16), the
    fp32 lora_act, the packed weights, L_up, a and b, and writes fp16 Y."""
    c = bench.algorithmic_counts(M, N, K, R)
    Mp = -(-M // 16) * 16
    assert c["layer_ops"] == 2 * M * N * K + 2 * M * R * K + 2 * M * R * N
    assert c["lin_ops"] == 2 * M * N * K + 2 * M * N * R
    act = Mp * K / 2 + Mp * (K / 64) * 2 + Mp * R * 4
    wts = N * K / 2 + N * (K / 64) * 2 + N * R * 2 + N * 4 * 2
    assert c["lin_bytes"] == act + wts + M * N * 2
    assert c["q_bytes"] == M * K * 2 + K * R * 2 + act


def test_traffic_record_is_ignored_once_the_kernels_change(tmp_path, monkeypatch):
    """A committed FETCH/WRITE record counts only while the kernel sources
    hash matches the one it was taken with."""
    rec = {"fetch_kib": 100.0, "write_kib": 50.0, "fetch_factor": 2.0, "write_factor": 1.0,
           "source_sha": bench.kernel_source_hash()}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"w": rec}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("w") == (100.0 * 2.0 + 50.0) * 1024
    rec["source_sha"] = "0" * 16
    f.write_text(json.dumps({"w": rec}))
    assert bench.measured_traffic("w") is None
    assert bench.measured_traffic("missing") is None


def test_kernel_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    """Comment-only edits of the kernel sources keep committed counters valid;
    any change to a line of code invalidates them."""
    import shutil
    for rel in bench.KERNEL_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(bench.ROOT, rel), dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    base = bench.kernel_source_hash()
    gemm = tmp_path / bench.KERNEL_SOURCES[0]
    text = gemm.read_text()
    gemm.write_text(text.replace("namespace w4a4 {", "namespace w4a4 {   // a new comment\n\n// and another", 1))
    assert bench.kernel_source_hash() == base
    gemm.write_text(text.replace("kTileGroupRows = 8", "kTileGroupRows = 4", 1))
    assert bench.kernel_source_hash() != base
