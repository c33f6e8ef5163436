"""Host-side checks of bench.py: the byte counts its roofline divides by, the
guard on committed counter summaries, and the one-GPU contract."""

import os
import subprocess
import sys

import bench
from workloads.configs import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_64k_layer():
    cfg = CONFIGS[4]
    pyr, sel = bench.algorithmic_bytes(cfg)
    H, d = 32, 128
    # pyramid: every prompt key read once (bf16), A_L written once (float32)
    assert pyr == H * 65536 * d * 2 + H * 1024 * d * 4 == 553648128
    # select-attend: Q, A_L, K of the 64 x 64 covered tokens, V of the 2048 kept,
    # K and V of the 512 generated, O (float32), the kept indices
    assert sel == H * (64 * d * 2 + 1024 * d * 4 + 4096 * d * 2 + 2048 * d * 2 + 2 * 512 * d * 2
                       + 64 * d * 4 + 4 * 2048) == 77332480


def test_attend_bytes_of_the_64k_layer():
    assert bench.attend_bytes(CONFIGS[4]) == 32 * (64 * 128 * 2 + 4 * 2048 + 2 * (2048 + 512) * 128 * 2
                                                   + 64 * 128 * 4)


def test_summaries_are_read_only_for_the_sources_they_were_taken_on(tmp_path):
    good = tmp_path / "good.txt"
    good.write_text(f"hbm_bytes_per_call: 123\nkernel_source_sha256_12: {bench.kernel_source_hash()}\n")
    assert bench.read_summary(str(good), ["hbm_bytes_per_call"]) == {"hbm_bytes_per_call": "123"}
    stale = tmp_path / "stale.txt"
    stale.write_text("hbm_bytes_per_call: 123\nkernel_source_sha256_12: 000000000000\n")
    assert bench.read_summary(str(stale), ["hbm_bytes_per_call"]) is None
    assert bench.read_summary(str(good), ["missing_key"]) is None
    assert bench.read_summary(str(tmp_path / "absent.txt"), ["hbm_bytes_per_call"]) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
