"""bench.py's contract on the host: more than one GPU is refused with a message and exit
status 2 (nothing here runs on several GPUs), and the algorithmic figures the roofline
objects divide by are the ones the per-token and per-head counts give."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes():
    # prefill: q, k (16 heads) and v, o (32 heads) bf16 at 128 per head, g and beta fp32 per
    # V head -- 24,832 bytes per token -- plus the states in and out (64 KiB per V head each)
    per_token = 2 * 16 * 128 * 2 + 2 * 32 * 128 * 2 + 2 * 32 * 4
    assert per_token == 24832
    assert bench.prefill_bytes(32768, 1, True) == 32768 * per_token + 2 * 32 * 128 * 128 * 4
    assert bench.prefill_bytes(32768, 1, True) == 817_889_280
    assert bench.prefill_bytes(4096, 1, False) == 4096 * per_token + 32 * 128 * 128 * 4
    # decode: every state read and written once, plus each sequence's inputs and output
    assert bench.decode_bytes(256) == 1_080_098_816
    assert bench.decode_bytes(256) > 2 * 256 * 32 * 128 * 128 * 4


def test_algorithmic_flops():
    # 10 C d + 6 d^2 FLOPs per token and V head (C = 64, d = 128)
    per = 10 * 64 * 128 + 6 * 128 * 128
    assert per == 180_224
    assert bench.prefill_flops(32768) == 32768 * 32 * per
    assert bench.prefill_flops(4096) == 23_622_320_128
