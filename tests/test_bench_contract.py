"""bench.py's contract, on the CPU: one GPU only, and the algorithmic work it
divides by (per-token matrix FLOPs, gate/up bytes) from the layer shapes."""
import os
import subprocess
import sys

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and not r.stdout


def test_per_token_matrix_work_of_the_real_layer():
    spec = synth.CONFIGS["prefill"]
    # pooler and unpooler 2 x 2HP, eight experts of 3 x 2PI each
    assert bench.layer_flops(spec, 1) == 2 * 2 * 8192 * 4096 + 8 * 3 * 2 * 4096 * 4096 == 939_524_096
    assert bench.layer_flops(spec, 16384) == 16384 * 939_524_096


def test_gate_up_bytes_count_touched_experts_once():
    spec = synth.CONFIGS["decode"]
    counts = np.zeros(256, np.int64)
    counts[:200] = 1
    counts[0] += 64 * 8 - 200
    expected = 200 * 2 * 4096 * 4096 * 2 + 512 * 4096 * 2 + 512 * 4096 * 2
    assert bench.gate_up_bytes(spec, counts, 64) == expected
    mx = synth.CONFIGS["mxfp4_decode"]  # E2M1 codes plus one E8M0 byte per 32
    assert bench.gate_up_bytes(mx, counts, 64) == 200 * 2 * 4096 * 4096 * (0.5 + 1 / 32) + 2 * 512 * 4096 * 2
