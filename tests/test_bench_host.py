"""Host-side logic of bench.py (CPU only): the one-GPU contract and the algorithmic byte and flop
model the roofline divides by."""
import os
import subprocess
import sys

import bench
from synth import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_gate_up_bytes_are_weights_inputs_and_outputs():
    # 128 active rows of the LLaDA-8B shapes: 2F x d weights, R x d inputs and R x F outputs, bf16
    d, F, R = 4096, 12288, 128
    assert bench.ffn_up_bytes(workloads.LLADA, R) == (2 * F * d + R * d + R * F) * 2 == 205_520_896


def test_gemm_work_model():
    w = bench.kernel_work(workloads.LLADA, 128)
    d, V, R = 4096, 126464, 128
    _, rows, nbytes, flops = w["lm_head"]
    assert rows == R
    assert nbytes == (V * d + R * d) * 2 + R * V * 4  # fp32 logits out
    assert flops == 2.0 * R * V * d
    _, _, nbytes, flops = w["qkv"]
    assert nbytes == (3 * d * d + R * d) * 2 + R * 3 * d * 2
    assert flops == 2.0 * R * 3 * d * d


def test_dilated_round_count():
    # ceil(log2 block): 16 positions take 4 rounds, one position one round
    assert [bench.n_dus_rounds(b) for b in (1, 2, 3, 16, 17)] == [1, 1, 2, 4, 5]
