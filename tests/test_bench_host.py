"""Host-side checks of the benchmark's accounting and contract (no GPU):
the algorithmic bytes it divides by the measured times, counted here tensor by
tensor, and the refusal of more than one GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from chunkwise_delta_rule_wy_amd import synth  # noqa: E402


def test_chunk_gradient_bytes_per_token_head():
    # per token and head at dk = 128, dv = 256: q, k, v, dO in bf16, beta and g in
    # fp32 read; dq, dk, dv, dbeta, dg in fp32 written (3600 B); the bf16 chunk
    # states the kernel also reads are intermediates, counted apart
    read = 128 * 2 + 128 * 2 + 256 * 2 + 256 * 2 + 4 + 4
    written = 128 * 4 + 128 * 4 + 256 * 4 + 4 + 4
    assert read + written == 3600
    assert bench.chunk_grad_bytes(synth.WORKLOADS[4]) == 3600 * 4 * 4096 * 16  # 943.7 MB
    assert round(bench.chunk_grad_bytes(synth.WORKLOADS[4]) / 1e6, 1) == 943.7
    assert bench.chunk_state_bytes(synth.WORKLOADS[4]) == 4096 * 2 * 128 * 256 * 2
    # 32-token chunks: twice the states
    assert bench.chunk_state_bytes(synth.WORKLOADS[4], 32) == 2 * bench.chunk_state_bytes(synth.WORKLOADS[4])


def test_forward_and_decode_floors():
    # the HBM floors of the forward workloads and the decode step at 8 TB/s
    floors = {w: bench.workload_bytes(synth.WORKLOADS[w], False) / 8e12 * 1e6 for w in (2, 3, 5)}
    assert [round(floors[w], 1) for w in (2, 3, 5)] == [34.7, 52.7, 274.7]
    assert round(bench.decode_bytes() / 8e12 * 1e6, 1) == 135.3


def test_forward_bytes():
    # gated forward B4 T4096 H16 dk128 dv256: q, k, v in bf16, beta, g, h0 read;
    # o in bf16 and hT written
    th = 4 * 4096 * 16
    state = 4 * 16 * 128 * 256 * 4
    expect = th * (2 * 128 * 2 + 256 * 2 + 8) + th * 256 * 2 + 2 * state
    assert bench.workload_bytes(synth.WORKLOADS[3], False) == expect


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_flops():
    # the method's flop counts (GFLOP): the forward workloads 2, 3, 5, the
    # backward of workload 4 (no recompute) and one decode step of 256 x 32 states
    g = lambda f: round(f / 1e9, 2)
    assert [g(bench.fwd_flops(synth.WORKLOADS[w])) for w in (2, 3, 5)] == [36.97, 67.1, 295.73]
    assert g(bench.bwd_flops(synth.WORKLOADS[4])) == 137.09
    assert g(bench.decode_flops()) == 0.81
    # per token-head at dk = 128, dv = 256, C = 64 (MACs): 63/2 128 + 65/2 (256 + 512)
    # + 3 128 256 + 64^2 / 6
    mac = 63 / 2 * 128 + 65 / 2 * 768 + 3 * 128 * 256 + 64 * 64 / 6
    assert bench.fwd_flops(synth.WORKLOADS[3]) == 2 * mac * 4 * 4096 * 16
