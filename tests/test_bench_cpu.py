"""bench.py's contract pieces that need no GPU: the one-GPU refusal for
--gpus N > 1, and the algorithmic byte / FLOP counts the roofline divides by
(hand-computed totals for the prefill shape)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line


def test_algorithmic_counts_at_prefill():
    import bench
    from workloads import get_workload
    w = get_workload("prefill")
    T, d, I, N, E, K = 16384, 6144, 2048, 512, 768, 12
    S, touched = 131072, 512
    a = bench.algorithmic(w, S, touched, 2)
    # gate/up: the touched experts' W_gate and W_up once, x once (rows are
    # gathered from it), h written once; 4 d I FLOPs per grouped row
    assert a["gemm_gate_up_swiglu"]["bytes"] == touched * 2 * I * d * 2 + T * d * 2 + S * I * 2
    assert a["gemm_gate_up_swiglu"]["flop"] == 4.0 * d * I * S
    # down: W_down once, h read, o written; 2 d I FLOPs per row
    assert a["gemm_down"]["bytes"] == touched * d * I * 2 + S * I * 2 + S * d * 2
    assert a["gemm_down"]["flop"] == 2.0 * d * I * S
    # router: x, fp32 W_router, fp32 logits; 2 T d E FLOPs
    assert a["router_gemm"]["bytes"] == T * d * 2 + E * d * 4 + T * E * 4
    assert a["router_gemm"]["flop"] == 2.0 * T * d * E
    # combine: the grouped rows, x, the residual and y once, plus the slots
    assert a["combine"]["bytes"] == S * d * 2 + 3 * T * d * 2 + T * K * 12
    # the totals quoted in the design notes
    assert a["gemm_gate_up_swiglu"]["bytes"] == pytest.approx(26.5e9, rel=0.01)
    assert a["combine"]["bytes"] == pytest.approx(2.22e9, rel=0.01)


def test_block_fp8_counts_weights_at_one_byte_plus_scales():
    import bench
    from workloads import get_workload
    w = get_workload("prefill")
    d, I = 6144, 2048
    a8 = bench.algorithmic(w, 131072, 512, 2, fp8=True)
    a16 = bench.algorithmic(w, 131072, 512, 2)
    diff = a16["gemm_gate_up_swiglu"]["bytes"] - a8["gemm_gate_up_swiglu"]["bytes"]
    assert diff == pytest.approx(512 * 2 * I * d * (2 - (1 + 1 / 32)))
