"""Seeded sweep over random small layer shapes, against the fp64 oracle.

The hand-picked edge shapes of the other GPU tests cover the cases the
kernels branch on; this sweep draws shapes at random (a fixed generator per
case, so every run checks the same ones) to reach combinations nobody picked:
widths d in multiples of 64 and I in multiples of 128, 1 to 70 FFN experts,
0 to 16 identity experts, K from 1 to min(E, 12), 1 to 699 tokens, a uniform
bias of three sizes or Zipf(1.2) logit offsets that pile rows onto a few
experts; a second set draws many tokens and experts on narrow widths
(500-3999 tokens, 2-599 FFN and 0-299 identity experts, K up to 32), where
experts span several row tiles.  Each case checks, through the C ABI:
- forward: the row-major and packed bf16 forwards give the same bits, and
  the layer output, routing and grouping meet the oracle bars of
  gpu_check.check_forward (with and without the residual);
- block FP8 (d a multiple of 128): gate/up, then gate/up and down, against
  oracle.mx;
- backward: every gradient against oracle.backward at the forward's bar."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_bias_amd as m
from gpu_check import check_forward, run_gpu
from test_gpu_backward import compare, gpu_forward_backward
from workloads import Workload, make_inputs, make_upstream_grad

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def draw(i: int, d_step: int = 64) -> Workload:
    r = np.random.default_rng(7000 + i)
    d = d_step * int(r.integers(1, 384 // d_step + 1))
    I = 128 * int(r.integers(1, 4))
    N = int(r.choice([1, 2, 3, 5, 8, 13, 24, 40, 70]))
    Z = int(r.choice([0, 1, 4, 9, 16]))
    K = int(r.integers(1, min(N + Z, 12) + 1))
    T = int(r.integers(1, 700))
    zipf = (1.2, 2.0) if r.random() < 0.25 else None
    bias = ("zero",) if zipf else ("uniform", float(r.choice([0.0, 0.02, 0.1])))
    return Workload(f"random{i}", T=T, d=d, I=I, N=N, Z=Z, K=K, dtype="bf16", seed=100 + i,
                    bias=bias, zipf=zipf)


def draw_wide(i: int, d_choices=(64, 128)) -> Workload:
    """Many tokens and experts on narrow widths: experts that span several
    row tiles and split ones, up to 600 FFN and 300 identity experts, K up to
    32 (the library's limit)."""
    r = np.random.default_rng(9000 + i)
    d = int(r.choice(d_choices))
    I = 128 * int(r.integers(1, 3))
    N = int(r.integers(2, 600))
    Z = int(r.integers(0, 300))
    K = int(r.integers(1, min(N + Z, 32) + 1))
    T = int(r.integers(500, 4000))
    zipf = (1.2, 2.0) if r.random() < 0.25 else None
    bias = ("zero",) if zipf else ("uniform", float(r.choice([0.0, 0.005, 0.02])))
    return Workload(f"wide{i}", T=T, d=d, I=I, N=N, Z=Z, K=K, dtype="bf16", seed=300 + i,
                    bias=bias, zipf=zipf)


@pytest.mark.parametrize("i", range(24))
def test_random_shape_forward(i):
    w = draw(i)
    print(f"[random forward {i}] {w.describe()} zipf={w.zipf} bias={w.bias}", flush=True)
    inp = make_inputs(w, device=DEV)
    residual = i % 3 == 0
    g = run_gpu(w, inp, residual=residual)
    if w.N > 0:
        packed = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
        gp = run_gpu(w, inp, residual=residual, packed=packed)
        assert torch.equal(g["y_t"], gp["y_t"]), "packed and row-major forwards differ"
    ref_inp = inp if residual else dict(inp, residual=None)
    print(i, check_forward(w, ref_inp, g), flush=True)


@pytest.mark.parametrize("i", range(8))
def test_random_shape_fp8(i):
    w = draw(100 + i, d_step=128)
    if w.N == 0:
        pytest.skip("no FFN expert")
    print(f"[random fp8 {i}] {w.describe()} zipf={w.zipf} bias={w.bias}", flush=True)
    inp = make_inputs(w, device=DEV, residual=False)
    ref_inp = dict(inp, residual=None)
    packed = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    g = run_gpu(w, inp, residual=False, fp8=True,
                packed=(m.moe_zc_pack_expert_weights_fp8(inp["w_gate"], inp["w_up"]), packed[1]))
    print(i, "gate/up fp8", check_forward(w, ref_inp, g, fp8=True), flush=True)
    g2 = run_gpu(w, inp, residual=False, fp8=True, down_fp8=True,
                 packed=m.moe_zc_pack_expert_weights_fp8(inp["w_gate"], inp["w_up"],
                                                         inp["w_down"]))
    print(i, "down fp8", check_forward(w, ref_inp, g2, fp8=True, down_fp8=True), flush=True)


@pytest.mark.parametrize("i", range(12))
def test_random_shape_backward(i):
    w = draw(200 + i)
    print(f"[random backward {i}] {w.describe()} zipf={w.zipf} bias={w.bias}", flush=True)
    inp = make_inputs(w, device=DEV)
    dy = make_upstream_grad(w, DEV)
    aux, (g,) = gpu_forward_backward(w, inp, dy)
    print(i, compare(w, inp, dy, aux, g), flush=True)


@pytest.mark.parametrize("i", range(12))
def test_random_wide_forward(i):
    w = draw_wide(i)
    print(f"[random wide forward {i}] {w.describe()} zipf={w.zipf} bias={w.bias}", flush=True)
    inp = make_inputs(w, device=DEV, residual=False)
    g = run_gpu(w, inp, residual=False)
    packed = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    gp = run_gpu(w, inp, residual=False, packed=packed)
    assert torch.equal(g["y_t"], gp["y_t"]), "packed and row-major forwards differ"
    print(i, check_forward(w, dict(inp, residual=None), g), flush=True)


@pytest.mark.parametrize("i", range(6))
def test_random_wide_backward(i):
    w = draw_wide(100 + i)
    print(f"[random wide backward {i}] {w.describe()} zipf={w.zipf} bias={w.bias}", flush=True)
    inp = make_inputs(w, device=DEV)
    dy = make_upstream_grad(w, DEV)
    aux, (g,) = gpu_forward_backward(w, inp, dy)
    print(i, compare(w, inp, dy, aux, g, dx_tokens=np.arange(min(w.T, 1024))), flush=True)


@pytest.mark.parametrize("i", range(6))
def test_random_wide_fp8(i):
    w = draw_wide(200 + i, d_choices=(128,))
    print(f"[random wide fp8 {i}] {w.describe()} zipf={w.zipf} bias={w.bias}", flush=True)
    inp = make_inputs(w, device=DEV, residual=False)
    ref_inp = dict(inp, residual=None)
    packed = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    g = run_gpu(w, inp, residual=False, fp8=True,
                packed=(m.moe_zc_pack_expert_weights_fp8(inp["w_gate"], inp["w_up"]), packed[1]))
    print(i, "gate/up fp8", check_forward(w, ref_inp, g, fp8=True), flush=True)
    g2 = run_gpu(w, inp, residual=False, fp8=True, down_fp8=True,
                 packed=m.moe_zc_pack_expert_weights_fp8(inp["w_gate"], inp["w_up"],
                                                         inp["w_down"]))
    print(i, "down fp8", check_forward(w, ref_inp, g2, fp8=True, down_fp8=True), flush=True)
