"""The bias controller run closed-loop on the GPU over a sequence of batches.

Each batch goes through moe_zc_forward with the current bias, then
moe_zc_bias_update moves the bias from that batch's loads, toward a target
that asks for a chosen number of FFN experts per token (the controller's
purpose on the LongCat pages: hold the compute activated per token near a
budget).  Every step is checked against the oracle on the same inputs:
  - loads equal the oracle's routing of the GPU's fp32 logits with the GPU's
    bias, bit for bit;
  - the new bias and error history equal the oracle's PID step on those loads
    (state stored in fp32, as the oracle's closed loop stores it);
and the whole trajectory is compared with the oracle's own closed loop run
from its own fp64 logits (equal up to routing near-ties)."""
import dataclasses

import numpy as np
import pytest
import torch

import mixture_experts_layer_bias_amd as m
import oracle
from gpu_check import LOGIT_TOL
from workloads import Workload, make_inputs
from workloads.gen import make_router_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

# Zipf(1.1) offsets over the FFN experts: the unbiased routing sends about 3.1
# of 8 slots to FFN experts (mostly the few top-ranked ones); the budget asks
# for 5, spread evenly
W = Workload("loop", T=2048, d=1024, I=128, N=64, Z=32, K=8, dtype="bf16", seed=21,
             bias=("zero",), zipf=(1.1, 2.0))
BUDGET = 5.0
STEPS = 12
GAINS = (0.5, 0.5, 0.0)


def test_closed_loop_pid_tracks_budget():
    w = W
    inp = make_inputs(w, device=DEV)
    batches = [inp["x"]]
    for s in range(1, STEPS):
        xs, _, _ = make_router_inputs(dataclasses.replace(w, seed=w.seed + 100 * s))
        batches.append(xs.to(DEV))
    target_np = oracle.budget_target(w.T, w.K, w.N, w.Z, BUDGET).astype(np.float32)
    target = torch.from_numpy(target_np).to(DEV)
    bias = inp["bias"].clone()
    pid = m.PidState(w.E, DEV, *GAINS)
    wr64 = inp["w_router"].cpu().double().numpy()
    gpu_ffn, oracle_logits = [], []
    for s, x in enumerate(batches):
        print(f"[closed loop] step {s}", flush=True)
        aux = m.alloc_aux(w.T, w.N, w.Z, w.K, DEV)
        b_before = bias.cpu().numpy().copy()
        e1_before = pid.e_prev.cpu().numpy().copy()
        e2_before = pid.e_prev2.cpu().numpy().copy()
        m.moe_zc_forward(x, inp["w_router"], bias, inp["w_gate"], inp["w_up"], inp["w_down"],
                         w.N, w.Z, w.K, aux=aux)
        m.moe_zc_bias_update(aux["loads"], target, bias, pid)
        torch.cuda.synchronize()
        l32 = aux["logits"].cpu().numpy()
        loads = aux["loads"].cpu().numpy()
        # router logits within the logit tolerance of fp64
        l64 = x.float().cpu().double().numpy() @ wr64.T
        assert np.abs(l32.astype(np.float64) - l64).max() <= LOGIT_TOL
        oracle_logits.append(l64.astype(np.float32))
        # routing of the GPU's logits with the GPU's bias: bit-exact loads
        rt = oracle.route(l32, b_before, w.K, w.N)
        assert np.array_equal(loads, rt["loads"]), f"step {s}: loads differ"
        assert np.array_equal(aux["topk_idx"].cpu().numpy(), rt["idx"])
        gpu_ffn.append(float(oracle.ffn_count_per_token(rt["idx"], w.N).mean()))
        # one PID step on those loads, state stored in fp32
        nb, ne1, ne2 = oracle.pid_step(loads, target_np, b_before, e1_before, e2_before, *GAINS)
        assert np.array_equal(bias.cpu().numpy(), nb.astype(np.float32)), f"step {s}: bias"
        assert np.array_equal(pid.e_prev.cpu().numpy(), ne1.astype(np.float32))
        assert np.array_equal(pid.e_prev2.cpu().numpy(), ne2.astype(np.float32))
    print("FFN experts per token, GPU loop:", np.round(gpu_ffn, 3), flush=True)
    # the oracle's own closed loop from its own logits
    ref = oracle.closed_loop(oracle_logits, inp["bias"].cpu().numpy(), target_np, w.K, w.N,
                             *GAINS)
    print("FFN experts per token, oracle loop:", np.round(ref["ffn_per_token"], 3), flush=True)
    assert np.abs(np.array(gpu_ffn) - ref["ffn_per_token"]).max() < 0.01
    assert np.abs(bias.cpu().numpy() - ref["bias"][-1]).max() < 1e-3
    # the loop pulls the FFN count from its unbiased level to the budget
    assert gpu_ffn[0] < BUDGET - 1.5
    assert abs(np.mean(gpu_ffn[-4:]) - BUDGET) < 0.25, gpu_ffn



def test_pid_save_restore_resumes_bit_for_bit():
    """The controller's whole state is (bias, e_prev, e_prev2): n straight
    closed-loop steps equal k steps, a save of that state to the host, a
    restore into fresh device buffers and a fresh PidState, and n - k more
    steps, bit for bit (bias, both histories, and every step's loads)."""
    w = W
    inp = make_inputs(w, device=DEV)
    packed = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    target = torch.from_numpy(oracle.budget_target(w.T, w.K, w.N, w.Z, 5.0).astype(np.float32)).to(DEV)
    n, k = 8, 3

    def run(bias, pid, steps, loads_log):
        aux = m.alloc_aux(w.T, w.N, w.Z, w.K, DEV, keys=("loads", "offsets"))
        for _ in range(steps):
            m.moe_zc_forward_packed(inp["x"], inp["w_router"], bias, packed[0], packed[1], w.N,
                                    w.Z, w.K, w.I, aux=aux)
            loads_log.append(aux["loads"].cpu().numpy().copy())
            m.moe_zc_bias_update(aux["loads"], target, bias, pid)
        torch.cuda.synchronize()

    straight_loads, resumed_loads = [], []
    b1 = inp["bias"].clone()
    p1 = m.PidState(w.E, DEV, kp=0.5, ki=0.3, kd=0.2)
    run(b1, p1, n, straight_loads)
    b2 = inp["bias"].clone()
    p2 = m.PidState(w.E, DEV, kp=0.5, ki=0.3, kd=0.2)
    run(b2, p2, k, resumed_loads)
    saved = {"bias": b2.cpu().numpy(), "e1": p2.e_prev.cpu().numpy(),
             "e2": p2.e_prev2.cpu().numpy(), "gains": (p2.kp, p2.ki, p2.kd)}
    del b2, p2
    b3 = torch.from_numpy(saved["bias"]).to(DEV)
    p3 = m.PidState(w.E, DEV, *saved["gains"])
    p3.e_prev.copy_(torch.from_numpy(saved["e1"]))
    p3.e_prev2.copy_(torch.from_numpy(saved["e2"]))
    run(b3, p3, n - k, resumed_loads)
    for s, (a, b) in enumerate(zip(straight_loads, resumed_loads)):
        assert np.array_equal(a, b), f"loads differ at step {s}"
    assert torch.equal(b1, b3)
    assert torch.equal(p1.e_prev, p3.e_prev)
    assert torch.equal(p1.e_prev2, p3.e_prev2)
    # the loop did move the bias (the test would be empty otherwise)
    assert not torch.equal(b1, inp["bias"])
