"""GPU parity at the full sizes of the decode, prefill and skewed workloads, in
the launch configuration the benchmark times (moe_zc_forward_packed on packed
expert weights, same sizes, same library), plus bitwise equality with the
row-major moe_zc_forward.  Routing and grouping are checked for every token;
the layer output on a seeded sample of tokens that the oracle evaluates one
by one (tokens are independent, so a sample is exact)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_bias_amd as m
import oracle
from gpu_check import check_forward, gpu_expert_getter, run_gpu
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("name,n_sample", [("decode", 10), ("prefill", 6)])
def test_full_size_layer(name, n_sample):
    w = get_workload(name)
    print(f"[{name}] generating inputs", flush=True)
    inp = make_inputs(w, device=DEV)
    packed = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    g = run_gpu(w, inp, packed=packed)
    y_rowmajor = run_gpu(w, inp)["y_t"]
    assert torch.equal(g["y_t"], y_rowmajor), "packed and row-major forwards differ"
    del y_rowmajor
    sample = np.sort(np.random.default_rng(1).choice(w.T, n_sample, replace=False))
    print(f"[{name}] checking against the oracle, tokens {sample.tolist()}", flush=True)
    rep = check_forward(w, inp, g, y_tokens=sample, get_expert=gpu_expert_getter(inp))
    print(name, rep, flush=True)
    ffn_per_tok = rep["S"] / w.T
    if name == "prefill":
        assert 7.8 <= ffn_per_tok <= 8.2, ffn_per_tok


def test_skew_layer_then_pid_step_then_reroute():
    w = get_workload("skew")
    print("[skew] generating inputs", flush=True)
    inp = make_inputs(w, device=DEV)
    g1 = run_gpu(w, inp)
    sample = np.sort(np.random.default_rng(2).choice(w.T, 6, replace=False))
    rep1 = check_forward(w, inp, g1, y_tokens=sample, get_expert=gpu_expert_getter(inp))
    print("skew before", rep1, flush=True)
    # one PID step toward uniform load, from the loads this forward measured
    target = np.full(w.E, w.T * w.K / w.E, np.float32)
    pid = m.PidState(w.E, DEV, kp=0.5, ki=0.5, kd=0.0)
    bias = inp["bias"].clone()
    loads_dev = torch.from_numpy(g1["loads"]).to(DEV)
    m.moe_zc_bias_update(loads_dev, torch.from_numpy(target).to(DEV), bias, pid)
    torch.cuda.synchronize()
    # oracle: same step from its own routing's loads
    x = inp["x"].cpu()
    l32 = oracle.router_logits(x, inp["w_router"].cpu()).astype(np.float32)
    rt = oracle.route(l32, inp["bias"].cpu().numpy(), w.K, w.N)
    nb, _, _ = oracle.pid_step(rt["loads"], target, inp["bias"].cpu().numpy(),
                               np.zeros(w.E), np.zeros(w.E), 0.5, 0.5, 0.0)
    dl = np.abs(g1["loads"] - rt["loads"]).astype(np.float64)
    slack = dl / target.sum() + 1e-7                   # near-tie flips move loads by a few
    assert (np.abs(bias.cpu().numpy() - nb) <= slack + 1e-6 * np.abs(nb)).all()
    inp2 = dict(inp, bias=bias)
    g2 = run_gpu(w, inp2)
    rep2 = check_forward(w, inp2, g2, y_tokens=sample, get_expert=gpu_expert_getter(inp))
    print("skew after", rep2, flush=True)
    l1, l2 = g1["loads"][: w.N].astype(float), g2["loads"][: w.N].astype(float)
    assert l2.max() / l2.mean() < l1.max() / l1.mean()          # busiest expert relieved
    assert np.abs(g2["loads"] - target).sum() < np.abs(g1["loads"] - target).sum()
