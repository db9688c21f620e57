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


def test_full_size_backward_prefill():
    """The training step that `bench.py --pass backward` times, at the prefill
    size: packed forward saving a | u, then moe_zc_backward from the saved
    values and the packed weight transposes.  Routing is checked for every
    token.  dx is checked on a token sample, since a token's dx depends only
    on that token.  The weight gradients are checked for two experts, each
    from exactly the tokens routed to it.  Bar: max |G - G_ref| <= 1e-2 *
    max |G_ref| per checked tensor.  dW_router needs every token's expert
    outputs and is covered at the mid and edge sizes (its dl enters dx here)."""
    from oracle import backward as obwd
    from workloads import make_upstream_grad
    w = get_workload("prefill")
    print("[backward prefill] generating inputs", flush=True)
    inp = make_inputs(w, device=DEV)
    dy = make_upstream_grad(w, DEV)
    aux = m.alloc_aux(w.T, w.N, w.Z, w.K, DEV, keys=m.AUX_KEYS + ("act",), I=w.I)
    gu, dn = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    m.moe_zc_forward_packed(inp["x"], inp["w_router"], inp["bias"], gu, dn, w.N, w.Z, w.K, w.I,
                            residual=inp["residual"], aux=aux)
    torch.cuda.synchronize()
    del gu, dn
    tr = m.moe_zc_transpose_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    print("[backward prefill] backward", flush=True)
    g = m.moe_zc_backward(inp["x"], inp["w_router"], None, None, tr, aux, dy, w.N, w.Z, w.K, w.I)
    torch.cuda.synchronize()
    del tr
    l32 = aux["logits"].cpu().numpy()
    bias = inp["bias"].cpu().numpy()
    idx = aux["topk_idx"].cpu().numpy()
    assert np.array_equal(idx, oracle.route(l32, bias, w.K, w.N)["idx"]), "routing"

    def check(name, got, want):
        scale = np.abs(want).max()
        err = np.abs(got - want).max()
        print(f"[backward prefill] {name}: max|err| / max|ref| = {err / scale:.2e}", flush=True)
        assert err <= 1e-2 * scale, f"{name}: {err:.3e} > 1e-2 * {scale:.3e}"

    rng = np.random.default_rng(3)
    s = np.sort(rng.choice(w.T, 4, replace=False))
    st = torch.from_numpy(s).to(DEV)
    ref = obwd.backward(inp["x"][st], inp["w_router"], bias, inp["w_gate"], inp["w_up"],
                        inp["w_down"], w.N, w.Z, w.K, dy[st], logits32=l32[s], experts=[])
    check(f"dx tokens {s.tolist()}", g["dx"][st].float().cpu().double().numpy(), ref["dx"])
    for e in np.sort(rng.choice(np.unique(idx[idx < w.N]), 2, replace=False)):
        tt = np.nonzero((idx == e).any(axis=1))[0]
        ti = torch.from_numpy(tt).to(DEV)
        ref = obwd.backward(inp["x"][ti], inp["w_router"], bias, inp["w_gate"], inp["w_up"],
                            inp["w_down"], w.N, w.Z, w.K, dy[ti], logits32=l32[tt],
                            experts=[int(e)], want_dx=False)
        for k in ("dw_gate", "dw_up", "dw_down"):
            check(f"{k}[{e}] ({len(tt)} rows)", g[k][int(e)].cpu().double().numpy(), ref[k][int(e)])
