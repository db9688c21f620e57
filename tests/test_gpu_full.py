"""GPU parity at the full sizes of the decode, prefill and skewed workloads, in
the launch configuration the benchmark times (moe_zc_forward_packed on packed
expert weights, same sizes, same library), plus bitwise equality with the
row-major moe_zc_forward.  Routing and grouping are checked for every token.

The layer output is checked with no residual, so y is the expert mixture
alone and the bar 1e-2 * max |y_ref| scales with what the experts contribute
(with the N(0, 1) residual added, max |y_ref| would be set by the residual and
the bar would be blind to a wrong weight panel; the residual itself is covered
at the edge shapes).  y is checked on a seeded token sample that the oracle
evaluates one by one (tokens are independent, so a sample is exact): every
token at decode; at prefill and skew 48 random tokens plus tokens whose rows
lie in the second row tile of an expert split over two tiles.  The saved
pre-activations (aux "act") are checked on every row and hidden unit of four
whole experts: the most loaded (split over two tiles), the least loaded and
two random ones, which covers every weight panel of their gate/up tiles."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_bias_amd as m
import oracle
from gpu_check import (act_experts, check_act, check_forward, gpu_expert_getter, run_gpu,
                       sample_tokens)
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_full_size_layer(name):
    w = get_workload(name)
    print(f"[{name}] generating inputs", flush=True)
    inp = make_inputs(w, device=DEV, residual=False)
    packed = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    g = run_gpu(w, inp, residual=False, packed=packed, act=True)
    del packed
    y_rowmajor = run_gpu(w, inp, residual=False)["y_t"]
    assert torch.equal(g["y_t"], y_rowmajor), "packed and row-major forwards differ"
    del y_rowmajor
    rng = np.random.default_rng(1)
    sample = np.arange(w.T) if name == "decode" else sample_tokens(g, w.N, rng)
    print(f"[{name}] checking y on {len(sample)} tokens against the oracle", flush=True)
    rep = check_forward(w, inp, g, y_tokens=sample, get_expert=gpu_expert_getter(inp))
    print(name, rep, flush=True)
    assert rep["tokens_checked"] >= min(w.T, 60)
    experts = act_experts(g["loads"], w.N, rng)
    print(f"[{name}] checking the pre-activations of experts {experts}", flush=True)
    print(name, "act", check_act(w, inp, g, experts), flush=True)
    ffn_per_tok = rep["S"] / w.T
    if name == "prefill":
        assert 7.8 <= ffn_per_tok <= 8.2, ffn_per_tok
        assert g["loads"][: w.N].max() > 256            # a split expert was checked whole


def test_skew_layer_then_pid_step_then_reroute():
    w = get_workload("skew")
    print("[skew] generating inputs", flush=True)
    inp = make_inputs(w, device=DEV, residual=False)
    g1 = run_gpu(w, inp, residual=False, act=True)
    rng = np.random.default_rng(2)
    sample = sample_tokens(g1, w.N, rng)
    rep1 = check_forward(w, inp, g1, y_tokens=sample, get_expert=gpu_expert_getter(inp))
    print("skew before", rep1, flush=True)
    print("skew act", check_act(w, inp, g1, act_experts(g1["loads"], w.N, rng)), flush=True)
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
    g2 = run_gpu(w, inp2, residual=False)
    rep2 = check_forward(w, inp2, g2, y_tokens=sample_tokens(g2, w.N, rng),
                         get_expert=gpu_expert_getter(inp))
    print("skew after", rep2, flush=True)
    l1, l2 = g1["loads"][: w.N].astype(float), g2["loads"][: w.N].astype(float)
    assert l2.max() / l2.mean() < l1.max() / l1.mean()          # busiest expert relieved
    assert np.abs(g2["loads"] - target).sum() < np.abs(g1["loads"] - target).sum()


@pytest.mark.parametrize("name", ["prefill", "skew"])
def test_full_size_backward(name):
    """The training step that `bench.py --pass backward` times, at the prefill
    size and at the skewed workload's (where the busiest expert holds
    thousands of rows, so its weight gradients are long reductions): packed
    forward saving a | u, then moe_zc_backward from the saved values and the
    packed weight transposes.  Routing is checked for every token.  dx is
    checked on a token sample, since a token's dx depends only on that token.
    The weight gradients are checked for the most loaded expert and a random
    one, each from exactly the tokens routed to it.  Bar: max |G - G_ref| <=
    1e-2 * max |G_ref| per checked tensor.

    dW_router sums every token's dl x^T, and dl needs the token's expert
    outputs, so with a dense dy the oracle cannot form it at this size.  The
    gradients are linear in dy and each token's share depends only on that
    token, so a second backward in the same configuration takes a dy that is
    zero outside 8 sampled tokens: then dW_router is exactly the oracle's sum
    over those tokens (checked whole, [E, d]), dx is zero on every other token,
    and the weight gradients are zero for every expert the sample did not
    choose."""
    from oracle import backward as obwd
    from workloads import make_upstream_grad
    w = get_workload(name)
    tag = f"[backward {name}]"
    print(f"{tag} generating inputs", flush=True)
    inp = make_inputs(w, device=DEV)
    dy = make_upstream_grad(w, DEV)
    aux = m.alloc_aux(w.T, w.N, w.Z, w.K, DEV, keys=m.AUX_KEYS + ("act",), I=w.I)
    gu, dn = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    m.moe_zc_forward_packed(inp["x"], inp["w_router"], inp["bias"], gu, dn, w.N, w.Z, w.K, w.I,
                            residual=inp["residual"], aux=aux)
    torch.cuda.synchronize()
    del gu, dn
    tr = m.moe_zc_transpose_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    print(f"{tag} backward", flush=True)
    g = m.moe_zc_backward(inp["x"], inp["w_router"], None, None, tr, aux, dy, w.N, w.Z, w.K, w.I)
    torch.cuda.synchronize()
    l32 = aux["logits"].cpu().numpy()
    bias = inp["bias"].cpu().numpy()
    idx = aux["topk_idx"].cpu().numpy()
    assert np.array_equal(idx, oracle.route(l32, bias, w.K, w.N)["idx"]), "routing"

    def check(what, got, want):
        scale = np.abs(want).max()
        err = np.abs(got - want).max()
        print(f"{tag} {what}: max|err| / max|ref| = {err / scale:.2e}", flush=True)
        assert err <= 1e-2 * scale, f"{what}: {err:.3e} > 1e-2 * {scale:.3e}"

    rng = np.random.default_rng(3)
    s = np.sort(rng.choice(w.T, 4, replace=False))
    st = torch.from_numpy(s).to(DEV)
    ref = obwd.backward(inp["x"][st], inp["w_router"], bias, inp["w_gate"], inp["w_up"],
                        inp["w_down"], w.N, w.Z, w.K, dy[st], logits32=l32[s], experts=[])
    check(f"dx tokens {s.tolist()}", g["dx"][st].float().cpu().double().numpy(), ref["dx"])
    loads = np.bincount(idx[idx < w.N].ravel(), minlength=w.N)
    busiest = int(np.argmax(loads))
    others = np.setdiff1d(np.unique(idx[idx < w.N]), [busiest])
    for e in sorted([busiest, int(rng.choice(others))]):
        tt = np.nonzero((idx == e).any(axis=1))[0]
        ti = torch.from_numpy(tt).to(DEV)
        ref = obwd.backward(inp["x"][ti], inp["w_router"], bias, inp["w_gate"], inp["w_up"],
                            inp["w_down"], w.N, w.Z, w.K, dy[ti], logits32=l32[tt],
                            experts=[int(e)], want_dx=False)
        for k in ("dw_gate", "dw_up", "dw_down"):
            check(f"{k}[{e}] ({len(tt)} rows)", g[k][int(e)].cpu().double().numpy(), ref[k][int(e)])
    del g

    s8 = np.sort(rng.choice(w.T, 8, replace=False))
    keep = torch.zeros(w.T, 1, dtype=dy.dtype, device=DEV)
    keep[torch.from_numpy(s8).to(DEV)] = 1
    dy8 = (dy * keep).contiguous()
    del dy
    print(f"{tag} sparse dy on tokens {s8.tolist()}", flush=True)
    g8 = m.moe_zc_backward(inp["x"], inp["w_router"], None, None, tr, aux, dy8, w.N, w.Z, w.K,
                           w.I)
    torch.cuda.synchronize()
    del tr
    chosen = np.unique(idx[s8][idx[s8] < w.N])
    e8 = int(chosen[0])
    st8 = torch.from_numpy(s8).to(DEV)
    ref = obwd.backward(inp["x"][st8], inp["w_router"], bias, inp["w_gate"], inp["w_up"],
                        inp["w_down"], w.N, w.Z, w.K, dy8[st8], logits32=l32[s8], experts=[e8])
    check("dW_router (sparse dy)", g8["dw_router"].cpu().double().numpy(), ref["dw_router"])
    check("dx sampled (sparse dy)", g8["dx"][st8].float().cpu().double().numpy(), ref["dx"])
    rest = torch.ones(w.T, dtype=torch.bool, device=DEV)
    rest[st8] = False
    assert not g8["dx"][rest].any(), "dx nonzero on a token with zero dy"
    for k in ("dw_gate", "dw_up", "dw_down"):
        check(f"{k}[{e8}] (sparse dy)", g8[k][e8].cpu().double().numpy(), ref[k][e8])
    unchosen = torch.ones(w.N, dtype=torch.bool, device=DEV)
    unchosen[torch.from_numpy(chosen).to(DEV)] = False
    for k in ("dw_gate", "dw_up", "dw_down"):
        flat = g8[k].view(w.N, -1)           # per-expert extremes: no copy of the gradients
        hi, lo = torch.amax(flat, dim=1), torch.amin(flat, dim=1)
        assert not (hi[unchosen].any() or lo[unchosen].any()), \
            f"{k} nonzero for an expert the sample did not choose"
