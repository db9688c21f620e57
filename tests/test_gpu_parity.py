"""GPU parity of the HIP path against the fp64 oracle: routing, grouping,
PID update and the whole layer on small and mid shapes, edge cases,
determinism.  Needs an MI355X and the built library."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_bias_amd as m
import oracle
from gpu_check import check_forward, run_gpu
from workloads import Workload, get_workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _inputs(w, **over):
    inp = make_inputs(w, device=DEV)
    for k, v in over.items():
        inp[k] = v
    return inp


# ---------------------------------------------------------------- routing --
@pytest.mark.parametrize("T,E,K,q", [(4096, 768, 12, None), (1000, 96, 8, None),
                                     (333, 12, 3, None), (256, 2048, 32, None),
                                     (2048, 768, 12, 8.0), (517, 32, 32, 4.0),
                                     (130, 64, 1, 2.0)])
def test_route_bit_exact(T, E, K, q):
    """moe_zc_route on given fp32 logits equals the oracle bit for bit
    (indices, order and gates).  q quantises logits and bias to multiples of
    1/q so that exact key ties occur and the lowest index must win."""
    g = torch.Generator().manual_seed(T * 7 + E)
    logits = torch.randn(T, E, generator=g) * 2.0
    bias = (torch.rand(E, generator=g) - 0.5) * 0.02
    if q is not None:
        logits = torch.round(logits * q) / q
        bias = torch.zeros(E)
    loads = torch.full((E,), -7, dtype=torch.int32, device=DEV)   # overwritten, not added to
    idx, gate = m.moe_zc_route(logits.to(DEV), bias.to(DEV), K, loads=loads)
    torch.cuda.synchronize()
    rt = oracle.route(logits.numpy(), bias.numpy(), K, min(E, 1))
    assert np.array_equal(idx.cpu().numpy(), rt["idx"])
    assert np.array_equal(gate.cpu().numpy(), rt["gate"])
    assert np.array_equal(loads.cpu().numpy(), rt["loads"])
    if q is not None:                                  # exact key ties were present
        assert (np.diff(np.sort(rt["key"], axis=1), axis=1) == 0).any()


@pytest.mark.parametrize("case", ["few_lanes_hold_the_top", "boundary_64", "all_equal",
                                  "two_levels"])
def test_route_bit_exact_structured(case):
    """Routing of logits whose best experts crowd into a few of the 64 lanes
    of a wavefront (lane l holds experts l, l + 64, ...), so that more than 64
    elements qualify as candidates and the selection takes its arg-max rounds
    ("few_lanes_hold_the_top", 6 lanes x 12 experts raised); exactly at and
    around that count ("boundary_64"); all keys equal (the lowest indices win);
    and two exact key levels.  Equal to the oracle bit for bit."""
    T, E, K = 257, 768, 12
    g = torch.Generator().manual_seed(11)
    logits = torch.randn(T, E, generator=g)
    bias = (torch.rand(E, generator=g) - 0.5) * 0.02
    lane = torch.arange(E) % 64
    if case == "few_lanes_hold_the_top":
        logits[:, lane < 6] += 8.0
        bias = torch.zeros(E)             # a bias would reorder the raised experts' keys
    elif case == "boundary_64":
        # token t raises the experts of its first 1 + t % 8 lanes, so the count
        # of qualifying elements moves across 64 from token to token
        for t in range(T):
            logits[t, lane < 1 + t % 8] += 8.0
        bias = torch.zeros(E)
    elif case == "all_equal":
        logits = torch.zeros(T, E)
        bias = torch.zeros(E)
    else:
        logits = torch.where(torch.rand(T, E, generator=g) < 0.05, torch.tensor(3.0),
                             torch.tensor(0.0))
        bias = torch.zeros(E)
    idx, gate = m.moe_zc_route(logits.to(DEV), bias.to(DEV), K)
    torch.cuda.synchronize()
    rt = oracle.route(logits.numpy(), bias.numpy(), K, 1)
    if case == "few_lanes_hold_the_top":
        assert (candidate_counts(rt["key"], K) > 64).all()
    if case == "boundary_64":
        c = candidate_counts(rt["key"], K)
        assert (c > 64).any() and (c <= 64).any()
    assert np.array_equal(idx.cpu().numpy(), rt["idx"])
    assert np.array_equal(gate.cpu().numpy(), rt["gate"])


def candidate_counts(key, K):
    """Per token: elements not worse, in the order (key descending, index
    ascending), than the K-th best of the 64 lane bests (lane l: experts l,
    l + 64, ...).  More than 64 sends the kernel to its arg-max rounds."""
    T, E = key.shape
    j = np.arange(E)
    out = np.empty(T, np.int64)
    for t in range(T):
        kk = key[t]
        o = np.lexsort((j, -kk))                       # best first
        seen, best = set(), []
        for e in o:
            if e % 64 not in seen:
                seen.add(e % 64)
                best.append(e)
                if len(best) == K:
                    break
        tau = best[-1]
        out[t] = np.sum((kk > kk[tau]) | ((kk == kk[tau]) & (j <= tau)))
    return out


def test_route_loads_with_no_tokens_are_zero():
    loads = torch.full((40,), 5, dtype=torch.int32, device=DEV)
    m.moe_zc_route(torch.zeros(0, 40, device=DEV), torch.zeros(40, device=DEV), 3, loads=loads)
    torch.cuda.synchronize()
    assert (loads.cpu() == 0).all()


def test_route_refuses_topk_above_limit():
    logits = torch.zeros(8, 40, device=DEV)
    with pytest.raises(m.MoeZcError) as ei:
        m.moe_zc_route(logits, torch.zeros(40, device=DEV), 33)
    assert ei.value.code == 3


# ------------------------------------------------------------------- PID --
def test_pid_matches_oracle_over_steps():
    E = 384
    r = np.random.default_rng(5)
    target = np.full(E, 256.0, np.float32)
    bias = torch.zeros(E, device=DEV)
    pid = m.PidState(E, DEV, kp=0.6, ki=0.3, kd=0.15)
    ob, oe1, oe2 = np.zeros(E), np.zeros(E), np.zeros(E)
    tg = torch.from_numpy(target).to(DEV)
    for step in range(6):
        loads = r.integers(0, 700, E).astype(np.int32)
        m.moe_zc_bias_update(torch.from_numpy(loads).to(DEV), tg, bias, pid)
        ob, oe1, oe2 = oracle.pid_step(loads, target, ob, oe1, oe2, 0.6, 0.3, 0.15)
        torch.cuda.synchronize()
        assert np.allclose(bias.cpu().numpy(), ob, rtol=1e-6, atol=1e-7), step
        assert np.allclose(pid.e_prev.cpu().numpy(), oe1, rtol=1e-6, atol=1e-9)


def test_pid_golden_on_gpu():
    import json, os
    G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pid_example.json")))
    gains = G["gains"]
    E = len(G["target"])
    bias = torch.tensor(G["bias0"], dtype=torch.float32, device=DEV)
    pid = m.PidState(E, DEV, **gains)
    tg = torch.tensor(G["target"], dtype=torch.float32, device=DEV)
    for st in G["steps"]:
        m.moe_zc_bias_update(torch.tensor(st["loads"], dtype=torch.int32, device=DEV), tg, bias, pid)
        torch.cuda.synchronize()
        assert bias.cpu().tolist() == st["bias"]          # exact binary fractions


# ------------------------------------------------------- whole layer -------
def test_tiny_f32_full():
    w = get_workload("tiny")
    inp = _inputs(w)
    rep = check_forward(w, inp, run_gpu(w, inp))
    assert rep["flips"] == 0


def test_mid_bf16_full_routing_sampled_outputs():
    """The mid layer with no residual (y is the expert mixture alone, so the
    bar scales with it); the residual is covered at the edge shapes."""
    w = get_workload("mid")
    inp = _inputs(w, residual=None)
    sample = np.random.default_rng(0).choice(w.T, 384, replace=False)
    rep = check_forward(w, inp, run_gpu(w, inp, residual=False), y_tokens=np.sort(sample))
    print(rep)


def _edge(T=200, d=128, I=128, N=8, Z=4, K=3, dtype="bf16", seed=3, bias=("uniform", 0.05)):
    return Workload("edge", T=T, d=d, I=I, N=N, Z=Z, K=K, dtype=dtype, seed=seed, bias=bias)


EDGE = {
    "T1": dict(T=1),
    "T65_ragged": dict(T=65),
    "T130_f32": dict(T=130, d=64, I=64, dtype="f32"),
    "Z0": dict(N=8, Z=0, K=2),
    "K_eq_E": dict(N=5, Z=3, K=8),
    "K1": dict(K=1),
    "N0_all_identity": dict(N=0, Z=6, K=3),
    "few_rows_per_expert": dict(T=64, N=64, Z=32, K=8),       # 32-row tile variant
    "many_experts_topk32": dict(T=96, N=1024, Z=1024, K=32, d=64 * 2, I=128),
    "wide_rows": dict(T=300, d=512, I=256, N=4, Z=2, K=2),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_shapes(name):
    w = _edge(**EDGE[name])
    inp = _inputs(w)
    rep = check_forward(w, inp, run_gpu(w, inp))
    print(name, rep)


def test_all_ffn_biased_away_gives_identity_closed_form():
    w = _edge(T=150)
    inp = _inputs(w)
    b = torch.zeros(w.E, device=DEV)
    b[: w.N] = -10.0
    inp["bias"] = b
    g = run_gpu(w, inp)
    assert (g["topk_idx"] >= w.N).all() and g["offsets"][w.N] == 0
    # y = (sum_k g_k) x + r, from the GPU's own gates: the identity path alone
    x = inp["x"].float().cpu().double().numpy()
    r = inp["residual"].float().cpu().double().numpy()
    ref = g["topk_gate"].astype(np.float64).sum(axis=1, keepdims=True) * x + r
    assert np.abs(g["y"] - ref).max() <= 1e-2 * np.abs(ref).max()
    check_forward(w, inp, g)


def test_one_hot_expert_takes_every_token():
    w = _edge(T=700, K=2)
    inp = _inputs(w)
    b = torch.zeros(w.E, device=DEV)
    b[3] = 10.0
    inp["bias"] = b
    g = run_gpu(w, inp)
    assert (g["topk_idx"][:, 0] == 3).all() and g["loads"][3] == w.T
    check_forward(w, inp, g)


def test_no_residual():
    w = _edge(T=129)
    inp = _inputs(w)
    check_forward(w, dict(inp, residual=None), run_gpu(w, inp, residual=False))


def test_deterministic_and_ignores_workspace_contents():
    w = get_workload("mid").with_tokens(1024)
    inp = _inputs(w)
    need = m.moe_zc_workspace_size(w.T, w.d, w.I, w.N, w.Z, w.K, torch.bfloat16)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    ws.fill_(0)
    a = run_gpu(w, inp, workspace=ws)
    ws.fill_(0xFF)                       # NaN in every fp32/bf16 slot
    b = run_gpu(w, inp, workspace=ws)
    c = run_gpu(w, inp)
    assert torch.equal(a["y_t"], b["y_t"]) and torch.equal(a["y_t"], c["y_t"])
    for k in ("logits", "topk_idx", "topk_gate", "loads", "perm", "pos"):
        assert np.array_equal(a[k], b[k]), k


def test_stage_events_time_every_stage():
    w = get_workload("mid").with_tokens(512)
    inp = _inputs(w)
    ev = m.StageEvents()
    run_gpu(w, inp, events=ev)
    ms = ev.stage_ms()
    assert set(ms) == set(m.STAGE_NAMES)
    assert all(v >= 0.0 for v in ms.values())
