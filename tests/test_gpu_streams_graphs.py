"""Stream and graph behaviour the C ABI promises: the entry points that take
a workspace keep no mutable global state, so calls on different streams with
their own workspaces may run concurrently; they allocate nothing, synchronise
nothing and record no memset, so a forward, the bias update and the backward
can be captured in a HIP graph and replayed.  Every result is compared bit for
bit with the same call run eagerly on the default stream."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_bias_amd as m
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _w(seed, T=700, d=256, I=256, N=16, Z=8, K=4):
    return Workload("streams", T=T, d=d, I=I, N=N, Z=Z, K=K, dtype="bf16", seed=seed,
                    bias=("uniform", 0.05))


def _packed_forward(w, inp, packed, ws, out, bias=None, aux=None):
    return m.moe_zc_forward_packed(inp["x"], inp["w_router"], inp["bias"] if bias is None else bias,
                                   packed[0], packed[1], w.N, w.Z, w.K, w.I,
                                   residual=inp["residual"], out=out, aux=aux, workspace=ws)


def _ws(w):
    n = m.moe_zc_workspace_size(w.T, w.d, w.I, w.N, w.Z, w.K, torch.bfloat16)
    return torch.empty(n, dtype=torch.uint8, device=DEV)


def test_concurrent_streams_match_eager():
    """Two layers (different inputs and weights) on two streams, interleaved
    three times without synchronisation, give exactly their eager results."""
    ws_ = [_w(11), _w(12, T=513, N=24, Z=8, K=6)]
    inps = [make_inputs(w, device=DEV) for w in ws_]
    packs = [m.moe_zc_pack_expert_weights(i["w_gate"], i["w_up"], i["w_down"]) for i in inps]
    ref = []
    for w, inp, pk in zip(ws_, inps, packs):
        ref.append(_packed_forward(w, inp, pk, _ws(w), None).clone())
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [_ws(w) for w in ws_]
    outs = [torch.empty_like(r) for r in ref]
    for _ in range(3):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                _packed_forward(ws_[i], inps[i], packs[i], wss[i], outs[i])
    torch.cuda.synchronize()
    for i in range(2):
        assert torch.equal(outs[i], ref[i]), f"stream {i} differs from the eager result"


def test_graph_replay_of_the_forward_matches_eager():
    """A captured forward replayed on new inputs copied into its static input
    buffer: every replay equals the eager forward of those inputs (eager work
    and synchronisation between replays)."""
    w = _w(21)
    inp = make_inputs(w, device=DEV)
    pk = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    ws = _ws(w)
    y = torch.empty(w.T, w.d, dtype=torch.bfloat16, device=DEV)
    aux = m.alloc_aux(w.T, w.N, w.Z, w.K, DEV)
    static_x = inp["x"].clone()
    static = dict(inp, x=static_x)
    _packed_forward(w, static, pk, ws, y, aux=aux)   # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _packed_forward(w, static, pk, ws, y, aux=aux)
    gen = torch.Generator().manual_seed(5)
    for rep in range(3):
        new_x = torch.randn(w.T, w.d, generator=gen).to(torch.bfloat16).to(DEV)
        static_x.copy_(new_x)
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        got_idx = aux["topk_idx"].clone()
        ea = m.alloc_aux(w.T, w.N, w.Z, w.K, DEV)
        eager = _packed_forward(w, dict(inp, x=new_x), pk, _ws(w), None, aux=ea)
        torch.cuda.synchronize()
        assert torch.equal(got, eager), f"replay {rep}: y differs from eager"
        assert torch.equal(got_idx, ea["topk_idx"]), f"replay {rep}: routing differs"


def test_graph_of_forward_and_bias_update_matches_eager_loop():
    """Forward + PID step captured together and replayed six times follows the
    same bias trajectory, bit for bit, as the eager closed loop."""
    w = _w(31)
    inp = make_inputs(w, device=DEV)
    pk = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    target = torch.full((w.E,), w.T * w.K / w.E, dtype=torch.float32, device=DEV)

    def loop(use_graph):
        bias = inp["bias"].clone()
        pid = m.PidState(w.E, DEV, kp=0.5, ki=0.5, kd=0.1)
        aux = m.alloc_aux(w.T, w.N, w.Z, w.K, DEV, keys=("loads",))
        ws = _ws(w)
        y = torch.empty(w.T, w.d, dtype=torch.bfloat16, device=DEV)

        def step():
            _packed_forward(w, inp, pk, ws, y, bias=bias, aux=aux)
            m.moe_zc_bias_update(aux["loads"], target, bias, pid)

        traj = []
        if use_graph:
            g = torch.cuda.CUDAGraph()
            bias0 = bias.clone()
            step()                               # warm-up outside the capture
            torch.cuda.synchronize()
            bias.copy_(bias0)
            pid.e_prev.zero_()
            pid.e_prev2.zero_()
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                step()
            for _ in range(6):
                g.replay()
                torch.cuda.synchronize()
                traj.append(bias.cpu().numpy().copy())
        else:
            for _ in range(6):
                step()
                torch.cuda.synchronize()
                traj.append(bias.cpu().numpy().copy())
        return traj

    eager = loop(False)
    graph = loop(True)
    for i, (a, b) in enumerate(zip(eager, graph)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"step {i}: bias differs"
    assert not np.array_equal(eager[0], eager[-1]), "the bias should move"


@pytest.mark.parametrize("down_fp8", [False, True])
def test_graph_replay_of_the_fp8_forward_matches_eager(down_fp8):
    """The block-FP8 forward (x quantized in the call, and with down_fp8 h
    quantized in the gate/up epilogue) captured once and replayed on new
    inputs: every replay equals the eager FP8 forward of those inputs."""
    w = _w(41, d=384, I=256)
    inp = make_inputs(w, device=DEV)
    if down_fp8:
        gu, dn = m.moe_zc_pack_expert_weights_fp8(inp["w_gate"], inp["w_up"], inp["w_down"])
    else:
        gu = m.moe_zc_pack_expert_weights_fp8(inp["w_gate"], inp["w_up"])
        dn = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])[1]
    n = m.moe_zc_workspace_size_fp8(w.T, w.d, w.I, w.N, w.Z, w.K)
    ws = torch.empty(n, dtype=torch.uint8, device=DEV)
    y = torch.empty(w.T, w.d, dtype=torch.bfloat16, device=DEV)
    aux = m.alloc_aux(w.T, w.N, w.Z, w.K, DEV)
    static_x = inp["x"].clone()

    def fwd(x, ws_, out, aux_):
        return m.moe_zc_forward_packed_fp8(x, inp["w_router"], inp["bias"], gu, dn, w.N, w.Z, w.K,
                                           w.I, residual=inp["residual"], out=out, aux=aux_,
                                           workspace=ws_, down_fp8=down_fp8)

    fwd(static_x, ws, y, aux)                    # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(static_x, ws, y, aux)
    gen = torch.Generator().manual_seed(9)
    for rep in range(3):
        new_x = torch.randn(w.T, w.d, generator=gen).to(torch.bfloat16).to(DEV)
        static_x.copy_(new_x)
        g.replay()
        torch.cuda.synchronize()
        got = y.clone()
        ea = m.alloc_aux(w.T, w.N, w.Z, w.K, DEV)
        eager = fwd(new_x, torch.empty_like(ws), None, ea)
        torch.cuda.synchronize()
        assert torch.equal(got, eager), f"replay {rep}: y differs from eager"
        assert torch.equal(aux["topk_idx"], ea["topk_idx"]), f"replay {rep}: routing differs"


def test_graph_replay_of_the_training_step_matches_eager():
    """Forward saving a | u plus the backward, captured together and replayed
    on new x and dy copied into their static buffers: every gradient of every
    replay equals, bit for bit, the eager forward and backward of those
    inputs."""
    w = _w(51, T=613, N=12, Z=4, K=4)
    inp = make_inputs(w, device=DEV)
    pk = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    tr = m.moe_zc_transpose_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    keys = m.AUX_KEYS + ("act",)
    nb = m.moe_zc_backward_workspace_size(w.T, w.d, w.I, w.N, w.Z, w.K)

    def buffers():
        aux = m.alloc_aux(w.T, w.N, w.Z, w.K, DEV, keys=keys, I=w.I)
        y = torch.empty(w.T, w.d, dtype=torch.bfloat16, device=DEV)
        return aux, y, _ws(w), torch.empty(nb, dtype=torch.uint8, device=DEV)

    def step(x, dy, aux, y, wsf, wsb, out):
        _packed_forward(w, dict(inp, x=x), pk, wsf, y, aux=aux)
        return m.moe_zc_backward(x, inp["w_router"], None, None, tr, aux, dy, w.N, w.Z, w.K, w.I,
                                 out=out, workspace=wsb)

    aux, y, wsf, wsb = buffers()
    static_x = inp["x"].clone()
    static_dy = torch.randn(w.T, w.d, generator=torch.Generator().manual_seed(3)).to(
        torch.bfloat16).to(DEV)
    g_out = step(static_x, static_dy, aux, y, wsf, wsb, None)   # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(static_x, static_dy, aux, y, wsf, wsb, g_out)
    gen = torch.Generator().manual_seed(13)
    for rep in range(3):
        new_x = torch.randn(w.T, w.d, generator=gen).to(torch.bfloat16).to(DEV)
        new_dy = torch.randn(w.T, w.d, generator=gen).to(torch.bfloat16).to(DEV)
        static_x.copy_(new_x)
        static_dy.copy_(new_dy)
        g.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in g_out.items()}
        got_y = y.clone()
        ea, ey, ewf, ewb = buffers()
        eager = step(new_x, new_dy, ea, ey, ewf, ewb, None)
        torch.cuda.synchronize()
        assert torch.equal(got_y, ey), f"replay {rep}: y differs from eager"
        for k in ("dx", "dw_router", "dw_gate", "dw_up", "dw_down"):
            assert torch.equal(got[k], eager[k]), f"replay {rep}: {k} differs from eager"
        assert got["dw_gate"].abs().max() > 0, "the gradients should be non-trivial"
