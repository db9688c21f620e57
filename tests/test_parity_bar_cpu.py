"""The full-size layer-output bar can see the expert path (CPU only).

The GPU tests at the full sizes score y against max |y - y_ref| <= 1e-2 *
max |y_ref| with no residual, so y_ref is the expert mixture alone.  This test
shows on the CPU, with the oracle, that the bar rejects a mistake confined to
one weight panel of the expert GEMMs at the prefill workload's shapes (d =
6144, I = 2048, N = 512 FFN + 256 zero experts, K = 12):
  * one gate/up panel wrong: hidden units 0..127 of every expert's W_gate and
    W_up zeroed (one 128-unit panel of the gate/up GEMM);
  * one down panel wrong: output columns 0..255 of every expert's W_down
    zeroed (one 256-column panel of the down GEMM).
Each planted mistake must move y by more than twice the bar.  It also reports
what the same mistakes do against the bar with the N(0, 1) residual added,
where max |y_ref| is set by the residual.

The mistakes are planted in the oracle's inputs on the CPU; no kernel is
touched.  Router inputs are the prefill workload's own (drawn on the CPU);
the expert weights are drawn with the workload's per-expert recipe on the CPU
generator (the GPU tests draw them on the device, a different stream of the
same distribution).  Sixteen seeded tokens keep the run to about half a
minute."""
import numpy as np
import torch

import oracle
from workloads import get_workload
from workloads.gen import make_expert_weights, make_router_inputs, _gen, _seed, _TAG_RES


def test_layer_output_bar_rejects_one_wrong_weight_panel_at_prefill():
    w = get_workload("prefill")
    x_all, wr, bias = make_router_inputs(w)
    rng = np.random.default_rng(11)
    toks = np.sort(rng.choice(w.T, 16, replace=False))
    x = x_all[torch.from_numpy(toks)]
    l32 = oracle.router_logits(x, wr).astype(np.float32)
    rt = oracle.route(l32, bias.numpy(), w.K, w.N)
    idx, gate = rt["idx"], rt["gate"]
    x64 = oracle.moe_zc._f64(x)
    rows = {k: np.zeros((len(toks), w.K, w.d)) for k in ("ref", "gate_up", "down")}
    for e in np.unique(idx[idx < w.N]):
        tt, kk = np.nonzero(idx == e)
        wg, wu, wd = make_expert_weights(w, int(e), "cpu")
        wg0, wu0, wd0 = wg.clone(), wu.clone(), wd.clone()
        wg0[:128] = 0
        wu0[:128] = 0
        wd0[:256] = 0
        rows["ref"][tt, kk] = oracle.swiglu_ffn(x64[tt], wg, wu, wd)
        rows["gate_up"][tt, kk] = oracle.swiglu_ffn(x64[tt], wg0, wu0, wd)
        rows["down"][tt, kk] = oracle.swiglu_ffn(x64[tt], wg, wu, wd0)
    y = {k: oracle.combine(x64, idx, gate, r, w.N) for k, r in rows.items()}
    bar = 1e-2 * np.abs(y["ref"]).max()
    moved = {k: float(np.abs(y[k] - y["ref"]).max()) for k in ("gate_up", "down")}
    # the same mistakes against the bar of the layer with the residual added
    r_all = torch.randn(w.T, w.d, generator=_gen(_seed(w, _TAG_RES), "cpu")).to(torch.bfloat16)
    res = oracle.moe_zc._f64(r_all[torch.from_numpy(toks)])
    bar_res = 1e-2 * np.abs(y["ref"] + res).max()
    print(f"bar {bar:.3e} (residual added: {bar_res:.3e}); y moved by "
          f"gate/up panel {moved['gate_up']:.3e}, down panel {moved['down']:.3e}")
    assert moved["gate_up"] > 2 * bar, (moved, bar)
    assert moved["down"] > 2 * bar, (moved, bar)
    # the residual-free bar is the one with teeth: the residual's bar is wider
    assert bar_res > 5 * bar
