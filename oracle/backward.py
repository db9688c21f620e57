"""fp64 oracle of the layer's backward pass (gradients of a scalar loss).

TEST INFRASTRUCTURE: imported only by the tests, the smoke check and the
benchmark's CPU-baseline leg.

The pages list deterministic computation among the training techniques
(『衝上熱搜！美團大模型，靠「快」火了』, section 模型擴展策略與多階段訓練, its
fourth point: fully reproducible results and detection of silent data
corruption); the backward of the MoE layer is the training side of the
forward in moe_zc.py.
For the layer of that module (routing fixed by the forward's top-K choice,
which is piecewise constant and passes no gradient; the bias steers routing
only and receives none), with upstream gradient dy = dL/dy:

  slot (t, k) on FFN expert e, a = W_gate x, u = W_up x, s = sigmoid(a),
  h = a s u, o = W_down h:
    dE   = g dy_t                      gradient into the expert's output
    dg   = <dy_t, o>                   gradient into the gate
    dh   = W_down^T dE
    da   = dh u s (1 + a (1 - s))      d silu(a) / da = s (1 + a (1 - s))
    du   = dh a s
    dx_t += W_gate^T da + W_up^T du
    dW_down += dE h^T,  dW_gate += da x_t^T,  dW_up += du x_t^T
  slot (t, k) on an identity expert:
    dg   = <dy_t, x_t>,  dx_t += g dy_t
  router (g = softmax(l)[chosen], l = W_r x):
    dp_t,i = dg of the slot that chose i (0 for experts not chosen)
    dl_t   = p_t * (dp_t - <p_t, dp_t>)
    dx_t  += W_r^T dl_t,  dW_r += dl_t x_t^T
  the residual passes dy unchanged (dr = dy) and is not returned.

Gates are taken as the probabilities themselves (their fp32 rounding passes
no gradient).  Pins (tests/pins.py): central finite differences of
sum(y * dy) through moe_zc.forward on a small layer; a single forced FFN
expert equals the gradient of a dense SwiGLU FFN from torch's autograd
(fp64, CPU); identity experts alone give dx = (sum g) dy plus the router term.
"""
from __future__ import annotations

import numpy as np

from . import moe_zc as _layer


def backward(x, w_router, bias, w_gate, w_up, w_down, N: int, Z: int, K: int, dy,
             logits32=None, experts=None, want_dx=True):
    """Gradients of sum(y * dy) for the layer of moe_zc.forward.  Routing uses
    ``logits32`` when given (as the forward does), else the fp64 logits rounded
    once to fp32.  Returns dict dx [T, d], dw_router [E, d], dw_gate,
    dw_up [N, I, d], dw_down [N, d, I] (fp64), and the routing used.

    Subsets for large layers (the arithmetic is the same):
    - ``experts``: a list of FFN experts; only their weight gradients are
      formed, returned as dicts {e: array} under the same keys.  Expert e's
      gradients depend only on the tokens routed to e, so passing exactly
      those tokens gives them in full.
    - ``want_dx=False`` skips dx, dlogits and dw_router.  dx of a token
      depends only on that token, so passing a sample of tokens gives their
      rows of dx in full."""
    x64 = _layer._f64(x)
    wr = _layer._f64(w_router)
    dy64 = _layer._f64(dy)
    T, d = x64.shape
    E = N + Z
    if logits32 is None:
        logits32 = _layer.router_logits(x64, wr).astype(np.float32)
    rt = _layer.route(logits32, bias, K, N)
    idx, p = rt["idx"], rt["p64"]
    gate = rt["gate"].astype(np.float64)
    I = w_gate.shape[1] if N > 0 else 0
    dx = np.zeros((T, d))
    if experts is None:
        dwg = np.zeros((N, I, d))
        dwu = np.zeros((N, I, d))
        dwd = np.zeros((N, d, I))
        loop = np.unique(idx[idx < N])
    else:
        dwg = {int(e): np.zeros((I, d)) for e in experts}
        dwu = {int(e): np.zeros((I, d)) for e in experts}
        dwd = {int(e): np.zeros((d, I)) for e in experts}
        loop = np.unique(idx[idx < N]) if want_dx else np.asarray(sorted(dwg), dtype=np.int64)
    dp = np.zeros((T, E))
    for e in loop:
        tt, kk = np.nonzero(idx == e)          # a token chooses an expert at most once
        if len(tt) == 0:
            continue
        xe = x64[tt]
        wg, wu, wd = (_layer._f64(w[int(e)]) for w in (w_gate, w_up, w_down))
        a = xe @ wg.T
        u = xe @ wu.T
        s = 1.0 / (1.0 + np.exp(-a))
        h = a * s * u
        o = h @ wd.T
        g = gate[tt, kk]
        dE = g[:, None] * dy64[tt]
        dp[tt, e] = (dy64[tt] * o).sum(axis=1)
        dh = dE @ wd
        da = dh * u * s * (1.0 + a * (1.0 - s))
        du = dh * a * s
        if want_dx:
            dx[tt] += da @ wg + du @ wu
        if experts is None or int(e) in dwg:
            dwd[int(e)] += dE.T @ h
            dwg[int(e)] += da.T @ xe
            dwu[int(e)] += du.T @ xe
    if not want_dx:
        return {"dw_gate": dwg, "dw_up": dwu, "dw_down": dwd, "route": rt}
    tz, kz = np.nonzero(idx >= N)
    dp[tz, idx[tz, kz]] = (dy64[tz] * x64[tz]).sum(axis=1)
    np.add.at(dx, tz, gate[tz, kz][:, None] * dy64[tz])
    dl = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dx += dl @ wr
    dwr = dl.T @ x64
    return {"dx": dx, "dw_router": dwr, "dw_gate": dwg, "dw_up": dwu, "dw_down": dwd,
            "dlogits": dl, "route": rt}
