"""The FP8 down projection's output bar, on the CPU (gpu_check.fp8_down_bar).

The GPU quantizes the hidden activation h from its fp32 value, the oracle
from its fp64 value, so a code next to a rounding midpoint can come out one
step apart; the bar allows rare tokens whose excess one flipped code per slot
explains, as it allows rare near-tie flips in routing.  On the oracle's own
path (layer of 592 tokens, d = 384, I = 256, 70 FFN experts, K = 1, bias
U(-0.1, 0.1)):
  * one code of h flipped by one step, where it moves the largest output
    most, must meet the bar although it moves that output past 1e-2;
  * an fp32 stand-in for the GPU path (float32 products of the same
    dequantized operands, float32 sigmoid) must meet it;
  * a flipped code in 3% of the tokens, one 32-wide block of h dropped, and
    W_down left unquantized must each fail it."""
import numpy as np
import torch

import oracle
from gpu_check import fp8_down_bar, fp8_down_code_flip_allowance
from workloads import Workload, make_inputs

MX = oracle.mx


def _layer():
    w = Workload("fp8down", T=592, d=384, I=256, N=70, Z=0, K=1, dtype="bf16", seed=207,
                 bias=("uniform", 0.1))
    inp = make_inputs(w, device="cpu", residual=False)
    x = inp["x"]
    l32 = oracle.router_logits(x, inp["w_router"]).astype(np.float32)
    b = inp["bias"].numpy()
    wg, wu, wd = inp["w_gate"], inp["w_up"], inp["w_down"]
    return w, x, l32, b, (lambda e: (wg[e], wu[e], wd[e]))


def _y(w, x, l32, b, get, h_fp32=False, flip_tokens=(), drop_block=False, raw_down=False):
    """The layer output with the FP8 down projection, from h in fp64 (the
    oracle's) or float32, optionally with one code of h flipped by one step in
    the rows of ``flip_tokens`` (where it moves the output most)."""
    x64 = x.double().numpy()
    x_dq = MX.mx_dequantize(*MX.mx_quantize(x64, axis=-1), axis=-1)
    rt = oracle.route(l32, b, w.K, w.N)
    idx, g = rt["idx"], rt["gate"]
    rows = np.zeros((w.T, w.K, w.d))
    flip = set(int(t) for t in flip_tokens)
    for e in np.unique(idx[idx < w.N]):
        tt, kk = np.nonzero(idx == e)
        wg, wu, wd = (MX.mx_dequantize(*MX.mx_quantize(t.double().numpy(), axis=-1), axis=-1)
                      for t in get(int(e)))
        if h_fp32:
            xa = x_dq[tt].astype(np.float32)
            a, u = xa @ wg.T.astype(np.float32), xa @ wu.T.astype(np.float32)
            h = (a * (np.float32(1) / (np.float32(1) + np.exp(-a))) * u).astype(np.float64)
        else:
            a, u = x_dq[tt] @ wg.T, x_dq[tt] @ wu.T
            h = a / (1.0 + np.exp(-a)) * u
        codes, scales = MX.mx_quantize(h, axis=-1)
        for r, t in enumerate(tt):
            if t in flip:
                h_dq = MX.mx_dequantize(codes[r:r + 1], scales[r:r + 1], axis=-1)[0]
                up = codes[r].astype(np.int64) + 1                   # one step up in magnitude
                ok = (codes[r] & 0x7F) < 0x7E
                h_up = MX.mx_dequantize(np.where(ok, up, codes[r]).astype(np.uint8)[None],
                                        scales[r:r + 1], axis=-1)[0]
                i = int(np.argmax(np.abs(h_up - h_dq) * np.abs(wd).max(axis=0)))
                codes[r, i] = np.uint8(up[i])
        h_dq = MX.mx_dequantize(codes, scales, axis=-1)
        if drop_block:
            h_dq[:, 64:96] = 0.0
        w_used = get(int(e))[2].double().numpy() if raw_down else wd
        rows[tt, kk] = h_dq @ w_used.T
    return oracle.moe_zc.combine(x64, idx, g, rows, w.N, None)


def _bar(w, x, l32, b, get, y):
    y_ref, _ = MX.forward_tokens_fp8(x, l32, b, get, w.N, w.K, None, down_fp8=True)
    tol = 1e-2 * np.abs(y_ref).max()
    diff = np.abs(y - y_ref)
    res = fp8_down_bar(diff, tol, lambda o: fp8_down_code_flip_allowance(
        x[torch.from_numpy(o)], l32[o], b, get, w.N, w.K))
    return res, diff.max() / tol


def test_one_flipped_code_meets_the_bar():
    w, x, l32, b, get = _layer()
    y0 = _y(w, x, l32, b, get)
    t = int(np.argmax(np.abs(y0).max(axis=1)))         # the largest output
    (ok, n_over, why), ratio = _bar(w, x, l32, b, get, _y(w, x, l32, b, get, flip_tokens=[t]))
    print("one flip: tokens over 1e-2:", n_over, "max err / bar:", ratio)
    assert ratio > 1.0, "the flip should move the output past the plain bar"
    assert ok, why


def test_fp32_path_meets_the_bar():
    w, x, l32, b, get = _layer()
    (ok, n_over, why), ratio = _bar(w, x, l32, b, get, _y(w, x, l32, b, get, h_fp32=True))
    print("fp32 h: tokens over 1e-2:", n_over, "max err / bar:", ratio)
    assert ok, why


def test_planted_mistakes_fail_the_bar():
    w, x, l32, b, get = _layer()
    many = np.random.default_rng(0).choice(w.T, int(0.03 * w.T), replace=False)
    for kw in (dict(flip_tokens=many), dict(drop_block=True), dict(raw_down=True)):
        (ok, n_over, why), ratio = _bar(w, x, l32, b, get, _y(w, x, l32, b, get, **kw))
        print(sorted(kw), "tokens over:", n_over, "max err / bar:", ratio, why)
        assert not ok, sorted(kw)
