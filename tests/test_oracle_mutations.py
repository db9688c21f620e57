"""Planted mistakes in the oracle (on the CPU) must each fail some pin.

Every mutation below is a plausible slip when writing the layer: a dropped
term, a wrong sign or index, a transposed operand, a bias in the wrong place.
The test replaces one oracle function with the mistaken version, runs every
pin, and requires at least one of them to fail.
"""
import numpy as np
import pytest

import pins
from oracle import moe_zc as om
from oracle import mx as omx

_orig = {name: getattr(om, name) for name in (
    "softmax_fp64", "selection_keys", "select_topk", "gates_of", "expert_loads",
    "ffn_offsets", "permutation", "silu", "swiglu_ffn", "combine", "pid_step",
    "route", "closed_loop", "budget_target")}


def m_bias_in_gate(mp):
    def sel(p64, bias):
        p32, key = _orig["selection_keys"](p64, bias)
        return key, key                       # gate becomes p + b
    mp.setattr(om, "selection_keys", sel)


def m_renormalised_gates(mp):
    def g(p32, idx):
        v = _orig["gates_of"](p32, idx).astype(np.float64)
        return (v / v.sum(axis=1, keepdims=True)).astype(np.float32)
    mp.setattr(om, "gates_of", g)


def m_softmax_ffn_only(mp):
    # probabilities normalised over the first half of the experts only
    def sm(l32):
        l = np.asarray(l32, np.float32).astype(np.float64)
        n = max(1, l.shape[1] // 2)
        e = np.exp(l - l.max(axis=1, keepdims=True))
        return e / e[:, :n].sum(axis=1, keepdims=True)
    mp.setattr(om, "softmax_fp64", sm)


def m_bias_on_logit(mp):
    def sm(l32):
        return _orig["softmax_fp64"](l32)
    def sel(p64, bias):
        # bias added before the softmax instead of to the probability
        lp = np.log(np.asarray(p64)) + np.asarray(bias, np.float64)[None, :]
        q = np.exp(lp - lp.max(axis=1, keepdims=True))
        q /= q.sum(axis=1, keepdims=True)
        return np.asarray(p64).astype(np.float32), q.astype(np.float32)
    mp.setattr(om, "selection_keys", sel)


def m_tie_to_higher_index(mp):
    def tk(key32, K):
        key32 = np.asarray(key32, np.float32)
        T, E = key32.shape
        order = np.lexsort((-np.broadcast_to(np.arange(E), (T, E)),
                            -key32.astype(np.float64)), axis=-1)
        return order[:, :K].astype(np.int64)
    mp.setattr(om, "select_topk", tk)


def m_smallest_keys(mp):
    def tk(key32, K):
        return _orig["select_topk"](-np.asarray(key32, np.float32), K)
    mp.setattr(om, "select_topk", tk)


def m_drop_identity_term(mp):
    def comb(x, idx, gates, rows, N, residual=None):
        g = np.where(np.asarray(idx) < N, gates, 0.0).astype(np.float32)
        return _orig["combine"](x, idx, g, rows, N, residual)
    mp.setattr(om, "combine", comb)


def m_drop_residual(mp):
    def comb(x, idx, gates, rows, N, residual=None):
        return _orig["combine"](x, idx, gates, rows, N, None)
    mp.setattr(om, "combine", comb)


def m_transposed_down(mp):
    def ffn(xr, wg, wu, wd):
        return _orig["swiglu_ffn"](xr, wg, wu, np.swapaxes(np.asarray(wd), -1, -2))
    mp.setattr(om, "swiglu_ffn", ffn)


def m_gate_up_swapped(mp):
    def ffn(xr, wg, wu, wd):
        return _orig["swiglu_ffn"](xr, wu, wg, wd)
    mp.setattr(om, "swiglu_ffn", ffn)


def m_silu_sign(mp):
    def s(v):
        v = np.asarray(v, np.float64)
        with np.errstate(over="ignore"):
            return v / (1.0 + np.exp(v))
    mp.setattr(om, "silu", s)


def m_sigmoid_not_silu(mp):
    def s(v):
        v = np.asarray(v, np.float64)
        with np.errstate(over="ignore"):
            return 1.0 / (1.0 + np.exp(-v))
    mp.setattr(om, "silu", s)


def m_loads_ffn_only(mp):
    def ld(idx, E):
        out = _orig["expert_loads"](idx, E)
        out[E // 2:] = 0
        return out
    mp.setattr(om, "expert_loads", ld)


def m_inclusive_offsets(mp):
    def off(loads, N):
        o = _orig["ffn_offsets"](loads, N)
        o[:N] = o[1:N + 1]
        return o
    mp.setattr(om, "ffn_offsets", off)


def m_unstable_permutation(mp):
    def perm(idx, N):
        p, pos = _orig["permutation"](idx, N)
        # tokens descending inside each expert instead of ascending
        idx = np.asarray(idx)
        counts = np.bincount(idx[idx < N].ravel(), minlength=N)[:N]
        starts = np.concatenate([[0], np.cumsum(counts)])
        p2 = p.copy()
        pos2 = pos.copy()
        for e in range(N):
            a, b = starts[e], starts[e + 1]
            p2[a:b] = p[a:b][::-1]
            for t, row in zip(p[a:b], range(a, b)):
                k = int(np.nonzero(idx[t] == e)[0][0])
                pos2[t, k] = a + b - 1 - row
        return p2, pos2
    mp.setattr(om, "permutation", perm)


def m_pid_sign(mp):
    def pid(loads, target, bias, e1, e2, kp, ki, kd):
        return _orig["pid_step"](target, loads, bias, e1, e2, kp, ki, kd)
    mp.setattr(om, "pid_step", pid)


def m_pid_p_on_error(mp):
    # proportional term on e instead of on its change (double counts P)
    def pid(loads, target, bias, e_prev, e_prev2, kp, ki, kd):
        b, e, e1 = _orig["pid_step"](loads, target, bias, e_prev, e_prev2, kp, ki, kd)
        return b + kp * np.asarray(e_prev, np.float64), e, e1
    mp.setattr(om, "pid_step", pid)


def m_pid_no_derivative(mp):
    def pid(loads, target, bias, e_prev, e_prev2, kp, ki, kd):
        return _orig["pid_step"](loads, target, bias, e_prev, e_prev2, kp, ki, 0.0)
    mp.setattr(om, "pid_step", pid)


def m_loop_without_feedback(mp):
    # every batch routed with the starting bias: the controller never acts
    def route(l32, bias, K, N):
        return _orig["route"](l32, np.zeros_like(np.asarray(bias)), K, N)
    mp.setattr(om, "route", route)


def m_loop_history_reset(mp):
    # the error histories are dropped between batches
    def pid(loads, target, bias, e_prev, e_prev2, kp, ki, kd):
        return _orig["pid_step"](loads, target, bias, np.zeros_like(e_prev),
                                 np.zeros_like(e_prev2), kp, ki, kd)
    mp.setattr(om, "pid_step", pid)


def m_budget_swapped(mp):
    # FFN and identity shares exchanged
    def bt(T, K, N, Z, f):
        return _orig["budget_target"](T, K, N, Z, K - f)
    mp.setattr(om, "budget_target", bt)


_mx = {name: getattr(omx, name) for name in (
    "mx_scale_exponent", "e4m3_encode", "mx_quantize", "mx_dequantize", "forward_fp8_gateup")}


def m_mx_floor_scale(mp):
    # scale from floor(log2 amax) - 8 alone: the block maximum can overflow 448
    def sc(amax):
        a = np.asarray(amax, np.float64)
        m, ex = np.frexp(np.where(a > 0, a, 1.0))
        return np.clip(np.where(a > 0, ex - 1 - 8, -127), -127, 127).astype(np.int64)
    mp.setattr(omx, "mx_scale_exponent", sc)


def m_mx_truncate(mp):
    # rounding toward zero instead of to nearest even
    def enc(y):
        y = np.asarray(y, np.float64)
        a = np.abs(y)
        grid = omx.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
        code = np.searchsorted(grid, a, side="right") - 1
        return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)
    mp.setattr(omx, "e4m3_encode", enc)


def m_mx_scale_bias_128(mp):
    def q(v, axis=-1):
        c, sc = _mx["mx_quantize"](v, axis)
        return c, (sc.astype(np.int64) + 1).astype(np.uint8)
    def dq(c, sc, axis=-1):
        return _mx["mx_dequantize"](c, (np.asarray(sc, np.int64) - 1).astype(np.uint8), axis)
    mp.setattr(omx, "mx_quantize", q)
    mp.setattr(omx, "mx_dequantize", dq)


def m_mx_block16(mp):
    mp.setattr(omx, "BLOCK", 16)


def m_fp8_identity_quantized(mp):
    # the identity experts fed the FP8 image of x
    def fwd(x, w_router, bias, w_gate, w_up, w_down, N, Z, K, residual=None, logits32=None,
            down_fp8=False):
        xq, xs = _mx["mx_quantize"](np.asarray(x, np.float64))
        x_dq = _mx["mx_dequantize"](xq, xs)
        rt = _mx["forward_fp8_gateup"](x_dq, w_router, bias, w_gate, w_up, w_down, N, Z, K,
                                       residual, om.router_logits(x, w_router).astype(np.float32),
                                       down_fp8=down_fp8)
        return rt
    mp.setattr(omx, "forward_fp8_gateup", fwd)


from oracle import backward as obw
_bw = obw.backward


def m_fp8_down_h_unquantized(mp):
    # the hidden activation enters the FP8 down projection unquantized
    def down(h, w_down):
        wd_dq = _mx["mx_dequantize"](*_mx["mx_quantize"](w_down, axis=-1), axis=-1)
        return np.asarray(h, np.float64) @ wd_dq.T
    mp.setattr(omx, "down_projection_fp8", down)


def m_fp8_down_weights_along_d(mp):
    # W_down quantized in blocks along its output axis d instead of along I
    def down(h, w_down):
        h_dq = _mx["mx_dequantize"](*_mx["mx_quantize"](h, axis=-1), axis=-1)
        wd_dq = _mx["mx_dequantize"](*_mx["mx_quantize"](w_down, axis=0), axis=0)
        return h_dq @ wd_dq.T
    mp.setattr(omx, "down_projection_fp8", down)


def _bw_variant(**flags):
    """The oracle backward with one planted slip (re-implemented here)."""
    def bw(x, w_router, bias, w_gate, w_up, w_down, N, Z, K, dy, logits32=None):
        out = _bw(x, w_router, bias, w_gate, w_up, w_down, N, Z, K, dy, logits32)
        wr = np.asarray(w_router, np.float64)
        if flags.get("drop_router"):
            out["dx"] = out["dx"] - out["dlogits"] @ wr
        return out
    return bw


def m_bwd_no_router_term(mp):
    mp.setattr(obw, "backward", _bw_variant(drop_router=True))


def m_bwd_silu_derivative_sigmoid(mp):
    # d silu / da taken as sigmoid(a) alone
    src = __import__("inspect").getsource(_bw)
    src = src.replace("s * (1.0 + a * (1.0 - s))", "s")
    ns = dict(obw.__dict__)
    exec(compile(src, "mutant", "exec"), ns)
    mp.setattr(obw, "backward", ns["backward"])


def m_bwd_gate_not_applied(mp):
    src = __import__("inspect").getsource(_bw).replace("dE = g[:, None] * dy64[tt]", "dE = dy64[tt]")
    ns = dict(obw.__dict__)
    exec(compile(src, "mutant", "exec"), ns)
    mp.setattr(obw, "backward", ns["backward"])


def m_bwd_identity_dx_dropped(mp):
    src = __import__("inspect").getsource(_bw).replace(
        "np.add.at(dx, tz, gate[tz, kz][:, None] * dy64[tz])", "pass")
    ns = dict(obw.__dict__)
    exec(compile(src, "mutant", "exec"), ns)
    mp.setattr(obw, "backward", ns["backward"])


def m_bwd_softmax_jacobian_wrong(mp):
    # dl = p * dp, without the centring term
    src = __import__("inspect").getsource(_bw).replace(
        "dl = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "dl = p * dp")
    ns = dict(obw.__dict__)
    exec(compile(src, "mutant", "exec"), ns)
    mp.setattr(obw, "backward", ns["backward"])


MUTATIONS = [
    m_bias_in_gate, m_renormalised_gates, m_softmax_ffn_only, m_bias_on_logit,
    m_tie_to_higher_index, m_smallest_keys, m_drop_identity_term,
    m_drop_residual, m_transposed_down, m_gate_up_swapped, m_silu_sign,
    m_sigmoid_not_silu, m_loads_ffn_only, m_inclusive_offsets,
    m_unstable_permutation, m_pid_sign, m_pid_p_on_error, m_pid_no_derivative,
    m_loop_without_feedback, m_loop_history_reset, m_budget_swapped,
    m_mx_floor_scale, m_mx_truncate, m_mx_scale_bias_128, m_mx_block16,
    m_fp8_identity_quantized, m_fp8_down_h_unquantized, m_fp8_down_weights_along_d,
    m_bwd_no_router_term, m_bwd_silu_derivative_sigmoid,
    m_bwd_gate_not_applied, m_bwd_identity_dx_dropped, m_bwd_softmax_jacobian_wrong,
]

# the statistical check is slow and not needed to catch any of these
_FAST = [c for c in pins.ALL_CHECKS if c is not pins.check_ffn_count_hypergeometric]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=lambda m: m.__name__)
def test_mutation_is_caught(mutation, monkeypatch):
    mutation(monkeypatch)
    caught = []
    for check in _FAST:
        try:
            check()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(check.__name__)
    assert caught, f"{mutation.__name__} passed every pin"
