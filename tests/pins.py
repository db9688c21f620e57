"""Checks that pin the fp64 oracle to facts other than itself.

Each check raises AssertionError on failure.  They are collected as tests in
test_oracle_pins.py, and test_oracle_mutations.py plants plausible mistakes in
the oracle (on the CPU) to show that at least one check catches each.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from oracle import moe_zc as om
from oracle import mx as omx
from oracle import backward as obw
from oracle import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def random_layer(T, d, I, N, Z, seed=0, bias_scale=0.05, residual=True):
    """Small random fp64 layer (test-local; not a product workload)."""
    r = _rng(seed)
    E = N + Z
    x = r.standard_normal((T, d))
    wr = r.standard_normal((E, d)) / math.sqrt(d)
    b = r.uniform(-bias_scale, bias_scale, E).astype(np.float32)
    wg = r.standard_normal((N, I, d)) / math.sqrt(d)
    wu = r.standard_normal((N, I, d)) / math.sqrt(d)
    wd = r.standard_normal((N, d, I)) / math.sqrt(I)
    res = r.standard_normal((T, d)) if residual else None
    return dict(x=x, w_router=wr, bias=b, w_gate=wg, w_up=wu, w_down=wd,
                residual=res)


# ---------------------------------------------------------------- golden --
def check_hand_example():
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        G = json.load(f)
    N, Z = G["shapes"]["N"], G["shapes"]["Z"]
    x = np.array(G["x"])
    wg, wu, wd = (np.array(G[k]) for k in ("w_gate", "w_up", "w_down"))
    for case in G["cases"]:
        # the router weights reproduce the case's logits for x = [1, 2]
        wr = np.zeros((N + Z, 2))
        wr[:, 0] = case["logits"]
        l64 = om.router_logits(x, wr)
        assert np.allclose(l64[0], case["logits"], rtol=0, atol=1e-15), case["name"]
        out = om.forward(x, wr, np.array(case["bias"], np.float32), wg, wu, wd,
                         N, Z, case["K"])
        assert out["idx"][0].tolist() == case["idx"], (case["name"], out["idx"])
        assert np.allclose(out["gate"][0], case["gate"], rtol=0, atol=1e-7), case["name"]
        assert np.allclose(out["y"][0], case["y"], rtol=0, atol=case["tol"]), \
            (case["name"], out["y"][0], case["y"])


def check_pid_golden():
    with open(os.path.join(GOLDEN, "pid_example.json")) as f:
        G = json.load(f)
    g = G["gains"]
    tgt = np.array(G["target"])
    b = np.array(G["bias0"])
    e1 = np.zeros_like(b)
    e2 = np.zeros_like(b)
    for st in G["steps"]:
        b, e1, e2 = om.pid_step(st["loads"], tgt, b, e1, e2, g["kp"], g["ki"], g["kd"])
        assert np.array_equal(e1, np.array(st["e"])), (e1, st["e"])
        assert np.array_equal(b, np.array(st["bias"])), (b, st["bias"])


# ------------------------------------------------------------ brute force --
def check_bruteforce_tiny(T=16, d=24, I=20, N=5, Z=3, K=3, seed=1):
    L = random_layer(T, d, I, N, Z, seed=seed, bias_scale=0.1)
    ref = bf.forward(L["x"], L["w_router"], L["bias"], L["w_gate"], L["w_up"],
                     L["w_down"], N, Z, K, L["residual"])
    out = om.forward(L["x"], L["w_router"], L["bias"], L["w_gate"], L["w_up"],
                     L["w_down"], N, Z, K, L["residual"], logits32=ref["logits32"])
    l_bf = np.array(bf.logits(L["x"], L["w_router"]))
    assert np.allclose(out["logits64"], l_bf, rtol=0, atol=1e-13)
    assert np.array_equal(out["idx"], ref["idx"]), "top-K differs from subset enumeration"
    assert np.array_equal(out["gate"], ref["gate"])
    assert np.array_equal(out["loads"], ref["loads"])
    assert np.array_equal(out["perm"], ref["perm"])
    assert np.array_equal(out["pos"], ref["pos"])
    err = np.abs(out["y"] - ref["y"]).max()
    assert err <= 1e-12 * max(1.0, np.abs(ref["y"]).max()), err


def check_topk_ties_enumeration(seed=3, T=200, E=8, K=3):
    r = _rng(seed)
    keys = r.choice(np.array([0.1, 0.2, 0.3, 0.2], np.float32), size=(T, E))
    idx = om.select_topk(keys, K)
    for t in range(T):
        assert idx[t].tolist() == bf.topk_by_enumeration(keys[t].tolist(), K), t


def check_softmax_bruteforce(seed=4, T=20, E=12):
    l32 = (_rng(seed).standard_normal((T, E)) * 3).astype(np.float32)
    p = om.softmax_fp64(l32)
    for t in range(T):
        ref = bf.softmax_row(l32[t])
        assert np.allclose(p[t], ref, rtol=1e-14, atol=0)
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-14)


# ---------------------------------------------------- special cases -------
def _dense_swiglu_torch(x, wg, wu, wd):
    x, wg, wu, wd = (torch.as_tensor(np.asarray(a), dtype=torch.float64)
                     for a in (x, wg, wu, wd))
    return ((F.silu(x @ wg.T) * (x @ wu.T)) @ wd.T).numpy()


def check_single_forced_ffn(T=12, d=16, seed=5):
    # N=1, Z=0, K=1: the only expert has p = 1, so the layer is a dense SwiGLU
    # FFN plus the residual.  d == I so that a transposed operand cannot hide.
    L = random_layer(T, d, d, 1, 0, seed=seed)
    out = om.forward(L["x"], L["w_router"], L["bias"], L["w_gate"], L["w_up"],
                     L["w_down"], 1, 0, 1, L["residual"])
    ref = _dense_swiglu_torch(L["x"], L["w_gate"][0], L["w_up"][0], L["w_down"][0]) + L["residual"]
    assert np.allclose(out["gate"], 1.0, rtol=0, atol=0)
    assert np.allclose(out["y"], ref, rtol=1e-12, atol=1e-12)
    # A +10 bias forces expert e into slot 0 with gate p_e (bias is not a gate).
    N, Z = 4, 2
    L = random_layer(T, d, d, N, Z, seed=seed + 1, residual=False)
    e = 2
    b = np.zeros(N + Z, np.float32)
    b[e] = 10.0
    out = om.forward(L["x"], L["w_router"], b, L["w_gate"], L["w_up"], L["w_down"], N, Z, 1)
    p = torch.softmax(torch.as_tensor(out["logits64"]).float().double(), dim=1).numpy()
    assert (out["idx"][:, 0] == e).all()
    assert np.allclose(out["gate"][:, 0], p[:, e], rtol=1e-6, atol=0)
    ref = p[:, e:e + 1] * _dense_swiglu_torch(L["x"], L["w_gate"][e], L["w_up"][e], L["w_down"][e])
    assert np.allclose(out["y"], ref, rtol=1e-6, atol=1e-9)


def check_all_identity(T=32, d=16, I=8, N=6, Z=5, K=3, seed=6):
    # every FFN expert biased by -10: all K slots go to identity experts and
    # y = (sum of their gates) x + r, gates = the K largest identity-expert
    # probabilities of a library softmax.
    L = random_layer(T, d, I, N, Z, seed=seed)
    b = np.zeros(N + Z, np.float32)
    b[:N] = -10.0
    out = om.forward(L["x"], L["w_router"], b, L["w_gate"], L["w_up"], L["w_down"],
                     N, Z, K, L["residual"])
    p = torch.softmax(torch.as_tensor(out["logits64"].astype(np.float32)).double(), dim=1)
    top = torch.topk(p[:, N:], K, dim=1).values.sum(dim=1).numpy()
    assert (out["idx"] >= N).all()
    ref = top[:, None] * L["x"] + L["residual"]
    assert np.allclose(out["y"], ref, rtol=1e-6, atol=1e-7)
    assert out["n_rows"] == 0
    # N = 0 (identity experts only) gives the same closed form
    out0 = om.forward(L["x"], L["w_router"][N:], np.zeros(Z, np.float32),
                      L["w_gate"][:0], L["w_up"][:0], L["w_down"][:0], 0, Z, K, None)
    p0 = torch.softmax(torch.as_tensor(out0["logits64"].astype(np.float32)).double(), dim=1)
    ref0 = torch.topk(p0, K, dim=1).values.sum(dim=1).numpy()[:, None] * L["x"]
    assert np.allclose(out0["y"], ref0, rtol=1e-6, atol=1e-7)


def check_k_equals_e(T=24, d=16, I=8, N=5, Z=3, seed=7):
    # K = E: every expert is chosen, so the output no longer depends on b:
    # y = sum_{i<N} p_i FFN_i(x) + (sum_{i>=N} p_i) x + r
    L = random_layer(T, d, I, N, Z, seed=seed)
    E = N + Z
    outs = []
    for bseed in (0, 1):
        b = _rng(100 + bseed).uniform(-0.3, 0.3, E).astype(np.float32)
        outs.append(om.forward(L["x"], L["w_router"], b, L["w_gate"], L["w_up"],
                               L["w_down"], N, Z, E, L["residual"]))
    p = torch.softmax(torch.as_tensor(outs[0]["logits64"].astype(np.float32)).double(), dim=1).numpy()
    ref = L["residual"] + p[:, N:].sum(axis=1, keepdims=True) * L["x"]
    for i in range(N):
        ref = ref + p[:, i:i + 1] * _dense_swiglu_torch(L["x"], L["w_gate"][i], L["w_up"][i], L["w_down"][i])
    for o in outs:
        assert np.allclose(o["y"], ref, rtol=1e-6, atol=1e-6)
    assert np.allclose(outs[0]["y"], outs[1]["y"], rtol=0, atol=1e-12)


def check_z_zero_textbook_moe(T=40, d=16, I=12, N=7, K=2, seed=8):
    # Z = 0: a plain softmax top-K MoE whose gates are not renormalised,
    # written with library routines (torch.softmax, torch.topk, F.silu).
    L = random_layer(T, d, I, N, 0, seed=seed, bias_scale=0.0)
    out = om.forward(L["x"], L["w_router"], np.zeros(N, np.float32), L["w_gate"],
                     L["w_up"], L["w_down"], N, 0, K, None)
    p = torch.softmax(torch.as_tensor(out["logits64"].astype(np.float32)).double(), dim=1)
    val, ind = torch.topk(p, K, dim=1)
    ref = np.zeros_like(L["x"])
    for t in range(T):
        for k in range(K):
            e = int(ind[t, k])
            ref[t] += float(val[t, k]) * _dense_swiglu_torch(
                L["x"][t:t + 1], L["w_gate"][e], L["w_up"][e], L["w_down"][e])[0]
    assert np.array_equal(np.sort(out["idx"], axis=1), np.sort(ind.numpy(), axis=1))
    assert np.allclose(out["y"], ref, rtol=1e-6, atol=1e-7)


# -------------------------------------------------------------- invariants --
def check_permutation_invariants(T=300, E=20, N=13, K=4, seed=9):
    l32 = _rng(seed).standard_normal((T, E)).astype(np.float32)
    b = _rng(seed + 1).uniform(-0.05, 0.05, E).astype(np.float32)
    rt = om.route(l32, b, K, N)
    idx, perm, pos, loads, off = rt["idx"], rt["perm"], rt["pos"], rt["loads"], rt["offsets"]
    assert loads.sum() == T * K
    assert (np.diff(off) >= 0).all() and off[0] == 0 and off[N] == rt["n_rows"]
    assert np.array_equal(np.diff(off), loads[:N])
    # grouped order = stable sort of the FFN slots by expert (library sort)
    tt, kk = np.nonzero(idx < N)                  # slots in token-major order
    order = np.argsort(idx[tt, kk], kind="stable")
    assert np.array_equal(perm, tt[order])
    assert np.array_equal(pos[tt[order], kk[order]], np.arange(len(order)))
    assert (pos[idx >= N] == -1).all()
    # perm is a bijection onto the FFN slots; round trip is the identity
    assert len(perm) == int((idx < N).sum())
    rows = np.arange(T, dtype=np.float64)[perm][:, None] * np.ones((1, 3))
    back = om.unpermute(rows, pos, idx, N)
    ffn = idx < N
    assert np.array_equal(back[ffn][:, 0], np.nonzero(ffn)[0].astype(np.float64))
    # each expert appears at most once per token
    for t in range(T):
        assert len(set(idx[t].tolist())) == K


def check_token_independence(T=48, d=16, I=8, N=6, Z=3, K=3, seed=10):
    L = random_layer(T, d, I, N, Z, seed=seed)
    full = om.forward(L["x"], L["w_router"], L["bias"], L["w_gate"], L["w_up"],
                      L["w_down"], N, Z, K, L["residual"])
    sub = np.array([3, 17, 5, 40])
    part = om.forward(L["x"][sub], L["w_router"], L["bias"], L["w_gate"], L["w_up"],
                      L["w_down"], N, Z, K, L["residual"][sub])
    assert np.array_equal(part["idx"], full["idx"][sub])
    assert np.allclose(part["y"], full["y"][sub], rtol=0, atol=1e-12)
    assert np.allclose(full["p64"].sum(axis=1), 1.0, atol=1e-14)
    assert (full["gate"].astype(np.float64).sum(axis=1) <= 1.0 + 1e-6).all()


def check_ffn_count_hypergeometric(T=20000, N=512, Z=256, K=12, seed=11):
    """With zero bias and iid logits the chosen set is a uniform K-subset, so
    the FFN count per token is Hypergeometric(E, N, K)."""
    from scipy.stats import hypergeom
    E = N + Z
    l32 = _rng(seed).standard_normal((T, E)).astype(np.float32)
    rt = om.route(l32, np.zeros(E, np.float32), K, N)
    c = om.ffn_count_per_token(rt["idx"], N)
    mean = K * N / E
    var = K * (N / E) * (Z / E) * (E - K) / (E - 1)
    assert abs(c.mean() - mean) < 4 * math.sqrt(var / T), (c.mean(), mean)
    assert abs(c.var() - var) < 0.05 * var, (c.var(), var)
    pmf = hypergeom(E, N, K).pmf(np.arange(K + 1))
    hist = np.bincount(c, minlength=K + 1) / T
    assert np.abs(hist - pmf).max() < 0.01, (hist, pmf)


# ----------------------------------------------------------------- PID -----
def check_pid_properties(E=64, seed=12):
    r = _rng(seed)
    tgt = np.full(E, 12.0)
    b0 = r.uniform(-0.01, 0.01, E)
    # zero error: no change
    b, e1, e2 = om.pid_step(tgt.copy(), tgt, b0, np.zeros(E), np.zeros(E), 0.7, 0.3, 0.2)
    assert np.array_equal(b, b0) and not e1.any()
    # equal totals: the updates sum to zero; the overloaded expert falls
    loads = tgt.copy()
    loads[0] += 5
    loads[1] -= 3
    loads[2] -= 2
    assert loads.sum() == tgt.sum()
    b, e1, _ = om.pid_step(loads, tgt, b0, np.zeros(E), np.zeros(E), 0.7, 0.3, 0.2)
    db = b - b0
    assert abs(db.sum()) < 1e-12
    assert np.array_equal(np.sign(db), np.sign(tgt - loads))
    # velocity form accumulates to the positional form
    kp, ki, kd = 0.4, 0.3, 0.2
    b, e1, e2 = b0.copy(), np.zeros(E), np.zeros(E)
    es = []
    for s in range(5):
        ld = r.integers(0, 25, E).astype(np.float64)
        b, e1, e2 = om.pid_step(ld, tgt, b, e1, e2, kp, ki, kd)
        es.append(e1)
    pos_form = b0 + kp * es[-1] + ki * np.sum(es, axis=0) + kd * (es[-1] - es[-2])
    assert np.allclose(b, pos_form, rtol=0, atol=1e-14)


# ------------------------------------------------------ closed-loop PID -----
def check_budget_target():
    T, K, N, Z = 96, 12, 512, 256
    for f in (0.0, 3.5, 8.0, 12.0):
        if (f == 0.0 and N == 0) or (f == 12.0 and Z == 0):
            continue
        t = om.budget_target(T, K, N, Z, f)
        assert t.shape == (N + Z,)
        assert abs(t[:N].sum() - T * f) < 1e-9 and abs(t[N:].sum() - T * (K - f)) < 1e-9
        assert np.ptp(t[:N]) == 0 and np.ptp(t[N:]) == 0
    for bad in (-0.5, 12.5):
        try:
            om.budget_target(T, K, N, Z, bad)
        except ValueError:
            continue
        raise AssertionError("budget outside [0, K] accepted")


def check_closed_loop_fixed_point(S=5):
    # E = 4 (2 FFN, 2 identity), K = 2: token t strongly prefers experts t and
    # t+1 (mod 4), so every expert gets 2 slots; the budget of one FFN expert
    # per token asks for exactly that, so the bias must never move
    T, N, Z, K = 4, 2, 2, 2
    l32 = np.zeros((T, N + Z), np.float32)
    for t in range(T):
        l32[t, t % 4], l32[t, (t + 1) % 4] = 5.0, 4.0
    b0 = np.array([0.01, -0.02, 0.005, -0.01], np.float32)
    tgt = om.budget_target(T, K, N, Z, 1.0)
    out = om.closed_loop([l32] * S, b0, tgt, K, N, 0.7, 0.3, 0.2)
    assert np.array_equal(out["bias"], np.broadcast_to(b0, (S + 1, 4)))
    assert (out["loads"] == 2).all() and np.allclose(out["ffn_per_token"], 1.0)


def _skewed_logits(r, T, N, Z, s=1.1, c=0.0):
    l = r.standard_normal((T, N + Z)) * 0.5
    ranks = r.permutation(N) + 1
    l[:, :N] += -s * np.log(ranks) + c
    return l.astype(np.float32)


def check_closed_loop_conservation_and_positional_form(S=8, seed=13):
    r = _rng(seed)
    T, N, Z, K = 600, 16, 8, 4
    kp, ki, kd = 0.4, 0.5, 0.2
    batches = [_skewed_logits(r, T, N, Z, c=0.8) for _ in range(S)]
    b0 = r.uniform(-0.01, 0.01, N + Z).astype(np.float32)
    tgt = om.budget_target(T, K, N, Z, 2.5)
    out = om.closed_loop(batches, b0, tgt, K, N, kp, ki, kd)
    # the target and the loads both sum to T K: the bias sum is conserved
    # (to fp32 rounding of the stored state)
    sums = out["bias"].astype(np.float64).sum(axis=1)
    assert np.abs(sums - sums[0]).max() < 1e-5, sums
    # the velocity-form steps add up to the positional PID over the recorded
    # loads: b_S = b_0 + kp e_S + ki sum(e) + kd (e_S - e_{S-1})
    e = (tgt[None, :] - out["loads"]) / tgt.sum()
    pos = b0 + kp * e[-1] + ki * e.sum(axis=0) + kd * (e[-1] - e[-2])
    assert np.abs(out["bias"][-1] - pos).max() < 1e-5
    # the skew comes down: the busiest FFN expert carries less at the end
    ld = out["loads"][:, :N].astype(np.float64)
    assert ld[-1].max() / ld[-1].mean() < ld[0].max() / ld[0].mean()


def check_closed_loop_integral_settles(seed=14, S=60):
    # one FFN and one identity expert, K = 1: expert 0 wins token t when
    # p0 + b0 > p1 + b1, so its load falls monotonically as b1 - b0 grows; an
    # integral controller on such a plant settles where the load meets the
    # target (to the granularity of one token)
    r = _rng(seed)
    T = 400
    a = r.normal(1.0, 1.0, T)
    l32 = np.stack([a, np.zeros(T)], axis=1).astype(np.float32)
    tgt = om.budget_target(T, 1, 1, 1, 0.25)          # 100 FFN slots, 300 identity
    out = om.closed_loop([l32] * S, np.zeros(2, np.float32), tgt, 1, 1, 0.0, 0.5, 0.0)
    assert out["loads"][0, 0] > 250                     # the skew it starts from
    assert np.abs(out["loads"][-10:, 0] - 100).max() <= 3, out["loads"][-10:, 0]
    assert abs(out["ffn_per_token"][-1] - 0.25) <= 3 / T


# ------------------------------------------------------- block FP8 (MX) -----
def check_e4m3_codes():
    c = np.arange(256, dtype=np.uint8)
    v = omx.e4m3_decode(c)
    nan = np.isnan(v)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    # closed-form landmarks of the format
    assert v[0x7E] == 448.0 and v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6
    assert v[0x38] == 1.0 and v[0x3C] == 1.5 and v[0xB8] == -1.0
    fin = ~nan
    assert np.array_equal(omx.e4m3_encode(v[fin]), c[fin])        # incl. -0 -> 0x80
    pos = v[:0x7F]
    assert (np.diff(pos) > 0).all()                               # codes increase with value


def check_e4m3_rounding_bruteforce(seed=15, n=4000):
    r = _rng(seed)
    grid = omx.e4m3_decode(np.arange(0x7F, dtype=np.uint8))      # 0 .. 448, increasing
    mids = (grid[1:] + grid[:-1]) / 2.0
    ys = np.concatenate([r.uniform(-448, 448, n), mids, -mids, grid,
                         r.uniform(0, 2.0 ** -5, n // 4), [0.0, -0.0, 448.0, -448.0]])
    got = omx.e4m3_encode(ys)
    for y, g in zip(ys, got):
        a = abs(y)
        d = np.abs(grid - a)
        best = np.flatnonzero(d == d.min())
        code = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        want = code | (0x80 if np.signbit(y) else 0)
        assert g == want, (y, g, want)
    try:
        omx.e4m3_encode(np.array([448.5]))
    except ValueError:
        return
    raise AssertionError("out-of-range value accepted")


def check_mx_scales_minimal(seed=16):
    r = _rng(seed)
    v = r.standard_normal((64, 256)) * np.ldexp(1.0, r.integers(-30, 30, (64, 1)))
    v[3, 32:64] = 0.0                                             # an all-zero block
    v[5, 0:32] = 0.0
    v[5, 7] = 448.0 * 2.0 ** 3                                    # amax exactly on the range
    codes, scales = omx.mx_quantize(v, axis=1)
    assert codes.shape == v.shape and scales.shape == (64, 8)
    s = scales.astype(np.int64) - 127
    amax = np.abs(v.reshape(64, 8, 32)).max(axis=2)
    live = amax > 0
    assert (amax[live] <= 448.0 * np.ldexp(1.0, s[live])).all()
    assert (amax[live] > 448.0 * np.ldexp(1.0, s[live] - 1)).all()   # the smallest such scale
    assert s[3, 1] == -127 and not codes[3, 32:64].any()
    assert s[5, 0] == 3 and codes[5, 7] == 0x7E
    # error within half a grid step at the value's magnitude
    dq = omx.mx_dequantize(codes, scales, axis=1)
    y = np.abs(v) / np.repeat(np.ldexp(1.0, s), 32, axis=1)
    E = np.floor(np.log2(np.maximum(y, 2.0 ** -6)))
    half = np.ldexp(1.0, (E - 4).astype(int)) * np.repeat(np.ldexp(1.0, s), 32, axis=1)
    assert (np.abs(dq - v) <= half).all()


def _on_block_grid(r, shape, axis_len):
    """Values already on an FP8 block grid: every 32-block holds one element
    of magnitude exactly 448 * 2^s, the rest are E4M3 values times 2^s."""
    grid = omx.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    v = r.choice(grid, shape) * r.choice([-1.0, 1.0], shape)
    nb = axis_len // 32
    s = r.integers(-12, -4, shape[:-1] + (nb,))
    v = v.reshape(shape[:-1] + (nb, 32))
    v[..., 0] = 448.0 * r.choice([-1.0, 1.0], shape[:-1] + (nb,))
    v = v * np.ldexp(1.0, s)[..., None]
    return v.reshape(shape)


def check_fp8_layer_lossless_on_grid(T=24, d=64, I=32, N=5, Z=3, K=3, seed=17):
    r = _rng(seed)
    x = _on_block_grid(r, (T, d), d) * 64.0
    wr = r.standard_normal((N + Z, d)) / np.sqrt(d)
    wg = _on_block_grid(r, (N, I, d), d)
    wu = _on_block_grid(r, (N, I, d), d)
    wd = r.standard_normal((N, d, I)) / np.sqrt(I)
    b = r.uniform(-0.05, 0.05, N + Z)
    res = r.standard_normal((T, d))
    xq, xs = omx.mx_quantize(x)
    assert np.array_equal(omx.mx_dequantize(xq, xs), x)
    ref = om.forward(x, wr, b, wg, wu, wd, N, Z, K, residual=res)
    got = omx.forward_fp8_gateup(x, wr, b, wg, wu, wd, N, Z, K, residual=res)
    assert np.array_equal(got["idx"], ref["idx"]) and np.array_equal(got["y"], ref["y"])
    # identity experts pass x itself, never its FP8 image: with every slot on
    # an identity expert the two layers agree exactly off the grid too
    x3 = r.standard_normal((T, d))
    b3 = np.concatenate([np.full(N, -10.0), np.zeros(Z)])
    a3 = om.forward(x3, wr, b3, wg, wu, wd, N, Z, K, residual=res)["y"]
    c3 = omx.forward_fp8_gateup(x3, wr, b3, wg, wu, wd, N, Z, K, residual=res)["y"]
    assert np.array_equal(a3, c3)
    # off the grid the two differ, by about the FP8 rounding of the gate/up inputs
    x2 = r.standard_normal((T, d))
    wg2 = r.standard_normal((N, I, d)) / np.sqrt(d)
    a = om.forward(x2, wr, b, wg2, wu, wd, N, Z, K)["y"]
    c = omx.forward_fp8_gateup(x2, wr, b, wg2, wu, wd, N, Z, K)["y"]
    rel = np.abs(a - c).max() / np.abs(a).max()
    assert 1e-4 < rel < 0.1, rel


def check_fp8_down_hand_example():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fp8_down_example.json")))
    h = np.zeros((1, g["I"]))
    for k, v in g["h_nonzero"]:
        h[0, k] = v
    wd = np.zeros((g["d"], g["I"]))
    for j, k, v in g["w_down_nonzero"]:
        wd[j, k] = v
    o = omx.down_projection_fp8(h, wd)
    assert np.array_equal(o[0], np.array(g["o"])), o
    assert np.array_equal(h @ wd.T, np.array([g["o_unquantized_h"]]))


def check_fp8_down_lossless_on_grid(m=40, d=48, I=96, seed=21):
    # h and W_down on their block grids along I: the FP8 product is exact
    r = _rng(seed)
    h = _on_block_grid(r, (m, I), I)
    wd = _on_block_grid(r, (d, I), I)
    assert np.array_equal(omx.down_projection_fp8(h, wd), h @ wd.T)
    # off the grid it is the product of the operands' FP8 images: it moves by
    # about the rounding of both, relative 2^-4 per value at most
    h2 = r.standard_normal((m, I))
    wd2 = r.standard_normal((d, I))
    exact = h2 @ wd2.T
    rel = np.abs(omx.down_projection_fp8(h2, wd2) - exact).max() / np.abs(exact).max()
    assert 1e-4 < rel < 0.1, rel


def check_fp8_down_layer(T=24, d=64, I=64, N=5, Z=3, K=3, seed=22):
    r = _rng(seed)
    x = r.standard_normal((T, d))
    wr = r.standard_normal((N + Z, d)) / np.sqrt(d)
    wg = r.standard_normal((N, I, d)) / np.sqrt(d)
    wu = r.standard_normal((N, I, d)) / np.sqrt(d)
    wd = r.standard_normal((N, d, I)) / np.sqrt(I)
    b = r.uniform(-0.05, 0.05, N + Z)
    a = omx.forward_fp8_gateup(x, wr, b, wg, wu, wd, N, Z, K)
    c = omx.forward_fp8_gateup(x, wr, b, wg, wu, wd, N, Z, K, down_fp8=True)
    assert np.array_equal(a["idx"], c["idx"])              # routing is not quantized
    rel = np.abs(a["y"] - c["y"]).max() / np.abs(a["y"]).max()
    assert 1e-4 < rel < 0.1, rel
    # an expert's FP8 down projection is down_projection_fp8 of its fp64
    # hidden activation (from the dequantized gate/up operands)
    t = int(np.nonzero((c["idx"] < N).any(axis=1))[0][0])
    k = int(np.nonzero(c["idx"][t] < N)[0][0])
    e = int(c["idx"][t, k])
    q = lambda v: omx.mx_dequantize(*omx.mx_quantize(v, axis=-1), axis=-1)
    xq = q(x[t:t + 1])
    hid = om.silu(xq @ q(wg[e]).T) * (xq @ q(wu[e]).T)
    row = omx.down_projection_fp8(hid, wd[e])[0]
    y_wo = c["y"][t] - c["gate"][t, k] * row          # the slot's term removed ...
    y_a = a["y"][t] - a["gate"][t, k] * om.swiglu_ffn(xq, q(wg[e]), q(wu[e]), wd[e])[0]
    assert np.allclose(y_wo, y_a, rtol=0, atol=1e-12)  # ... leaves the same other terms
    # identity experts pass x itself: with every slot on one, both agree exactly
    b3 = np.concatenate([np.full(N, -10.0), np.zeros(Z)])
    a3 = omx.forward_fp8_gateup(x, wr, b3, wg, wu, wd, N, Z, K)["y"]
    c3 = omx.forward_fp8_gateup(x, wr, b3, wg, wu, wd, N, Z, K, down_fp8=True)["y"]
    assert np.array_equal(a3, c3)


# ------------------------------------------------------------- backward -----
def _loss(x, wr, b, wg, wu, wd, N, Z, K, dy):
    rt = om.forward(x, wr, b, wg, wu, wd, N, Z, K)
    return float((rt["y"] * dy).sum()), rt["idx"]


def check_backward_finite_differences(T=6, d=8, I=5, N=3, Z=2, K=2, seed=18, h=1e-3):
    r = _rng(seed)
    x = r.standard_normal((T, d))
    wr = r.standard_normal((N + Z, d)) / np.sqrt(d)
    wg = r.standard_normal((N, I, d)) / np.sqrt(d)
    wu = r.standard_normal((N, I, d)) / np.sqrt(d)
    wd = r.standard_normal((N, d, I)) / np.sqrt(I)
    b = r.uniform(-0.05, 0.05, N + Z)
    dy = r.standard_normal((T, d))
    g = obw.backward(x, wr, b, wg, wu, wd, N, Z, K, dy)
    _, idx0 = _loss(x, wr, b, wg, wu, wd, N, Z, K, dy)
    params = {"dx": x, "dw_router": wr, "dw_gate": wg, "dw_up": wu, "dw_down": wd}
    checked = 0
    for name, P in params.items():
        an = g[name]
        fd = np.full(P.shape, np.nan)
        for i in np.ndindex(P.shape):
            old = P[i]
            P[i] = old + h
            lp, ip = _loss(x, wr, b, wg, wu, wd, N, Z, K, dy)
            P[i] = old - h
            lm, im = _loss(x, wr, b, wg, wu, wd, N, Z, K, dy)
            P[i] = old
            if np.array_equal(ip, idx0) and np.array_equal(im, idx0):   # routing unchanged
                fd[i] = (lp - lm) / (2 * h)
        ok = ~np.isnan(fd)
        assert ok.mean() > 0.9, (name, ok.mean())
        err = np.abs(fd[ok] - an[ok]).max()
        assert err <= 2e-3 * max(np.abs(an).max(), 1e-3), (name, err, np.abs(an).max())
        checked += int(ok.sum())
    assert checked > 400


def check_backward_single_ffn_textbook(T=10, d=12, I=7, seed=19):
    # one FFN expert, K = 1: p = 1, so y = FFN(x) + r and the router gets nothing
    import torch
    r = _rng(seed)
    x = r.standard_normal((T, d))
    wr = r.standard_normal((1, d))
    wg = r.standard_normal((1, I, d)) / np.sqrt(d)
    wu = r.standard_normal((1, I, d)) / np.sqrt(d)
    wd = r.standard_normal((1, d, I)) / np.sqrt(I)
    dy = r.standard_normal((T, d))
    g = obw.backward(x, wr, np.zeros(1), wg, wu, wd, 1, 0, 1, dy)
    tx, tg, tu, td = (torch.tensor(a, dtype=torch.float64, requires_grad=True)
                      for a in (x, wg[0], wu[0], wd[0]))
    y = (torch.nn.functional.silu(tx @ tg.T) * (tx @ tu.T)) @ td.T
    (y * torch.tensor(dy)).sum().backward()
    for name, t in (("dx", tx), ("dw_down", td)):
        ref = t.grad.numpy()
        got = g[name] if name == "dx" else g[name][0]
        assert np.abs(got - ref).max() <= 1e-12 * max(np.abs(ref).max(), 1.0), name
    assert np.abs(g["dw_gate"][0] - tg.grad.numpy()).max() <= 1e-12 * max(np.abs(tg.grad.numpy()).max(), 1.0)
    assert np.abs(g["dw_up"][0] - tu.grad.numpy()).max() <= 1e-12 * max(np.abs(tu.grad.numpy()).max(), 1.0)
    assert not g["dw_router"].any()


def check_backward_identity_closed_form(T=20, d=9, Z=5, K=3, seed=20):
    # identity experts only: y_t = (sum over chosen p) x_t + r_t
    r = _rng(seed)
    x = r.standard_normal((T, d))
    wr = r.standard_normal((Z, d)) / np.sqrt(d)
    b = r.uniform(-0.05, 0.05, Z)
    dy = r.standard_normal((T, d))
    g = obw.backward(x, wr, b, np.zeros((0, 1, d)), np.zeros((0, 1, d)), np.zeros((0, d, 1)),
                     0, Z, K, dy)
    rt = g["route"]
    p, idx = rt["p64"], rt["idx"]
    chosen = np.zeros_like(p)
    np.put_along_axis(chosen, idx, 1.0, axis=1)
    sel = (p * chosen).sum(axis=1)                   # sum of the chosen gates
    xy = (x * dy).sum(axis=1)
    # d/dl_j of sum_{i chosen} p_i = p_j ([j chosen] - sel)
    dl = xy[:, None] * p * (chosen - sel[:, None])
    assert np.allclose(g["dlogits"], dl, rtol=1e-12, atol=1e-14)
    # the direct path multiplies x by the gates as stored (fl32 of p)
    gsum = rt["gate"].astype(np.float64).sum(axis=1)
    assert np.allclose(g["dx"], gsum[:, None] * dy + dl @ wr, rtol=1e-12, atol=1e-12)
    assert np.allclose(g["dw_router"], dl.T @ x, rtol=1e-12, atol=1e-12)


ALL_CHECKS = [
    check_hand_example, check_pid_golden, check_bruteforce_tiny,
    check_topk_ties_enumeration, check_softmax_bruteforce,
    check_single_forced_ffn, check_all_identity, check_k_equals_e,
    check_z_zero_textbook_moe, check_permutation_invariants,
    check_token_independence, check_ffn_count_hypergeometric,
    check_pid_properties, check_budget_target, check_closed_loop_fixed_point,
    check_closed_loop_conservation_and_positional_form,
    check_closed_loop_integral_settles, check_e4m3_codes, check_e4m3_rounding_bruteforce,
    check_mx_scales_minimal, check_fp8_layer_lossless_on_grid,
    check_fp8_down_hand_example, check_fp8_down_lossless_on_grid, check_fp8_down_layer,
    check_backward_finite_differences, check_backward_single_ffn_textbook,
    check_backward_identity_closed_form,
]
