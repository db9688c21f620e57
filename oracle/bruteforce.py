"""Pure-Python loop version of the layer for tiny shapes (TEST INFRASTRUCTURE).

Written independently of the vectorised oracle, from the same definition
(see the module docstring of ``oracle.moe_zc``), so that each can pin the
other: dot products by math.fsum, softmax by math.exp, the top-K set by
enumerating every K-subset of experts, the grouping by nested loops.
Suitable for T*E*d up to about 1e6.
"""
from __future__ import annotations

import itertools
import math

import numpy as np


def _rows(a):
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64).tolist()


def logits(x, w_router):
    X, W = _rows(x), _rows(w_router)
    return [[math.fsum(a * b for a, b in zip(xt, wi)) for wi in W] for xt in X]


def softmax_row(l32_row):
    vals = [float(np.float32(v)) for v in l32_row]
    m = max(vals)
    ex = [math.exp(v - m) for v in vals]
    s = math.fsum(ex)
    return [v / s for v in ex]


def _beats(a, b, key):
    """Expert a precedes expert b: larger key, or equal key and lower index."""
    return key[a] > key[b] or (key[a] == key[b] and a < b)


def topk_by_enumeration(key_row, K):
    """The unique K-subset whose every member precedes every non-member,
    found by checking all C(E, K) subsets; returned in precedence order."""
    E = len(key_row)
    found = None
    for sub in itertools.combinations(range(E), K):
        inside = set(sub)
        if all(_beats(a, b, key_row) for a in sub for b in range(E) if b not in inside):
            if found is not None:
                raise AssertionError("more than one dominating subset")
            found = sub
    if found is None:
        raise AssertionError("no dominating subset")
    # order the chosen experts by precedence (selection sort with _beats)
    rest = list(found)
    ordered = []
    while rest:
        best = rest[0]
        for c in rest[1:]:
            if _beats(c, best, key_row):
                best = c
        ordered.append(best)
        rest.remove(best)
    return ordered


def swiglu_row(xt, wg, wu, wd):
    I = len(wg)
    h = []
    for j in range(I):
        a = math.fsum(p * q for p, q in zip(wg[j], xt))
        u = math.fsum(p * q for p, q in zip(wu[j], xt))
        h.append(a / (1.0 + math.exp(-a)) * u)
    return [math.fsum(wd[c][j] * h[j] for j in range(I)) for c in range(len(wd))]


def forward(x, w_router, bias, w_gate, w_up, w_down, N, Z, K, residual=None,
            logits32=None):
    X = _rows(x)
    T, d = len(X), len(X[0])
    E = N + Z
    if logits32 is None:
        l32 = [[float(np.float32(v)) for v in row] for row in logits(x, w_router)]
    else:
        l32 = [[float(v) for v in row] for row in np.asarray(logits32, np.float32)]
    b32 = [np.float32(v) for v in np.asarray(bias, dtype=np.float32)]
    WG = [_rows(w_gate[e]) for e in range(N)]
    WU = [_rows(w_up[e]) for e in range(N)]
    WD = [_rows(w_down[e]) for e in range(N)]
    R = _rows(residual) if residual is not None else None
    idx, gate, y = [], [], []
    for t in range(T):
        p = softmax_row(l32[t])
        p32 = [np.float32(v) for v in p]
        key = [float(np.float32(p32[i] + b32[i])) for i in range(E)]
        chosen = topk_by_enumeration(key, K)
        idx.append(chosen)
        gate.append([float(p32[i]) for i in chosen])
        acc = [0.0] * d if R is None else list(R[t])
        for i in chosen:
            out = swiglu_row(X[t], WG[i], WU[i], WD[i]) if i < N else X[t]
            g = float(p32[i])
            acc = [a + g * o for a, o in zip(acc, out)]
        y.append(acc)
    loads = [0] * E
    for row in idx:
        for i in row:
            loads[i] += 1
    perm, pos = [], [[-1] * K for _ in range(T)]
    for e in range(N):
        for t in range(T):
            for k in range(K):
                if idx[t][k] == e:
                    pos[t][k] = len(perm)
                    perm.append(t)
    return {"idx": np.array(idx), "gate": np.array(gate, dtype=np.float32),
            "y": np.array(y), "loads": np.array(loads), "perm": np.array(perm),
            "pos": np.array(pos), "logits32": np.array(l32, dtype=np.float32)}
