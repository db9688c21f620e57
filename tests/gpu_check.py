"""Comparison of the HIP path with the fp64 oracle (used by the GPU tests).

Routing.  Both sides choose experts from fp32 logits: the oracle from its fp64
logits rounded once, the GPU from its own fp32 logits (within 1e-4 of fp64).
Where a token's top keys are separated by more than what that logit error can
move them, the choice is unique and must match exactly (indices and order).
Where two keys are closer than that, either choice is correct; the GPU's must
then be a valid one (no chosen expert's oracle key below an unchosen one's by
more than the bound) and such tokens must be rare.

Grouping.  loads, offsets, perm and pos are checked for validity against the
GPU's own routing (bijection, expert-major, tokens ascending) and, when every
token's expert set matches the oracle's, for exact equality with the oracle.

Output.  y is compared with the oracle's fp64 y on tokens whose expert sets
match: max |y - y_ref| <= 1e-2 * max |y_ref| for bf16 storage, 1e-5 for fp32.
"""
from __future__ import annotations

import numpy as np
import torch

import mixture_experts_layer_bias_amd as m
import oracle

LOGIT_TOL = 1e-4
Y_TOL = {"bf16": 1e-2, "f32": 1e-5}


def run_gpu(w, inp, residual=True, workspace=None, events=None, packed=None, fp8=False):
    """One forward through the C ABI; ``packed`` = (gate_up, down) from
    moe_zc_pack_expert_weights selects moe_zc_forward_packed, and with ``fp8``
    ``packed`` = (gate_up_fp8, down) selects moe_zc_forward_packed_fp8."""
    dev = inp["x"].device
    aux = m.alloc_aux(w.T, w.N, w.Z, w.K, dev)
    res = inp["residual"] if residual else None
    if fp8:
        gu, dn = packed if packed is not None else (None, None)
        y = m.moe_zc_forward_packed_fp8(inp["x"], inp["w_router"], inp["bias"], gu, dn,
                                        w.N, w.Z, w.K, w.I, residual=res, aux=aux,
                                        workspace=workspace, events=events)
    elif packed is None:
        y = m.moe_zc_forward(inp["x"], inp["w_router"], inp["bias"], inp["w_gate"], inp["w_up"],
                             inp["w_down"], w.N, w.Z, w.K, residual=res, aux=aux,
                             workspace=workspace, events=events)
    else:
        y = m.moe_zc_forward_packed(inp["x"], inp["w_router"], inp["bias"], packed[0], packed[1],
                                    w.N, w.Z, w.K, w.I, residual=res, aux=aux,
                                    workspace=workspace, events=events)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in aux.items()}
    out["y_t"] = y
    out["y"] = y.float().cpu().double().numpy()
    return out


def key_bound(p64):
    """How far a selection key can move when every logit moves by <= LOGIT_TOL:
    |dp_i| <= 2 p_i max|dl|, plus fp32 rounding of p and of p + b."""
    return 4.0 * LOGIT_TOL * p64.max(axis=1) + 1e-6


def validate_grouping(idx, loads, offsets, perm, pos, N, E):
    T, K = idx.shape
    assert (idx >= 0).all() and (idx < E).all()
    for t in range(min(T, 4096)):
        assert len(set(idx[t].tolist())) == K, f"token {t} repeats an expert"
    assert np.array_equal(loads, np.bincount(idx.ravel(), minlength=E)), "loads"
    assert loads.sum() == T * K
    off = np.zeros(N + 1, dtype=np.int64)
    off[1:] = np.cumsum(loads[:N])
    assert np.array_equal(offsets, off), "offsets"
    S = int(off[N])
    ffn = idx < N
    assert (pos[~ffn] == -1).all(), "zero-expert slots must have pos -1"
    rows = pos[ffn]
    assert np.array_equal(np.sort(rows), np.arange(S)), "pos is not a bijection onto rows"
    tt = np.nonzero(ffn)[0]
    assert np.array_equal(perm[rows], tt), "perm[pos[t,k]] != t"
    ee = idx[ffn]
    assert ((rows >= off[ee]) & (rows < off[ee + 1])).all(), "row outside its expert block"
    for e in range(N):
        blk = perm[off[e]:off[e + 1]]
        assert (np.diff(blk) > 0).all(), f"expert {e}: tokens not ascending"


def check_forward(w, inp, g, y_tokens=None, max_flip_frac=1e-3, get_expert=None, fp8=False):
    """Compare a GPU forward (``g`` from run_gpu) with the oracle (with the
    gate/up projection in block FP8 when ``fp8``)."""
    T, N, K, E = w.T, w.N, w.K, w.E
    x = inp["x"].cpu()
    wr = inp["w_router"].cpu()
    b = inp["bias"].cpu().numpy()
    res = inp["residual"].cpu() if inp.get("residual") is not None else None
    l64 = oracle.router_logits(x, wr)
    lerr = np.abs(g["logits"].astype(np.float64) - l64).max()
    assert lerr <= LOGIT_TOL, f"router logits off by {lerr}"
    l32 = l64.astype(np.float32)
    rt = oracle.route(l32, b, K, N)
    key, p64 = rt["key"].astype(np.float64), rt["p64"]
    gi = g["topk_idx"].astype(np.int64)
    bound = key_bound(p64)
    srt = -np.sort(-key, axis=1)[:, : min(K + 1, E)]
    gaps = srt[:, :-1] - srt[:, 1:]
    clean = gaps.min(axis=1) > bound if gaps.shape[1] else np.ones(T, bool)
    assert np.array_equal(gi[clean], rt["idx"][clean]), "routing differs on a clean token"
    same = (np.sort(gi, axis=1) == np.sort(rt["idx"], axis=1)).all(axis=1)
    flips = np.nonzero(~same)[0]
    for t in flips:
        chosen = np.zeros(E, bool)
        chosen[gi[t]] = True
        assert key[t][chosen].min() >= key[t][~chosen].max() - bound[t], f"token {t}: invalid choice"
    assert len(flips) <= max(1, int(max_flip_frac * T)), f"{len(flips)} near-tie flips"
    # gates of matching tokens, expert by expert
    gref = {}
    for t in np.nonzero(same)[0][:2048]:
        gref = dict(zip(rt["idx"][t].tolist(), rt["gate"][t].tolist()))
        for e, gg in zip(gi[t].tolist(), g["topk_gate"][t].tolist()):
            assert abs(gg - gref[e]) <= 3 * LOGIT_TOL * gref[e] + 1e-7, (t, e, gg, gref[e])
    validate_grouping(gi, g["loads"], g["offsets"], g["perm"], g["pos"], N, E)
    if same.all():
        assert np.array_equal(g["loads"], rt["loads"]), "loads vs oracle"
        assert np.array_equal(g["offsets"], rt["offsets"]), "offsets vs oracle"
        S = rt["n_rows"]
        assert np.array_equal(g["perm"][:S], rt["perm"]), "perm vs oracle"
        # pos as a map (token, expert) -> row, independent of slot order
        for t in range(min(T, 4096)):
            mg = {e: r for e, r in zip(gi[t].tolist(), g["pos"][t].tolist())}
            mo = {e: r for e, r in zip(rt["idx"][t].tolist(), rt["pos"][t].tolist())}
            assert mg == mo, f"pos of token {t}"
    toks = np.arange(T) if y_tokens is None else np.asarray(y_tokens)
    toks = toks[same[toks]]
    if get_expert is None:
        wg, wu, wd = (inp[k].cpu() for k in ("w_gate", "w_up", "w_down"))

        def get_expert(e):
            return wg[e], wu[e], wd[e]
    fwd = oracle.mx.forward_tokens_fp8 if fp8 else oracle.forward_tokens
    y_ref, _ = fwd(x[toks], l32[toks], b, get_expert, N, K, None if res is None else res[toks])
    scale = max(np.abs(y_ref).max(), 1e-30)
    err = np.abs(g["y"][toks] - y_ref).max() if len(toks) else 0.0
    tol = Y_TOL[w.dtype] * scale
    assert err <= tol, f"y: max|err| {err:.3e} > {tol:.3e}"
    return {"logit_err": float(lerr), "y_err": float(err), "y_tol": float(tol),
            "flips": int(len(flips)), "clean_frac": float(clean.mean()),
            "S": int(g["offsets"][N]), "tokens_checked": int(len(toks))}


def gpu_expert_getter(inp):
    """Expert weights fetched from the device one expert at a time."""
    def get(e):
        return inp["w_gate"][e].cpu(), inp["w_up"][e].cpu(), inp["w_down"][e].cpu()
    return get
