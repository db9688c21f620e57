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


def run_gpu(w, inp, residual=True, workspace=None, events=None, packed=None, fp8=False,
            act=False, down_fp8=False):
    """One forward through the C ABI; ``packed`` = (gate_up, down) from
    moe_zc_pack_expert_weights selects moe_zc_forward_packed, and with ``fp8``
    ``packed`` = (gate_up_fp8, down) selects moe_zc_forward_packed_fp8 (down in
    FP8 when ``down_fp8``).  With
    ``act`` the forward also saves the expert pre-activations (aux "act", left
    on the device as out["act_t"])."""
    dev = inp["x"].device
    keys = m.AUX_KEYS + (("act",) if act else ())
    aux = m.alloc_aux(w.T, w.N, w.Z, w.K, dev, keys=keys, I=w.I if act else None)
    res = inp["residual"] if residual else None
    if fp8:
        gu, dn = packed if packed is not None else (None, None)
        y = m.moe_zc_forward_packed_fp8(inp["x"], inp["w_router"], inp["bias"], gu, dn,
                                        w.N, w.Z, w.K, w.I, residual=res, aux=aux,
                                        workspace=workspace, events=events, down_fp8=down_fp8)
    elif packed is None:
        y = m.moe_zc_forward(inp["x"], inp["w_router"], inp["bias"], inp["w_gate"], inp["w_up"],
                             inp["w_down"], w.N, w.Z, w.K, residual=res, aux=aux,
                             workspace=workspace, events=events)
    else:
        y = m.moe_zc_forward_packed(inp["x"], inp["w_router"], inp["bias"], packed[0], packed[1],
                                    w.N, w.Z, w.K, w.I, residual=res, aux=aux,
                                    workspace=workspace, events=events)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in aux.items() if k != "act"}
    if act:
        out["act_t"] = aux["act"]
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


def check_forward(w, inp, g, y_tokens=None, max_flip_frac=1e-3, get_expert=None, fp8=False,
                  down_fp8=False):
    """Compare a GPU forward (``g`` from run_gpu) with the oracle (with the
    gate/up projection in block FP8 when ``fp8``, and the down projection too
    when ``down_fp8``)."""
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
    res_t = None if res is None else res[toks]
    if fp8:
        y_ref, _ = oracle.mx.forward_tokens_fp8(x[toks], l32[toks], b, get_expert, N, K, res_t,
                                                down_fp8=down_fp8)
    else:
        y_ref, _ = oracle.forward_tokens(x[toks], l32[toks], b, get_expert, N, K, res_t)
    scale = max(np.abs(y_ref).max(), 1e-30)
    tol = Y_TOL[w.dtype] * scale
    diff = np.abs(g["y"][toks] - y_ref)
    err = diff.max() if len(toks) else 0.0
    out = {"logit_err": float(lerr), "y_err": float(err), "y_tol": float(tol),
           "flips": int(len(flips)), "clean_frac": float(clean.mean()),
           "S": int(g["offsets"][N]), "tokens_checked": int(len(toks))}
    if down_fp8 and len(toks):
        ok, n_over, why = fp8_down_bar(
            diff, tol, lambda o: fp8_down_code_flip_allowance(x[toks[o]], l32[toks[o]], b,
                                                              get_expert, N, K))
        assert ok, why
        out["code_flip_tokens"] = n_over
    else:
        assert err <= tol, f"y: max|err| {err:.3e} > {tol:.3e}"
    return out


def fp8_down_bar(diff, tol, allowance_of):
    """The layer-output bar of the FP8 down projection.  diff = |y - y_ref|
    [tokens, d]; allowance_of(rows) gives fp8_down_code_flip_allowance for
    those rows of the token set.  Every token within tol, except tokens where
    an FP8 code of h flipped next to a rounding point: those must be rare (at
    most max(1, 0.2%) of the tokens, as near-tie routing flips are) and each
    excess within one flip per slot.  Returns (ok, tokens over tol, reason)."""
    over = np.nonzero((diff > tol).any(axis=1))[0]
    if len(over) == 0:
        return True, 0, ""
    if len(over) > max(1, int(2e-3 * diff.shape[0])):
        return False, len(over), f"{len(over)} tokens over the bar {tol:.3e}"
    excess = (diff[over] - allowance_of(over)).max()
    if excess > tol:
        return False, len(over), f"y: max|err| less one code flip per slot {excess:.3e} > {tol:.3e}"
    return True, len(over), ""


def fp8_down_code_flip_allowance(x_rows, logits32_rows, bias, get_expert, N, K):
    """What one flipped FP8 code of h per slot can move the FP8 down
    projection's output by, per token and output column [T, d].

    The GPU quantizes h = silu(a) u from its fp32 value, the oracle from its
    fp64 value (the reading of the FP8 down projection: h is quantized from
    its value as computed).  The code is an integer that floating point
    decides: where h lies within the fp32 error of a rounding midpoint,
    either neighbouring code is correct, as either expert is at a near-tie
    in routing, and the two sides' codes then differ by one step of the E4M3
    grid at that magnitude (times the block's scale).  The output moves by
    that step times g |W_down_dq[j, i]|.  Such flips are rare (the fp32
    error is about 1e-6 of h, a step about 1/8), so this allows the largest
    single flip in each slot's row of h."""
    mx = oracle.mx
    x64 = x_rows.double().numpy() if torch.is_tensor(x_rows) else np.asarray(x_rows, np.float64)
    x_dq = mx.mx_dequantize(*mx.mx_quantize(x64, axis=-1), axis=-1)
    rt = oracle.route(logits32_rows, bias, K, N)
    idx, gate = rt["idx"], rt["gate"].astype(np.float64)
    allow = np.zeros_like(x64)
    for e in np.unique(idx[idx < N]):
        tt, kk = np.nonzero(idx == e)
        wg, wu, wd = (w.double().numpy() if torch.is_tensor(w) else np.asarray(w, np.float64)
                      for w in get_expert(int(e)))
        wg, wu, wd = (mx.mx_dequantize(*mx.mx_quantize(w, axis=-1), axis=-1)
                      for w in (wg, wu, wd))
        a, u = x_dq[tt] @ wg.T, x_dq[tt] @ wu.T
        h = a / (1.0 + np.exp(-a)) * u
        m, n = h.shape
        hb = h.reshape(m, n // 32, 32)
        sc = mx.mx_scale_exponent(np.abs(hb).max(axis=-1))
        f = np.ldexp(1.0, sc)[..., None]
        v = np.abs(hb) / f                              # scaled magnitude, <= 448
        # grid step at v: 2^(E - 3) in a normal binade [2^E, 2^(E+1)), 2^-9
        # below 2^-6; at a binade's lower edge the step below is half as
        # large, so the larger one bounds a flip either way
        ex = np.floor(np.log2(np.maximum(v, 2.0 ** -6)))
        step = (np.ldexp(1.0, (ex - 3).astype(np.int64)) * f).reshape(m, n)
        flip = np.abs(wd)[None, :, :] * step[:, None, :]   # [rows, d, I]
        allow[tt] += gate[tt, kk][:, None] * flip.max(axis=-1)
    return allow


def gpu_expert_getter(inp):
    """Expert weights fetched from the device one expert at a time."""
    def get(e):
        return inp["w_gate"][e].cpu(), inp["w_up"][e].cpu(), inp["w_down"][e].cpu()
    return get


def check_act(w, inp, g, experts, fp8=False, get_expert=None):
    """Pre-activations a | u that the forward saved (aux "act", bf16) for every
    grouped row of each expert in ``experts``, against the oracle's fp64
    a = x W_gate^T and u = x W_up^T of the same tokens (with ``fp8``, on the
    oracle's dequantized block-FP8 operands).  Every hidden unit of every row
    is compared, so each weight panel and row block of those experts' tiles
    is covered.  Bar: max |act - ref| <= 1e-2 * max |ref| per expert (the
    layer's bf16 bar; the stored values carry one bf16 rounding)."""
    off = g["offsets"]
    perm = g["perm"]
    x = inp["x"].cpu()
    if get_expert is None:
        get_expert = gpu_expert_getter(inp)
    out = {}
    for e in experts:
        r0, r1 = int(off[e]), int(off[e + 1])
        assert r1 > r0, f"expert {e} has no rows"
        wg, wu, _ = get_expert(int(e))
        wg, wu = oracle.moe_zc._f64(wg), oracle.moe_zc._f64(wu)
        if fp8:
            wg = oracle.mx.mx_dequantize(*oracle.mx.mx_quantize(wg, axis=-1), axis=-1)
            wu = oracle.mx.mx_dequantize(*oracle.mx.mx_quantize(wu, axis=-1), axis=-1)
        xr = oracle.moe_zc._f64(x[torch.from_numpy(perm[r0:r1].astype(np.int64))])
        if fp8:  # x is quantized per token, so its rows quantize alone
            xr = oracle.mx.mx_dequantize(*oracle.mx.mx_quantize(xr, axis=-1), axis=-1)
        ref = np.concatenate([xr @ wg.T, xr @ wu.T], axis=1)
        got = g["act_t"][r0:r1].float().cpu().double().numpy()
        scale = np.abs(ref).max()
        err = np.abs(got - ref).max()
        assert err <= 1e-2 * scale, f"act of expert {e}: {err:.3e} > 1e-2 * {scale:.3e}"
        out[int(e)] = {"rows": r1 - r0, "err_frac": float(err / scale)}
    return out


def act_experts(loads, N, rng, tile_rows=256):
    """Experts whose whole rows check_act covers: the most loaded (split over
    two row tiles when it holds more than ``tile_rows`` rows), the least loaded
    touched one, and two random touched ones."""
    ld = np.asarray(loads[:N])
    touched = np.nonzero(ld > 0)[0]
    hi = int(touched[np.argmax(ld[touched])])
    lo = int(touched[np.argmin(ld[touched])])
    rest = np.setdiff1d(touched, [hi, lo])
    pick = rng.choice(rest, min(2, len(rest)), replace=False).tolist()
    return [hi, lo] + [int(e) for e in pick]


def sample_tokens(g, N, rng, n_random=48, n_split=16, tile_rows=256):
    """Tokens for the layer-output check: ``n_random`` at random plus up to
    ``n_split`` whose rows sit in the second row part of an expert that the
    GEMM splits over two tiles (more than ``tile_rows`` rows), so that every
    tile class is exercised."""
    T = g["topk_idx"].shape[0]
    off = g["offsets"]
    loads = np.diff(off)
    split = np.nonzero(loads > tile_rows)[0]
    picks = set(rng.choice(T, min(n_random, T), replace=False).tolist())
    if len(split):
        for e in rng.choice(split, min(n_split, len(split)), replace=False):
            mt = (loads[e] + tile_rows - 1) // tile_rows
            rpt = ((loads[e] + mt - 1) // mt + 31) // 32 * 32   # rows of the first part
            r = rng.integers(off[e] + rpt, off[e + 1])
            picks.add(int(g["perm"][r]))
    return np.array(sorted(picks))
