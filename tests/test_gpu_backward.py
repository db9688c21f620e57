"""Backward of the layer (moe_zc_transpose_expert_weights, moe_zc_backward)
against the fp64 oracle's gradients (oracle.backward).

The forward on the GPU saves its routing (fp32 logits, top-K, gates, grouping);
the oracle routes from those same fp32 logits, so both differentiate the same
piecewise-smooth function.  Tolerance, per output tensor:
max |G - G_ref| <= 1e-2 * max |G_ref|, the forward's bf16 bar.  The GPU rounds
da, du, h, g dy and dl to bf16 as operands of fp32-accumulated products (a
relative 2^-9 per operand), and dx once at the end, so errors sit near 1e-3
of the maximum.  Determinism is exact: two calls give the same bits."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_bias_amd as m
from oracle import backward as obwd
from workloads import Workload, get_workload, make_inputs, make_upstream_grad

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 1e-2
GRADS = ("dx", "dw_router", "dw_gate", "dw_up", "dw_down")


def _edge(T=200, d=128, I=128, N=8, Z=4, K=3, seed=5, bias=("uniform", 0.05), zipf=None):
    return Workload("edge", T=T, d=d, I=I, N=N, Z=Z, K=K, dtype="bf16", seed=seed, bias=bias,
                    zipf=zipf)


def gpu_forward_backward(w, inp, dy, repeat=1):
    aux = m.alloc_aux(w.T, w.N, w.Z, w.K, DEV)
    m.moe_zc_forward(inp["x"], inp["w_router"], inp["bias"], inp["w_gate"], inp["w_up"],
                     inp["w_down"], w.N, w.Z, w.K, aux=aux)
    tr = None
    if w.N > 0:
        tr = m.moe_zc_transpose_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    outs = []
    for _ in range(repeat):
        outs.append(m.moe_zc_backward(inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"], tr,
                                      aux, dy, w.N, w.Z, w.K, w.I))
    torch.cuda.synchronize()
    return aux, outs


def compare(w, inp, dy, aux, g, dx_tokens=None):
    """Every gradient against the oracle's; dx optionally on a token sample
    (the weight gradients need every token)."""
    l32 = aux["logits"].cpu().numpy()
    ref = obwd.backward(inp["x"].cpu(), inp["w_router"].cpu(), inp["bias"].cpu().numpy(),
                        inp["w_gate"].cpu(), inp["w_up"].cpu(), inp["w_down"].cpu(),
                        w.N, w.Z, w.K, dy.cpu(), logits32=l32)
    assert np.array_equal(aux["topk_idx"].cpu().numpy(), ref["route"]["idx"]), "routing"
    rep = {}
    for k in GRADS:
        got = g[k].float().cpu().double().numpy()
        want = ref[k]
        if k == "dx" and dx_tokens is not None:
            got, want = got[dx_tokens], want[dx_tokens]
        scale = np.abs(want).max() if want.size else 0.0
        err = np.abs(got - want).max() if want.size else 0.0
        rep[k] = float(err / scale) if scale > 0 else float(err)
        assert err <= TOL * scale + 1e-30, f"{k}: max|err| {err:.3e} > {TOL} * {scale:.3e}"
    # experts no token chose have exactly zero weight gradients
    if w.N > 0:
        loads = np.bincount(ref["route"]["idx"].ravel(), minlength=w.E)[: w.N]
        for k in ("dw_gate", "dw_up", "dw_down"):
            assert not g[k][torch.from_numpy(loads == 0).to(DEV)].any(), k
    return rep


CASES = {
    "T1": dict(T=1),
    "T65_ragged": dict(T=65),
    "Z0": dict(N=8, Z=0, K=2),
    "K_eq_E": dict(N=5, Z=3, K=8),
    "N0_all_identity": dict(N=0, Z=6, K=3),
    "N1_single_expert": dict(N=1, Z=3, K=2),
    "few_rows_32_tiles": dict(T=64, N=64, Z=32, K=8),
    "rows_128_tiles": dict(T=512, N=24, Z=8, K=6),
    "rows_256_tiles": dict(T=1100, N=8, Z=4, K=3, d=256, I=256),
    "wide_d": dict(T=130, d=1344, I=384, N=6, Z=2, K=2),
    "many_experts": dict(T=300, d=128, I=128, N=300, Z=20, K=12),
    # experts of 257 .. 439 rows: two row parts each in the forward's GEMMs
    "rows_past_256": dict(T=1300, d=320, I=384, N=10, Z=4, K=3, seed=3),
    # the most experts the library takes (E = 2048): the weight gradients'
    # XCD plan sorts 1800 groups and assigns them in 29 batches of 64
    "max_experts": dict(T=400, N=1800, Z=248, K=12),
    # Zipf(2) logit offsets: one expert takes most rows, so its weight
    # gradients are long reductions and the plan's per-XCD group cap binds
    "zipf_one_dominant": dict(T=2000, N=16, Z=8, K=4, bias=("zero",), zipf=(2.0, 4.0)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_backward_vs_oracle(name):
    w = _edge(**CASES[name])
    print(f"[backward {name}] {w.describe()}", flush=True)
    inp = make_inputs(w, device=DEV)
    dy = make_upstream_grad(w, DEV)
    aux, (g,) = gpu_forward_backward(w, inp, dy)
    print(name, compare(w, inp, dy, aux, g), flush=True)


def test_backward_mid_vs_oracle():
    w = get_workload("mid")
    print(f"[backward mid] {w.describe()}", flush=True)
    inp = make_inputs(w, device=DEV)
    dy = make_upstream_grad(w, DEV)
    aux, (g,) = gpu_forward_backward(w, inp, dy)
    print("mid", compare(w, inp, dy, aux, g), flush=True)


def test_backward_is_deterministic():
    """Bitwise-equal gradients on repeated calls (no atomics, fixed orders)."""
    w = _edge(T=1500, d=256, I=256, N=16, Z=8, K=6)
    inp = make_inputs(w, device=DEV)
    dy = make_upstream_grad(w, DEV)
    _, outs = gpu_forward_backward(w, inp, dy, repeat=3)
    for k in GRADS:
        for o in outs[1:]:
            assert torch.equal(outs[0][k].view(torch.int16 if k == "dx" else torch.int32),
                               o[k].view(torch.int16 if k == "dx" else torch.int32)), k


@pytest.mark.parametrize("n,d,I", [(3, 128, 256), (2, 320, 128), (1, 512, 384)])
def test_transpose_expert_weights(n, d, I):
    """The packed transposes equal the packed layout (the down projection's,
    checked byte for byte against its definition in test_gpu_packed) of
    [W_gate; W_up]^T and W_down^T."""
    from test_gpu_packed import _u16, pack_reference
    g = torch.Generator().manual_seed(7 * n + d)
    wg, wu = (torch.randn(n, I, d, generator=g).to(torch.bfloat16) for _ in range(2))
    wd = torch.randn(n, d, I, generator=g).to(torch.bfloat16)
    gut, dnt = m.moe_zc_transpose_expert_weights(wg.to(DEV), wu.to(DEV), wd.to(DEV))
    torch.cuda.synchronize()
    gb, db = m.moe_zc_transposed_expert_bytes(d, I)
    assert gut.numel() == n * gb and dnt.numel() == n * db
    ref_gu = pack_reference(_u16(torch.cat([wg, wu], dim=1).transpose(1, 2)), None, False)
    ref_dn = pack_reference(_u16(wd.transpose(1, 2)), None, False)
    assert np.array_equal(gut.cpu().numpy().reshape(n, -1), ref_gu)
    assert np.array_equal(dnt.cpu().numpy().reshape(n, -1), ref_dn)


def test_backward_empty_batch():
    w = _edge(T=0)
    inp = make_inputs(w, device=DEV)
    dy = make_upstream_grad(w, DEV)
    aux, (g,) = gpu_forward_backward(w, inp, dy)
    assert g["dx"].shape == (0, w.d)


def test_backward_rejects_f32():
    w = Workload("f32", T=16, d=128, I=256, N=4, Z=2, K=2, dtype="f32", seed=0,
                 bias=("zero",))
    inp = make_inputs(w, device=DEV)
    aux = m.alloc_aux(w.T, w.N, w.Z, w.K, DEV)
    with pytest.raises(ValueError):
        m.moe_zc_backward(inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"], None, aux,
                          inp["x"], w.N, w.Z, w.K, w.I)


# ---- pre-activations saved by the forward --------------------------------------
def _act_reference(w, inp, aux, fp8=False):
    """a | u of every grouped row in fp64 from the GPU's grouping (perm,
    offsets), on the dequantized FP8 operands when ``fp8``."""
    from oracle import mx as omx
    x = inp["x"].float().cpu().double().numpy()
    if fp8:
        x = omx.mx_dequantize(*omx.mx_quantize(x, axis=-1), axis=-1)
    perm = aux["perm"].cpu().numpy()
    off = aux["offsets"].cpu().numpy()
    ref = np.zeros((int(off[w.N]), 2 * w.I))
    for e in range(w.N):
        rows = slice(int(off[e]), int(off[e + 1]))
        if off[e + 1] == off[e]:
            continue
        wg = inp["w_gate"][e].float().cpu().double().numpy()
        wu = inp["w_up"][e].float().cpu().double().numpy()
        if fp8:
            wg = omx.mx_dequantize(*omx.mx_quantize(wg, axis=-1), axis=-1)
            wu = omx.mx_dequantize(*omx.mx_quantize(wu, axis=-1), axis=-1)
        xe = x[perm[rows]]
        ref[rows, : w.I] = xe @ wg.T
        ref[rows, w.I:] = xe @ wu.T
    return ref


@pytest.mark.parametrize("name", ["T65_ragged", "few_rows_32_tiles", "rows_256_tiles", "wide_d"])
def test_forward_saves_preactivations(name):
    """Saving a | u leaves y unchanged bit for bit, the saved values match fp64
    (bf16 storage bar), and the packed and row-major forwards save the same
    bits; the block-FP8 forward saves its own products."""
    w = _edge(**CASES[name])
    print(f"[act {name}] {w.describe()}", flush=True)
    inp = make_inputs(w, device=DEV)
    keys = m.AUX_KEYS + ("act",)
    packed = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    outs = {}
    for kind in ("rowmajor", "packed", "plain"):
        aux = m.alloc_aux(w.T, w.N, w.Z, w.K, DEV, keys=keys if kind != "plain" else m.AUX_KEYS,
                          I=w.I)
        if kind == "rowmajor":
            y = m.moe_zc_forward(inp["x"], inp["w_router"], inp["bias"], inp["w_gate"],
                                 inp["w_up"], inp["w_down"], w.N, w.Z, w.K, aux=aux)
        else:
            y = m.moe_zc_forward_packed(inp["x"], inp["w_router"], inp["bias"], packed[0],
                                        packed[1], w.N, w.Z, w.K, w.I, aux=aux)
        torch.cuda.synchronize()
        outs[kind] = (y, aux)
    assert torch.equal(outs["plain"][0], outs["packed"][0]), "saving a | u changed y"
    assert torch.equal(outs["rowmajor"][0], outs["packed"][0])
    S = int(outs["packed"][1]["offsets"][w.N].item())
    act_p = outs["packed"][1]["act"][:S]
    assert torch.equal(act_p, outs["rowmajor"][1]["act"][:S]), "row-major and packed a | u differ"
    ref = _act_reference(w, inp, outs["packed"][1])
    err = np.abs(act_p.float().cpu().double().numpy() - ref).max()
    assert err <= 1e-2 * np.abs(ref).max(), f"a | u off by {err}"
    if w.d % 128 == 0:
        fp8w = m.moe_zc_pack_expert_weights_fp8(inp["w_gate"], inp["w_up"])
        y_plain = m.moe_zc_forward_packed_fp8(inp["x"], inp["w_router"], inp["bias"], fp8w,
                                              packed[1], w.N, w.Z, w.K, w.I)
        aux = m.alloc_aux(w.T, w.N, w.Z, w.K, DEV, keys=keys, I=w.I)
        y8 = m.moe_zc_forward_packed_fp8(inp["x"], inp["w_router"], inp["bias"], fp8w, packed[1],
                                         w.N, w.Z, w.K, w.I, aux=aux)
        torch.cuda.synchronize()
        assert torch.equal(y8, y_plain), "saving a | u changed the FP8 forward's y"
        ref8 = _act_reference(w, inp, aux, fp8=True)
        err8 = np.abs(aux["act"][:S].float().cpu().double().numpy() - ref8).max()
        assert err8 <= 1e-2 * np.abs(ref8).max(), f"FP8 a | u off by {err8}"


def gpu_forward_backward_saved(w, inp, dy):
    """Packed forward saving a | u, then the backward without the row-major
    gate / up weights."""
    keys = m.AUX_KEYS + ("act",)
    aux = m.alloc_aux(w.T, w.N, w.Z, w.K, DEV, keys=keys, I=w.I)
    tr = None
    gu = dn = None
    if w.N > 0:
        gu, dn = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
        tr = m.moe_zc_transpose_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    m.moe_zc_forward_packed(inp["x"], inp["w_router"], inp["bias"], gu, dn, w.N, w.Z, w.K, w.I,
                            aux=aux)
    g = m.moe_zc_backward(inp["x"], inp["w_router"], None, None, tr, aux, dy, w.N, w.Z, w.K, w.I)
    torch.cuda.synchronize()
    return aux, g


@pytest.mark.parametrize("name", ["T1", "T65_ragged", "Z0", "N0_all_identity",
                                  "few_rows_32_tiles", "rows_256_tiles", "wide_d",
                                  "many_experts", "rows_past_256"])
def test_backward_from_saved_preactivations(name):
    w = _edge(**CASES[name])
    print(f"[backward saved {name}] {w.describe()}", flush=True)
    inp = make_inputs(w, device=DEV)
    dy = make_upstream_grad(w, DEV)
    aux, g = gpu_forward_backward_saved(w, inp, dy)
    print(name, compare(w, inp, dy, aux, g), flush=True)


def test_backward_from_saved_preactivations_mid():
    w = get_workload("mid")
    inp = make_inputs(w, device=DEV)
    dy = make_upstream_grad(w, DEV)
    aux, g = gpu_forward_backward_saved(w, inp, dy)
    print("mid saved", compare(w, inp, dy, aux, g), flush=True)
