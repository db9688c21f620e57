"""Packed expert weights (moe_zc_pack_expert_weights + moe_zc_forward_packed).

The packed layout is checked byte for byte against a NumPy statement of its
definition (include/moe_zc.h leaves it opaque; the kernel source defines it:
32 KB blocks per (expert, 256-row panel, 64-k stage), four 8 KB quarters per
block, eight 1 KB pieces per quarter, 16 bytes per lane).  The packed forward
must equal the row-major forward bit for bit (same products, same
accumulation order), and both are compared with the oracle."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_bias_amd as m
from gpu_check import LOGIT_TOL, check_forward, run_gpu
from workloads import Workload, get_workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def pack_reference(w0, w1, swiglu):
    """[n, rows, K] row-major bf16 bits (w1: the up rows for SwiGLU) -> packed bytes."""
    n, rows, K = w0.shape
    panels = rows // 128 if swiglu else -(-rows // 256)
    nk = K // 64
    out = np.zeros((n, panels, nk, 4, 8, 64, 8), np.uint16)
    for nt in range(panels):
        for w in range(4):
            for ks in range(4):
                for j in range(2):
                    for lane in range(64):
                        c, k0 = lane % 32, 16 * ks + 8 * (lane // 32)
                        if swiglu:
                            src, r = (w1 if j else w0), nt * 128 + 32 * w + c
                        else:
                            src, r = w0, nt * 256 + 64 * w + 32 * j + c
                        if r < rows:
                            blk = src[:, r, :].reshape(n, nk, 64)
                            out[:, nt, :, w, 2 * ks + j, lane, :] = blk[:, :, k0:k0 + 8]
    return out.reshape(n, -1).view(np.uint8)


@pytest.mark.parametrize("n,d,I", [(3, 192, 256), (2, 320, 128), (1, 64, 384)])
def test_pack_layout_matches_definition(n, d, I):
    g = torch.Generator().manual_seed(n * 1000 + d + I)
    wg, wu = (torch.randn(n, I, d, generator=g).bfloat16() for _ in range(2))
    wd = torch.randn(n, d, I, generator=g).bfloat16()
    gu, dn = m.moe_zc_pack_expert_weights(wg.to(DEV), wu.to(DEV), wd.to(DEV))
    torch.cuda.synchronize()
    ref_gu = pack_reference(_u16(wg), _u16(wu), True)
    ref_dn = pack_reference(_u16(wd), None, False)
    assert np.array_equal(gu.cpu().numpy().reshape(n, -1), ref_gu)
    assert np.array_equal(dn.cpu().numpy().reshape(n, -1), ref_dn)


def test_pack_expert_by_expert_equals_pack_all():
    n, d, I = 4, 128, 256
    g = torch.Generator().manual_seed(5)
    wg, wu = (torch.randn(n, I, d, generator=g).bfloat16().to(DEV) for _ in range(2))
    wd = torch.randn(n, d, I, generator=g).bfloat16().to(DEV)
    gu, dn = m.moe_zc_pack_expert_weights(wg, wu, wd)
    bgu, bdn = m.moe_zc_packed_expert_bytes(d, I)
    gu2 = torch.empty_like(gu)
    dn2 = torch.empty_like(dn)
    for e in range(n):
        m.moe_zc_pack_expert_weights(wg[e:e + 1], wu[e:e + 1], wd[e:e + 1],
                                     gu2[e * bgu:(e + 1) * bgu], dn2[e * bdn:(e + 1) * bdn])
    torch.cuda.synchronize()
    assert torch.equal(gu, gu2) and torch.equal(dn, dn2)


def _edge(T=200, d=128, I=128, N=8, Z=4, K=3, seed=3, bias=("uniform", 0.05)):
    return Workload("edge", T=T, d=d, I=I, N=N, Z=Z, K=K, dtype="bf16", seed=seed, bias=bias)


CASES = {
    "T1": dict(T=1),
    "T65_ragged": dict(T=65),
    "Z0": dict(N=8, Z=0, K=2),
    "K_eq_E": dict(N=5, Z=3, K=8),
    "K1": dict(K=1),
    "N0_all_identity": dict(N=0, Z=6, K=3),
    "few_rows_32_tiles": dict(T=64, N=64, Z=32, K=8),
    "rows_128_tiles": dict(T=512, N=24, Z=8, K=6),
    "rows_256_tiles_split": dict(T=1100, N=8, Z=4, K=3, d=256, I=256),
    "d_not_panel_multiple": dict(T=300, d=192, I=256, N=6, Z=2, K=3),
    "many_experts_topk32": dict(T=96, N=1024, Z=1024, K=32, I=128),
    "long_k": dict(T=257, d=1024, I=512, N=4, Z=4, K=2),
    "odd_stage_counts": dict(T=200, d=1216, I=640, N=6, Z=2, K=2),   # 19 and 10 k-stages
    # experts just past one 256-row tile (257, 268, 289, 310 rows) and well past
    # it (373, 439): each runs as two row parts of whole 32-row blocks
    "rows_past_256": dict(T=1300, d=320, I=384, N=10, Z=4, K=3),
}


@pytest.mark.parametrize("name", list(CASES))
def test_packed_forward_equals_rowmajor_and_oracle(name):
    w = _edge(**CASES[name])
    print(f"[packed {name}] {w.describe()}", flush=True)
    inp = make_inputs(w, device=DEV)
    packed = None
    if w.N > 0:
        packed = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    g_row = run_gpu(w, inp)
    g_pk = run_gpu(w, inp, packed=packed)
    assert torch.equal(g_row["y_t"], g_pk["y_t"]), "packed forward differs from row-major"
    for k in m.AUX_KEYS:
        assert np.array_equal(g_row[k], g_pk[k]), k
    rep = check_forward(w, inp, g_pk)
    print(name, rep, flush=True)


def test_rows_past_256_case_holds_its_boundaries():
    """The rows_past_256 case holds experts of exactly 257 rows (the fewest
    that split) and 289 rows (ten 32-row blocks), a few of nine and of ten
    blocks, and one far past 320 rows."""
    w = _edge(**CASES["rows_past_256"])
    inp = make_inputs(w, device=DEV)
    loads = run_gpu(w, inp)["loads"][:w.N]
    assert 257 in loads and 289 in loads, sorted(loads)
    assert ((loads > 256) & (loads <= 288)).sum() >= 2 and ((loads > 288) & (loads <= 320)).sum() >= 2
    assert (loads > 320).sum() >= 1


def test_packed_mid_vs_oracle():
    w = get_workload("mid")
    inp = make_inputs(w, device=DEV)
    packed = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    g = run_gpu(w, inp, packed=packed)
    sample = np.sort(np.random.default_rng(0).choice(w.T, 384, replace=False))
    print("mid packed", check_forward(w, inp, g, y_tokens=sample), flush=True)


# The router is one group of T rows in 256 tiles of 32 * na rows (E <= 256:
# one weight panel) over 2 d / 64 k-stages.  The grouped GEMM runs its stages
# three at a time and the last one or two after the loop, so every remainder
# of the stage count by three is taken with several row-block counts.
@pytest.mark.parametrize("d", [1216, 1280, 1344])   # 38, 40, 42 router k-stages
@pytest.mark.parametrize("na", [1, 2, 3, 8])
def test_router_logits_stage_remainders(d, na):
    w = _edge(T=8192 * na, d=d, I=128, N=8, Z=4, K=2)
    print(f"[router tails] d={d} na={na} {w.describe()}", flush=True)
    inp = make_inputs(w, device=DEV)
    g = run_gpu(w, inp)
    x = inp["x"].float().cpu().double().numpy()
    ref = x @ inp["w_router"].cpu().double().numpy().T
    err = np.abs(g["logits"].astype(np.float64) - ref).max()
    assert err <= LOGIT_TOL, f"router logits off by {err}"


# Few tokens: the bf16 router splits its K range (2d in stages of 64) into
# equal parts whose partial logits the top-K stage sums in part order.  The
# cases give 1 (T=1, d=128: 4 stages), several and many parts (e.g. T=128 at
# d=6144, E=768: 12 row tiles, 16 parts of 12 stages).
@pytest.mark.parametrize("T,d,N,Z", [(1, 128, 8, 4), (40, 2048, 64, 32), (128, 6144, 512, 256),
                                     (300, 1344, 6, 2), (1000, 4096, 24, 8)])
def test_router_split_k(T, d, N, Z):
    w = _edge(T=T, d=d, I=128, N=N, Z=Z, K=min(12, N + Z))
    print(f"[router split] {w.describe()}", flush=True)
    inp = make_inputs(w, device=DEV)
    g1 = run_gpu(w, inp)
    g2 = run_gpu(w, inp)
    assert np.array_equal(g1["logits"].view(np.uint32), g2["logits"].view(np.uint32)), \
        "split router logits differ between runs"
    print(check_forward(w, inp, g1), flush=True)
