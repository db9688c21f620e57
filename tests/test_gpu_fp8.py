"""Block-FP8 gate/up projection (moe_zc_quantize_mx, moe_zc_pack_expert_weights_fp8,
moe_zc_forward_packed_fp8) against the oracle.

Codes and scales are integer results of the quantization rule and must equal
the oracle's bit for bit.  The packed weight bytes are checked against a NumPy
statement of the layout (the kernel source defines it: 33 KB blocks per
(expert, 128-unit panel, 128-k stage), 32 KB of codes in four 8 KB quarters of
eight 1 KB pieces, then 1 KB of scales; a 32-code scale block is split 16/16
between lanes r and r + 32, as the matrix cores read it).  The forward is compared with the
oracle's layer whose gate/up projection uses the dequantized FP8 operands; its
routing equals the bf16 forward's (the router is not quantized)."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_bias_amd as m
from gpu_check import check_forward, run_gpu
from oracle import mx as omx
from workloads import Workload, get_workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _bf16_blocks(rows, d, seed):
    """bf16 rows whose 32-blocks span many binades, with zero blocks, blocks
    whose maximum sits exactly on a range edge (448 * 2^s and just above
    1.75 * 2^E), bf16 subnormals, and signed zeros."""
    r = np.random.default_rng(seed)
    v = r.standard_normal((rows, d // 32, 32)) * np.ldexp(1.0, r.integers(-60, 60, (rows, d // 32, 1)))
    v[0, 0] = 0.0
    v[0, 1] = -0.0
    v[1, :3] = r.uniform(-1.0, 1.0, (3, 32))        # small blocks whose maxima are set below
    v[1, 0, 3] = 448.0 * 2.0 ** 5
    v[1, 1, 7] = 1.75 * 2.0 ** 3
    v[1, 2, 9] = 1.7578125 * 2.0 ** 3               # mantissa just above 1.75 in bf16
    v[2, 0] = r.standard_normal(32) * 2.0 ** -130   # bf16 subnormals
    v[2, 1, :16] = -0.0
    t = torch.from_numpy(v.reshape(rows, d)).float().to(torch.bfloat16)
    return t


def test_quantize_mx_matches_oracle():
    x = _bf16_blocks(300, 512, seed=1)
    codes, scales = m.moe_zc_quantize_mx(x.to(DEV))
    torch.cuda.synchronize()
    ref_c, ref_s = omx.mx_quantize(x.float().double().numpy(), axis=-1)
    assert np.array_equal(scales.cpu().numpy(), ref_s), "scales"
    assert np.array_equal(codes.cpu().numpy(), ref_c), "codes"


def pack_fp8_reference(wg, wu):
    """[n, I, d] bf16 gate and up -> packed FP8 bytes [n, panels * stages * 33792]."""
    n, I, d = wg.shape
    P, S = I // 128, d // 128
    out = np.zeros((n, P, S, 33792), np.uint8)
    quant = []
    for wt in (wg, wu):
        c, s = omx.mx_quantize(wt.float().double().numpy(), axis=-1)
        quant.append((c.reshape(n, P, 128, S, 4, 32), s.reshape(n, P, 128, S, 4)))
    for w in range(4):
        for j in range(2):
            c8, s8 = quant[j]
            for cc in range(32):
                for kb in range(4):
                    ks, half = kb >> 1, kb & 1
                    q = 4 * ks + 2 * j + half
                    blk = c8[:, :, 32 * w + cc, :, kb, :]            # [n, P, S, 32]
                    for h in range(2):                              # lanes cc, cc + 32
                        o = w * 8192 + q * 1024 + (cc + 32 * h) * 16
                        out[..., o:o + 16] = blk[..., 16 * h:16 * h + 16]
                    lane_s = cc + 32 * half
                    out[..., 32768 + w * 256 + lane_s * 4 + 2 * ks + j] = s8[:, :, 32 * w + cc, :, kb]
    return out.reshape(n, -1)


@pytest.mark.parametrize("n,d,I", [(3, 256, 256), (2, 384, 128), (1, 128, 384)])
def test_pack_fp8_layout_matches_definition(n, d, I):
    g = torch.Generator().manual_seed(n * 1000 + d + I)
    wg = (torch.randn(n, I, d, generator=g) * 0.05).to(torch.bfloat16)
    wu = (torch.randn(n, I, d, generator=g) * 0.05).to(torch.bfloat16)
    wu[0, 5, 32:64] = 0.0                                 # an all-zero block
    packed = m.moe_zc_pack_expert_weights_fp8(wg.to(DEV), wu.to(DEV))
    torch.cuda.synchronize()
    assert packed.numel() == n * m.moe_zc_packed_fp8_expert_bytes(d, I)
    got = packed.cpu().numpy().reshape(n, -1)
    assert np.array_equal(got, pack_fp8_reference(wg, wu))


def _edge(T=200, d=128, I=128, N=8, Z=4, K=3, seed=3, bias=("uniform", 0.05)):
    return Workload("edge", T=T, d=d, I=I, N=N, Z=Z, K=K, dtype="bf16", seed=seed, bias=bias)


CASES = {
    "T1": dict(T=1),
    "T65_ragged": dict(T=65),
    "Z0": dict(N=8, Z=0, K=2),
    "K_eq_E": dict(N=5, Z=3, K=8),
    "N0_all_identity": dict(N=0, Z=6, K=3),
    "few_rows_32_tiles": dict(T=64, N=64, Z=32, K=8),
    "rows_128_tiles": dict(T=512, N=24, Z=8, K=6),
    "rows_256_tiles_split": dict(T=1100, N=8, Z=4, K=3, d=256, I=256),
    "stages_10": dict(T=257, d=1280, I=256, N=4, Z=4, K=2),     # 10 k-stages: 1 after the loop
    "stages_11": dict(T=300, d=1408, I=384, N=6, Z=2, K=2),     # 11 k-stages: 2 after the loop
}


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_forward_vs_oracle(name):
    w = _edge(**CASES[name])
    print(f"[fp8 {name}] {w.describe()}", flush=True)
    inp = make_inputs(w, device=DEV)
    packed = fp8 = None
    if w.N > 0:
        packed = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
        fp8 = (m.moe_zc_pack_expert_weights_fp8(inp["w_gate"], inp["w_up"]), packed[1])
    g_bf = run_gpu(w, inp, packed=packed)
    g_8 = run_gpu(w, inp, packed=fp8, fp8=True)
    for k in m.AUX_KEYS:                       # the router and the grouping are unquantized
        assert np.array_equal(g_bf[k], g_8[k]), k
    rep = check_forward(w, inp, g_8, fp8=True)
    scale = np.abs(g_bf["y"]).max()
    print(name, rep, "fp8 vs bf16 max|dy| / max|y|:",
          float(np.abs(g_8["y"] - g_bf["y"]).max() / max(scale, 1e-30)), flush=True)


def test_fp8_mid_vs_oracle():
    w = get_workload("mid")
    inp = make_inputs(w, device=DEV)
    packed = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    fp8 = (m.moe_zc_pack_expert_weights_fp8(inp["w_gate"], inp["w_up"]), packed[1])
    g = run_gpu(w, inp, packed=fp8, fp8=True)
    sample = np.sort(np.random.default_rng(0).choice(w.T, 384, replace=False))
    print("mid fp8", check_forward(w, inp, g, y_tokens=sample, fp8=True), flush=True)


def test_fp8_rejects_unsupported_shapes():
    w = _edge(d=192)                           # d not a multiple of 128
    inp = make_inputs(w, device=DEV)
    with pytest.raises(m.MoeZcError):
        m.moe_zc_packed_fp8_expert_bytes(192, 128)
    with pytest.raises(m.MoeZcError):
        m.moe_zc_forward_packed_fp8(inp["x"], inp["w_router"], inp["bias"], None, None, 0,
                                    w.N + w.Z, w.K, w.I)


def test_fp8_full_size_prefill():
    """The block-FP8 forward that `bench.py --precision fp8` times, at the
    prefill size: routing and grouping for every token (equal to the bf16
    path's, the router is not quantized), and the layer output on a token
    sample against the oracle's layer on dequantized FP8 operands (tokens are
    independent, so a sample is exact)."""
    from gpu_check import gpu_expert_getter
    w = get_workload("prefill")
    print("[fp8 prefill] generating inputs", flush=True)
    inp = make_inputs(w, device=DEV)
    gu8 = m.moe_zc_pack_expert_weights_fp8(inp["w_gate"], inp["w_up"])
    dn = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])[1]
    g = run_gpu(w, inp, packed=(gu8, dn), fp8=True)
    del gu8, dn
    sample = np.sort(np.random.default_rng(4).choice(w.T, 6, replace=False))
    print(f"[fp8 prefill] checking tokens {sample.tolist()}", flush=True)
    print("prefill fp8", check_forward(w, inp, g, y_tokens=sample, fp8=True,
                                       get_expert=gpu_expert_getter(inp)), flush=True)
