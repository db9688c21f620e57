"""moe_zc_forward_packed_noalloc (the packed forward on the library's fixed
per-GPU scratch, for callers that cannot allocate) against
moe_zc_forward_packed: bitwise equal outputs and aux on two calls in a row,
the second with fewer tokens (the scratch keeps the first call's contents),
and a refusal of sizes whose workspace exceeds the scratch.  Called through
the C ABI via the Python binding."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_bias_amd as m
from workloads import get_workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _pair(w, inp, packed, T):
    x, res = inp["x"][:T].contiguous(), inp["residual"][:T].contiguous()
    keys = m.AUX_KEYS
    a1 = m.alloc_aux(T, w.N, w.Z, w.K, DEV, keys=keys)
    a2 = m.alloc_aux(T, w.N, w.Z, w.K, DEV, keys=keys)
    y1 = m.moe_zc_forward_packed(x, inp["w_router"], inp["bias"], packed[0], packed[1], w.N,
                                 w.Z, w.K, w.I, residual=res, aux=a1)
    y2 = torch.empty_like(y1)
    m.moe_zc_forward_packed_noalloc(x, inp["w_router"], inp["bias"], packed[0], packed[1], w.N,
                                    w.Z, w.K, w.I, residual=res, out=y2, aux=a2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2), f"T={T}: y differs"
    S = int(a1["offsets"][w.N])
    for k in keys:
        got, want = a2[k], a1[k]
        if k == "perm":                      # only the first S entries are defined
            got, want = got[:S], want[:S]
        assert torch.equal(got, want), f"T={T}: aux {k} differs"
    return S


@pytest.mark.parametrize("name,T1,T2", [("decode", 128, 37), ("mid", 512, 100)])
def test_noalloc_equals_workspace_forward(name, T1, T2):
    w = get_workload(name)
    print(f"[noalloc {name}] T={T1} then T={T2}", flush=True)
    inp = make_inputs(w.with_tokens(T1), device=DEV)
    packed = m.moe_zc_pack_expert_weights(inp["w_gate"], inp["w_up"], inp["w_down"])
    _pair(w, inp, packed, T1)
    _pair(w, inp, packed, T2)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    w = get_workload("decode")
    T = 256                                 # workspace about 73 MiB > 64 MiB
    assert m.moe_zc_workspace_size(T, w.d, w.I, w.N, w.Z, w.K, torch.bfloat16) > \
        m._lib.MOE_ZC_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(T, w.d, dtype=torch.bfloat16, device=DEV)
    wr = torch.zeros(w.E, w.d, device=DEV)
    b = torch.zeros(w.E, device=DEV)
    gu, dn = m.moe_zc_packed_expert_bytes(w.d, w.I)
    # the weights are never read: the call is refused on the host
    fake = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        m.moe_zc_forward_packed_noalloc(x, wr, b, fake, fake, w.N, w.Z, w.K, w.I)
    lib = m._lib.load()
    y = torch.empty_like(x)
    code = lib.moe_zc_forward_packed_noalloc(
        x.data_ptr(), wr.data_ptr(), b.data_ptr(), fake.data_ptr(), fake.data_ptr(), None,
        y.data_ptr(), T, w.d, w.I, w.N, w.Z, w.K, m._lib.MOE_ZC_BF16, None, None)
    assert code == m._lib.MOE_ZC_ERR_WORKSPACE
