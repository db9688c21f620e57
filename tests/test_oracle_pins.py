"""The fp64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check()


def test_backward_accepts_torch_bf16_inputs():
    """The GPU tests hand the oracle torch bf16 tensors; the result must equal
    the call on the same values as fp64 NumPy arrays."""
    import torch
    from oracle import backward as obw
    g = torch.Generator().manual_seed(21)
    T, d, I, N, Z, K = 9, 64, 16, 3, 2, 2
    x = torch.randn(T, d, generator=g).to(torch.bfloat16)
    wr = torch.randn(N + Z, d, generator=g) / 8
    wg, wu = (torch.randn(N, I, d, generator=g).div(8).to(torch.bfloat16) for _ in range(2))
    wd = torch.randn(N, d, I, generator=g).div(4).to(torch.bfloat16)
    dy = torch.randn(T, d, generator=g).to(torch.bfloat16)
    b = np.zeros(N + Z)
    a = obw.backward(x, wr, b, wg, wu, wd, N, Z, K, dy)
    f = lambda t: t.double().numpy()
    n = obw.backward(f(x), f(wr), b, f(wg), f(wu), f(wd), N, Z, K, f(dy))
    for k in ("dx", "dw_router", "dw_gate", "dw_up", "dw_down"):
        assert np.array_equal(a[k], n[k]), k
