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


def test_backward_subsets_equal_the_full_backward():
    """The subset options that full-size GPU tests use: dx of a token sample
    (want_dx only, no weight gradients) and one expert's weight gradients
    from exactly the tokens routed to it equal the full call's values."""
    from oracle import backward as obw, moe_zc as layer
    rng = np.random.default_rng(22)
    T, d, I, N, Z, K = 60, 32, 24, 7, 3, 3
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((N + Z, d)) / d ** 0.5
    wg, wu = (rng.standard_normal((N, I, d)) / d ** 0.5 for _ in range(2))
    wd = rng.standard_normal((N, d, I)) / I ** 0.5
    dy = rng.standard_normal((T, d))
    b = rng.uniform(-0.05, 0.05, N + Z)
    lg = layer.router_logits(x, wr).astype(np.float32)
    full = obw.backward(x, wr, b, wg, wu, wd, N, Z, K, dy, logits32=lg)
    s = np.array([3, 17, 18, 41, 59])
    sub = obw.backward(x[s], wr, b, wg, wu, wd, N, Z, K, dy[s], logits32=lg[s], experts=[])
    np.testing.assert_allclose(sub["dx"], full["dx"][s], rtol=1e-12, atol=1e-12)
    assert sub["dw_gate"] == {}
    idx = full["route"]["idx"]
    for e in (0, 4):
        tt = np.nonzero((idx == e).any(axis=1))[0]
        assert len(tt) > 0
        one = obw.backward(x[tt], wr, b, wg, wu, wd, N, Z, K, dy[tt], logits32=lg[tt],
                           experts=[e], want_dx=False)
        assert "dx" not in one and sorted(one["dw_gate"]) == [e]
        for k in ("dw_gate", "dw_up", "dw_down"):
            np.testing.assert_allclose(one[k][e], full[k][e], rtol=1e-12, atol=1e-12)
