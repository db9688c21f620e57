"""Workload recipes checked with the oracle on the CPU (router side only)."""
import numpy as np

from oracle import moe_zc as om
from workloads import get_workload
from workloads.gen import make_router_inputs


def _route(w, bias=None):
    x, wr, b = make_router_inputs(w)
    l32 = om.router_logits(x, wr).astype(np.float32)
    return l32, (b.numpy() if bias is None else bias)


def test_skew_offsets_give_eight_ffn_experts_and_pid_rebalances():
    w = get_workload("skew")
    l32, b = _route(w)
    rt = om.route(l32, b, w.K, w.N)
    c = om.ffn_count_per_token(rt["idx"], w.N)
    assert 7.9 <= c.mean() <= 8.1, c.mean()
    loads = rt["loads"].astype(np.float64)
    before = loads[: w.N].max() / loads[: w.N].mean()
    assert before > 10.0                      # a hot Zipf expert exists
    target = np.full(w.E, w.T * w.K / w.E)
    nb, _, _ = om.pid_step(loads, target, b, np.zeros(w.E), np.zeros(w.E), 0.5, 0.5, 0.0)
    rt2 = om.route(l32, nb.astype(np.float32), w.K, w.N)
    l2 = rt2["loads"].astype(np.float64)
    after = l2[: w.N].max() / l2[: w.N].mean()
    # busy experts lose load, the imbalance and the distance to target shrink
    hot = int(np.argmax(loads[: w.N]))
    assert l2[hot] < loads[hot]
    assert after < before, (before, after)
    assert np.abs(l2 - target).sum() < np.abs(loads - target).sum()


def test_prefill_zero_bias_gives_eight_ffn_experts():
    w = get_workload("prefill").with_tokens(2048)
    l32, b = _route(w)
    rt = om.route(l32, b, w.K, w.N)
    c = om.ffn_count_per_token(rt["idx"], w.N)
    assert 7.8 <= c.mean() <= 8.2, c.mean()


def test_tiny_and_mid_inputs_are_deterministic():
    for name in ("tiny", "mid"):
        w = get_workload(name).with_tokens(32)
        a = make_router_inputs(w)
        b = make_router_inputs(w)
        for u, v in zip(a, b):
            assert u.dtype == v.dtype and bool((u == v).all())
