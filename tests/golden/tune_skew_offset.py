"""Bisect the Zipf constant c of the skewed workload with the fp64 oracle.

The skewed workload shifts FFN expert i's logit by -1.1*ln(r_i) + c (r_i a
seeded rank).  With zero bias, c is chosen so that on average 8 of the K = 12
chosen experts are FFN experts, the activated-expert count the page
『美团LongCat-Flash：算力调度新纪元』 gives for its Figure 3 (about 8).
Routing uses only the oracle; the router inputs come from the seeded
generator.  Prints c; workloads/configs.py stores it as SKEW_ZIPF_C.

    python tests/golden/tune_skew_offset.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import moe_zc as om  # noqa: E402
from workloads import get_workload  # noqa: E402
from workloads.gen import make_router_inputs  # noqa: E402


def mean_ffn_per_token(c, base, offs_unit, N, K):
    l32 = (base + offs_unit + c * (np.arange(base.shape[1]) < N)).astype(np.float32)
    rt = om.route(l32, np.zeros(base.shape[1], np.float32), K, N)
    return om.ffn_count_per_token(rt["idx"], N).mean()


def main():
    w = get_workload("skew")
    x, wr, _ = make_router_inputs(w)
    x = x.double().numpy()
    wr = wr.double().numpy()
    # logits without the offset column, and the rank part of the offsets
    offs = wr[:, w.d - 1].copy()
    c_stored = w.zipf[1]
    unit = np.where(np.arange(w.E) < w.N, offs - c_stored, 0.0)
    base = om.router_logits(x[:, : w.d - 1], wr[:, : w.d - 1])
    lo, hi = 0.0, 10.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if mean_ffn_per_token(mid, base, unit[None, :], w.N, w.K) < 8.0:
            lo = mid
        else:
            hi = mid
    c = round(0.5 * (lo + hi), 4)
    print(f"c = {c}  mean FFN/token at c: "
          f"{mean_ffn_per_token(c, base, unit[None, :], w.N, w.K):.4f}")


if __name__ == "__main__":
    main()
