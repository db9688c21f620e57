"""Seeded tensor generation for the workloads in configs.py.

Recipe (all draws in fp32, then rounded to the workload dtype with
round-to-nearest-even by torch's ``.to``):
  x          N(0, 1)                       [T, d]   generated on the CPU
  W_router   N(0, 1/d)  (std d**-0.5)      [E, d]   fp32, generated on the CPU
  bias       per the workload recipe       [E]      fp32, generated on the CPU
  residual   N(0, 1)                       [T, d]   generated on the CPU
  dy         N(0, 1)                       [T, d]   upstream gradient of the
                                                    backward, on the CPU
  W_gate     N(0, 1/d)                     [N, I, d]
  W_up       N(0, 1/d)                     [N, I, d]
  W_down     N(0, 1/d)                     [N, d, I]
Each FFN expert e draws its three matrices from a generator of its own
(``expert_seed``), so any single expert can be regenerated alone.  FFN weights
are drawn on ``ffn_device``: the CPU for the tiny and mid workloads, the GPU
for the larger ones (torch's CPU and GPU generators give different streams, so
a consumer on the other device receives copies, never a regeneration).

Nothing here evaluates the layer; only random tensors are produced.
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from .configs import Workload

_TAG_X, _TAG_WR, _TAG_BIAS, _TAG_RES, _TAG_ZIPF, _TAG_DY = 1, 2, 3, 4, 5, 6


def _seed(w: Workload, tag: int, sub: int = 0) -> int:
    return (w.seed * 1_000_003 + tag * 65_537 + sub * 7_919 + 12_345) % (2**63 - 1)


def expert_seed(w: Workload, e: int) -> int:
    return _seed(w, 16, e)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def torch_dtype(w: Workload) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[w.dtype]


def default_ffn_device(w: Workload, device) -> str:
    small = w.N * w.I * w.d * 3 <= 512 * 1024 * 1024
    return "cpu" if small else str(device)


def make_router_inputs(w: Workload):
    """x (fp32, before rounding), W_router (fp32) and bias (fp32), on the CPU."""
    dt = torch_dtype(w)
    x = torch.randn(w.T, w.d, generator=_gen(_seed(w, _TAG_X), "cpu"))
    wr = torch.randn(w.E, w.d, generator=_gen(_seed(w, _TAG_WR), "cpu"))
    wr *= 1.0 / math.sqrt(w.d)
    kind = w.bias[0]
    if kind == "uniform":
        a = float(w.bias[1])
        u = torch.rand(w.E, generator=_gen(_seed(w, _TAG_BIAS), "cpu"))
        bias = (u * 2.0 - 1.0) * a
    elif kind == "zero":
        bias = torch.zeros(w.E)
    else:
        raise ValueError(f"unknown bias recipe {w.bias!r}")
    if w.zipf is not None:
        s, c = w.zipf
        ranks = torch.randperm(w.N, generator=_gen(_seed(w, _TAG_ZIPF), "cpu")) + 1
        offs = torch.zeros(w.E)
        offs[: w.N] = -s * torch.log(ranks.double()).float() + c
        x[:, w.d - 1] = 1.0
        wr[:, w.d - 1] = offs
    return x.to(dt), wr.float().contiguous(), bias.float().contiguous()


def make_expert_weights(w: Workload, e: int, device="cpu"):
    """(W_gate[e] [I,d], W_up[e] [I,d], W_down[e] [d,I]) in the workload dtype."""
    dt = torch_dtype(w)
    g = _gen(expert_seed(w, e), device)
    std = 1.0 / math.sqrt(w.d)
    wg = (torch.randn(w.I, w.d, generator=g, device=device) * std).to(dt)
    wu = (torch.randn(w.I, w.d, generator=g, device=device) * std).to(dt)
    wd = (torch.randn(w.d, w.I, generator=g, device=device) * std).to(dt)
    return wg, wu, wd


def make_inputs(w: Workload, device="cpu", ffn_device: Optional[str] = None,
                residual: bool = True) -> dict:
    """All layer inputs, placed on ``device``."""
    dt = torch_dtype(w)
    if ffn_device is None:
        ffn_device = default_ffn_device(w, device)
    x, wr, bias = make_router_inputs(w)
    out = {"x": x.to(device), "w_router": wr.to(device), "bias": bias.to(device)}
    if residual:
        r = torch.randn(w.T, w.d, generator=_gen(_seed(w, _TAG_RES), "cpu"))
        out["residual"] = r.to(dt).to(device)
    else:
        out["residual"] = None
    wg = torch.empty(w.N, w.I, w.d, dtype=dt, device=device)
    wu = torch.empty(w.N, w.I, w.d, dtype=dt, device=device)
    wd = torch.empty(w.N, w.d, w.I, dtype=dt, device=device)
    for e in range(w.N):
        g_, u_, d_ = make_expert_weights(w, e, ffn_device)
        wg[e].copy_(g_)
        wu[e].copy_(u_)
        wd[e].copy_(d_)
    out.update(w_gate=wg, w_up=wu, w_down=wd)
    return out


def make_upstream_grad(w: Workload, device="cpu") -> torch.Tensor:
    """dy = dL/dy [T, d] for the backward, N(0, 1) in the workload dtype."""
    dy = torch.randn(w.T, w.d, generator=_gen(_seed(w, _TAG_DY), "cpu"))
    return dy.to(torch_dtype(w)).to(device)
