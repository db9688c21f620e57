"""fp64 CPU oracle for the MoE layer with zero-computation experts.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import or run anything in this package.  It shares no
code with the HIP library or its Python binding, and neither side imports the
other.  Seeded inputs come from the separate ``workloads`` package.

Sources (web pages about Meituan's LongCat-Flash; the formula that defines the
MoE module was an image and did not survive on the page that introduces it):
  * 『衝上熱搜！美團大模型，靠「快」火了』 (dhxrcw.cn), section 零計算專家:
    pool of N FFN experts extended by Z zero-computation experts that return
    their input unchanged; softmax router R; per-expert bias b_i; K experts per
    token; the bias adjusts routing scores from recent usage and is decoupled
    from the training objective; a PID controller tunes it.
  * 『美团的 LongCat-Flash：用 27B 激活算力跑起一个 560B 模型』 (aiai.cafe),
    section 关键要点: PID on the expert bias keeps mean activation near 27B.
  * 『美团 LongCat-Flash 这个5600亿参数的懒AI，竟然比勤奋的模型跑得更快？』
    (longshidata.com), section on the "lazy" experts: the controller takes load
    from busy experts and gives it to idle ones.
  * 『美团LongCat-Flash：算力调度新纪元』 (vpshk.cn), section 1 技术创新 and
    its Figure 3 caption: about 8 activated experts per token on average.

Pinned functions and their pins are listed in ``moe_zc.py``; the PID gains and
the convergence rate on a real model are parity unpinned (the pages give no
values).
"""
from .moe_zc import (  # noqa: F401
    router_logits, softmax_fp64, selection_keys, select_topk, gates_of,
    expert_loads, ffn_offsets, permutation, unpermute, silu, swiglu_ffn,
    combine, route, forward, forward_tokens, pid_step, ffn_count_per_token,
    budget_target, closed_loop,
)
from . import bruteforce  # noqa: F401
from . import mx  # noqa: F401
from . import backward  # noqa: F401
