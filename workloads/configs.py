"""The five synthetic layer configurations and their input recipes.

Shapes follow the LongCat-Flash description (a pool of N FFN experts extended
by Z zero-computation experts, K experts chosen per token; page
『衝上熱搜！美團大模型，靠「快」火了』, section 零計算專家).  The expert FFN is
SwiGLU.  Every distribution below is a choice of this project, written out so
that a reader can regenerate the inputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    T: int              # tokens
    d: int              # model width
    I: int              # SwiGLU intermediate width of one FFN expert
    N: int              # FFN experts
    Z: int              # zero-computation (identity) experts
    K: int              # experts chosen per token
    dtype: str          # "f32" or "bf16": x, FFN weights, residual and y
    seed: int = 0
    # bias recipe: ("uniform", a) -> U(-a, a) on every expert;
    #              ("zero",)       -> all zeros
    bias: Tuple = ("zero",)
    # Zipf logit offsets over FFN experts: (s, c).  Implemented as an input
    # construction only: x[:, d-1] := 1 and W_router[i, d-1] := -s*ln(r_i) + c
    # for FFN expert i with seeded rank r_i in 1..N, 0 for zero experts.
    zipf: Optional[Tuple[float, float]] = None
    note: str = ""

    @property
    def E(self) -> int:
        return self.N + self.Z

    @property
    def expected_ffn_slots(self) -> float:
        """T*K*N/E: FFN slots expected under exchangeable routing."""
        return self.T * self.K * self.N / self.E

    def with_tokens(self, T: int) -> "Workload":
        return Workload(self.name, T, self.d, self.I, self.N, self.Z, self.K,
                        self.dtype, self.seed, self.bias, self.zipf, self.note)

    def describe(self) -> dict:
        return {"workload": self.name, "T": self.T, "d": self.d, "I": self.I,
                "N": self.N, "Z": self.Z, "K": self.K, "dtype": self.dtype,
                "seed": self.seed}


# Zipf constant c for the skewed workload.  It shifts every FFN expert's logit
# so that, with zero bias, about 8 of the 12 chosen experts per token are FFN
# experts (the activated-expert count the LongCat pages describe).  The value
# is produced by tests/golden/tune_skew_offset.py, which bisects c with the
# fp64 oracle's routing on the CPU-generated router inputs of this workload.
SKEW_ZIPF_C = 3.7617

WORKLOADS = {
    "tiny": Workload("tiny", T=64, d=128, I=256, N=8, Z=4, K=3, dtype="f32",
                     bias=("uniform", 0.1),
                     note="tiny fp32 layer"),
    "mid": Workload("mid", T=4096, d=2048, I=1024, N=64, Z=32, K=8,
                    dtype="bf16", bias=("uniform", 0.05),
                    note="mid bf16 layer"),
    "decode": Workload("decode", T=128, d=6144, I=2048, N=512, Z=256, K=12,
                       dtype="bf16", bias=("zero",),
                       note="decode-shaped, weight-bandwidth bound"),
    "prefill": Workload("prefill", T=16384, d=6144, I=2048, N=512, Z=256,
                        K=12, dtype="bf16", bias=("zero",),
                        note="prefill-shaped; zero bias gives K*N/E = 8 FFN "
                             "experts per token by symmetry"),
    "skew": Workload("skew", T=8192, d=4096, I=1536, N=256, Z=128, K=12,
                     dtype="bf16", bias=("zero",), zipf=(1.1, SKEW_ZIPF_C),
                     note="Zipf(1.1) logit offsets over FFN experts, then one "
                          "bias update toward uniform load"),
}


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; have {sorted(WORKLOADS)}")
