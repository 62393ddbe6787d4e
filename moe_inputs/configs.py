"""Workload shapes for the grouped expert MLP.

The layer shape is the Mixtral-8x7B expert MLP (hidden 4096, intermediate
14336, 8 experts, top-2 routing) named in the Mixtral-8x7B benchmark figure of
the "BioNeMo Uses Grouped Kernels and MXFP8" page (Figure 5) and in the
sparse-MoE diagram of the same page (Figure 1: top-2 of 8 experts).  The other
workloads are a tiny parity case, a skewed MXFP8 case, the backward pass and a
fine-grained 64-expert case.
"""
from dataclasses import dataclass, replace
from typing import Optional


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int            # tokens
    H: int            # hidden size (FC1 K, FC2 N)
    I: int            # intermediate size (FC1 N = 2*I, FC2 K)
    E: int            # local experts
    k: int            # experts per token
    precision: str    # "bf16" or "mxfp8": operand format of both grouped GEMMs
    x_dtype: str      # "f32" or "bf16": dtype of the layer input and output
    routing: str      # "normal": logits N(0,1); "zipf": popularity ~ rank^-s
    zipf_s: float = 0.0
    zero_expert: Optional[int] = None   # expert forced to receive no tokens
    backward: bool = False
    seed: int = 0

    @property
    def R(self) -> int:
        return self.T * self.k

    def fwd_flops(self) -> float:
        # FC1: 2*R*H*(2I); FC2: 2*R*I*H
        return 6.0 * self.R * self.H * self.I

    def bwd_flops(self) -> float:
        # dgrad + wgrad of both GEMMs
        return 12.0 * self.R * self.H * self.I

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


CONFIGS = {
    1: MoEConfig("tiny-fwd-f32io", T=256, H=128, I=256, E=4, k=2, precision="bf16",
                 x_dtype="f32", routing="normal", seed=1001),
    2: MoEConfig("mixtral8x7b-fwd-bf16", T=4096, H=4096, I=14336, E=8, k=2, precision="bf16",
                 x_dtype="bf16", routing="normal", seed=1002),
    3: MoEConfig("mixtral8x7b-fwd-mxfp8-zipf1.2", T=8192, H=4096, I=14336, E=8, k=2,
                 precision="mxfp8", x_dtype="bf16", routing="zipf", zipf_s=1.2, zero_expert=4,
                 seed=1003),
    4: MoEConfig("mixtral8x7b-bwd-bf16", T=8192, H=4096, I=14336, E=8, k=2, precision="bf16",
                 x_dtype="bf16", routing="normal", backward=True, seed=1004),
    5: MoEConfig("finegrained-e64-fwd-mxfp8-zipf1.0", T=16384, H=2048, I=1408, E=64, k=8,
                 precision="mxfp8", x_dtype="bf16", routing="zipf", zipf_s=1.0, seed=1005),
}


def get_config(i: int) -> MoEConfig:
    return CONFIGS[int(i)]
