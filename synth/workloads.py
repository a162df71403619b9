"""Workload shapes and input recipes for the BitLinear projection.

A projection maps d_in = K channels to d_out = N channels (W is [N][K]); a
call carries M tokens (X is [M][K]).  Standard deviations are stated as
sigma; seeds default to 0.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from fractions import Fraction

import numpy as np

from .generators import make_acts, make_weight


@dataclass(frozen=True)
class Projection:
    name: str
    K: int  # d_in
    N: int  # d_out


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    projections: tuple
    tokens: tuple           # the M values exercised
    w_sigma: float
    x_recipe: dict = field(default_factory=dict)
    out_dtype: str = "bf16"  # "f32" or "bf16"
    seed: int = 0
    shared_input: bool = False   # every projection reads the same X (q/k/v, gate/up)

    def weight(self, proj: Projection) -> np.ndarray:
        return make_weight(self.seed, f"{self.name}/{proj.name}/W", proj.N, proj.K,
                           self.w_sigma)

    def acts(self, proj: Projection, M: int) -> np.ndarray:
        tag = "shared" if self.shared_input else proj.name
        return make_acts(self.seed, f"{self.name}/{tag}/X/M{M}", M, proj.K, self.x_recipe)


WORKLOADS = {
    w.name: w
    for w in (
        Workload(
            name="layer-512x256",
            description="single BitLinear layer 512->256, 4 tokens, 1% channels x50, fp32 out",
            projections=(Projection("proj", 512, 256),),
            tokens=(4,),
            w_sigma=0.02,
            x_recipe={"outlier_frac": Fraction(1, 100), "outlier_scale": 50.0},
            out_dtype="f32",
        ),
        Workload(
            name="decode-3b",
            description="one-token decode, 3B FFN: 3200->8640 (up) and 8640->3200 (down), bf16 out",
            projections=(Projection("ffn_up", 3200, 8640), Projection("ffn_down", 8640, 3200)),
            tokens=(1,),
            w_sigma=0.02,
        ),
        Workload(
            name="decode-7b",
            description="batched decode, 7B: 4096->11008, 11008->4096, 4096->4096; "
                        "M in {1,8,32,64}; 0.5% channels x100; bf16 out",
            projections=(Projection("ffn_up", 4096, 11008), Projection("ffn_down", 11008, 4096),
                         Projection("attn", 4096, 4096)),
            tokens=(1, 8, 32, 64),
            w_sigma=0.02,
            x_recipe={"outlier_frac": Fraction(1, 200), "outlier_scale": 100.0},
        ),
        Workload(
            name="attn-qkv-7b",
            description="query, key and value projections of one 7B attention block, 3 x "
                        "(4096->4096) reading the same X; M in {1,8,16}; 0.5% channels x100; "
                        "bf16 out",
            projections=(Projection("q", 4096, 4096), Projection("k", 4096, 4096),
                         Projection("v", 4096, 4096)),
            tokens=(1, 8, 16),
            w_sigma=0.02,
            x_recipe={"outlier_frac": Fraction(1, 200), "outlier_scale": 100.0},
            shared_input=True,
        ),
        Workload(
            name="prefill-7b",
            description="prefill, 7B FFN up 4096->11008, M=2048; 1% channels Student-t(3); bf16 out",
            projections=(Projection("ffn_up", 4096, 11008),),
            tokens=(2048,),
            w_sigma=0.02,
            x_recipe={"t3_frac": Fraction(1, 100)},
        ),
        Workload(
            name="ffn-70b",
            description="70B FFN: 8192->28672 and 28672->8192; M in {1,16} decode, 1024 prefill; "
                        "W sigma 0.015; bf16 out",
            projections=(Projection("ffn_up", 8192, 28672), Projection("ffn_down", 28672, 8192)),
            tokens=(1, 16, 1024),
            w_sigma=0.015,
        ),
    )
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]
