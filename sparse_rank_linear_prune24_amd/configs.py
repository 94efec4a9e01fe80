"""Workload registry: the five synthetic layer sets the kernels are tested and timed on.

The shapes stand in for the Llama-3-8B layers that the HASSLE-free page ("HASSLE-free: A unified
Framework for Sparse plus Low-Rank Matrix Decomposition for LLMs", abstract and §1) and the 3BASiL
article ("Can sparse plus low-rank decomposition compress large language models without
performance loss?") compress at 2:4 sparsity plus a rank-64 component. The pages print no layer
widths; the widths below are Llama-3-8B's (hidden 4096, 8 KV heads of 128 -> 1024, MLP 14336).
The token count 2048 of the prefill workload equals one calibration segment (HASSLE-free §5.1).

A layer is (name, n_in, n_out): W is [n_out x n_in], S is 2:4 along n_in, U is [n_out x r],
V is [r x n_in], X is [M x n_in] and Y = X S^T + (X V^T) U^T is [M x n_out].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple


@dataclass(frozen=True)
class Config:
    name: str
    config_id: int          # enters every seed of this workload
    dtype: str              # "fp32" or "bf16": storage/arithmetic type of X, S, U, V
    M: int                  # tokens
    r: int                  # rank of the thin factors
    layers: Tuple[Tuple[str, int, int], ...]   # (name, n_in, n_out)
    n_outliers: int         # whole input columns of X scaled by `outlier_scale`
    outlier_scale: float = 20.0
    w_std: float = 0.02
    # workload whose W/U/V this one reuses bit-for-bit (only X differs)
    weights_from: Optional[str] = None
    description: str = ""

    @property
    def uv_std(self) -> float:
        # U, V ~ N(0, 0.02^2 / r): the product U V then has entry variance 0.02^4 / r
        return self.w_std / math.sqrt(self.r) if self.r > 0 else 0.0

    def dense_equiv_flop(self) -> int:
        """2*M*n_out*n_in summed over layers: the FLOP of the dense layer Y = X W^T."""
        return sum(2 * self.M * n_out * n_in for _, n_in, n_out in self.layers)


CONFIGS = {
    "C1": Config("C1", 1, "fp32", 32, 16, (("linear", 512, 512),), 0,
                 description="single fp32 linear 512->512, 32 tokens, rank 16"),
    "C2": Config("C2", 2, "bf16", 2048, 64, (("q_proj", 4096, 4096),), 8,
                 description="Llama-3-8B q_proj prefill, 2048 tokens, rank 64, bf16"),
    "C3": Config("C3", 3, "bf16", 16, 64, (("q_proj", 4096, 4096),), 8, weights_from="C2",
                 description="decode: 16 tokens through the C2 layer"),
    "C4": Config("C4", 4, "bf16", 4096, 64,
                 (("gate_proj", 4096, 14336), ("up_proj", 4096, 14336), ("down_proj", 14336, 4096)), 8,
                 description="Llama-3-8B MLP, 4096 tokens, rank 64"),
    "C5": Config("C5", 5, "bf16", 8192, 128,
                 (("q_proj", 4096, 4096), ("k_proj", 4096, 1024), ("v_proj", 4096, 1024),
                  ("o_proj", 4096, 4096), ("gate_proj", 4096, 14336), ("up_proj", 4096, 14336),
                  ("down_proj", 14336, 4096)), 8,
                 description="full Llama-3-8B block linear set, 8192 tokens, rank 128"),
}


def get(name: str) -> Config:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}") from None
