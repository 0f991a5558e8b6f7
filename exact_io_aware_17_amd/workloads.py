"""Seeded synthetic workloads for the attention library and its checks.

This module holds the five workload shapes, their seeded input generators and
the FLOP/byte accounting used for throughput. It contains none of the
attention arithmetic itself, so both the GPU path and the CPU oracle can be
fed from it without sharing any of their computation.

Recipe (one CPU ``torch.Generator`` per workload, seed 17000 + workload id):
  randn float32 [B, H, N, d] drawn in the order Q, K, V (then dO when the
  workload has a backward), then the per-workload multiplier on Q, then the
  cast to the workload dtype (round-to-nearest-even for bf16 and fp16), then per-batch
  key lengths when the workload is padded: [0, 1, then B-2 uniform draws on
  {0, ..., N}] from the same generator.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    id: int
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str              # "f32", "bf16" or "f16"
    causal: object  # False, True (key j visible iff j <= i) or "strict" (iff j < i)
    q_mult: float = 1.0     # Q is multiplied by this before the cast
    padded: bool = False    # per-batch key lengths are drawn
    backward: bool = False  # an upstream gradient dO is drawn too

    @property
    def scale(self) -> float:
        """The float32 value of 1/sqrt(d) that every path receives."""
        return float(torch.tensor(1.0 / math.sqrt(self.d), dtype=torch.float32).item())

    @property
    def seed(self) -> int:
        return 17000 + self.id

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[self.dtype]

    def describe(self) -> Dict:
        return {"workload": self.name, "B": self.B, "H": self.H, "N": self.N, "d": self.d,
                "dtype": self.dtype, "causal": self.causal, "q_mult": self.q_mult,
                "padded": self.padded}


WORKLOADS = [
    Workload(1, "single-head N=256 d=64 fp32 non-causal", 1, 1, 256, 64, "f32", False),
    Workload(2, "MHA fwd B=4 H=16 N=2048 d=64 bf16 non-causal", 4, 16, 2048, 64, "bf16", False),
    Workload(3, "causal MHA fwd large logits B=2 H=16 N=4096 d=64 bf16 Qx8", 2, 16, 4096, 64,
             "bf16", True, q_mult=8.0),
    Workload(4, "causal fwd key padding B=8 H=32 N=16384 d=128 bf16", 8, 32, 16384, 128,
             "bf16", True, padded=True),
    Workload(5, "causal fwd+bwd B=2 H=16 N=4096 d=128 bf16", 2, 16, 4096, 128, "bf16", True,
             backward=True),
]

BY_ID = {w.id: w for w in WORKLOADS}


def with_shape(w: Workload, **changes) -> Workload:
    """The same recipe at another shape (parity runs at reduced sizes)."""
    return dataclasses.replace(w, **changes)


def forward_name(w: Workload) -> str:
    """The workload's forward alone (what a forward throughput line measures)."""
    return w.name.replace("causal fwd+bwd", "causal fwd")


def make_inputs(w: Workload, seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Draw the workload's inputs on the CPU, following the recipe in the module doc.

    Returns CPU tensors: q, k, v (and do) in the workload dtype, and kv_lens
    (int32 [B]) when the workload is padded.
    """
    g = torch.Generator().manual_seed(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.d)
    out: Dict[str, torch.Tensor] = {}
    names = ["q", "k", "v"] + (["do"] if w.backward else [])
    for name in names:
        t = torch.randn(shape, generator=g, dtype=torch.float32)
        if name == "q" and w.q_mult != 1.0:
            t.mul_(w.q_mult)
        out[name] = t.to(w.torch_dtype)
        del t
    if w.padded:
        forced = [0, 1][: w.B]
        rest = torch.randint(0, w.N + 1, (max(0, w.B - len(forced)),), generator=g)
        out["kv_lens"] = torch.tensor(forced + rest.tolist(), dtype=torch.int32)
    return out


def fwd_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    """Forward FLOPs 4*B*H*N^2*d (two contractions of 2*N*N*d per head), halved for causal."""
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def bwd_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    """Backward FLOPs by the five-contraction convention 10*B*H*N^2*d, halved for causal."""
    f = 10.0 * B * H * N * N * d
    return f / 2 if causal else f


def fwd_bytes(B: int, H: int, N: int, d: int, elem_bytes: int) -> float:
    """Algorithmic HBM bytes of one forward: Q, K, V read once, O written once, lse (fp32)."""
    return float(B * H * N * (4 * d * elem_bytes + 4))


def score_matrix_bytes(N: int, elem_bytes: int = 4) -> int:
    """Bytes of one head's N x N score matrix (what the fused forward never stores)."""
    return N * N * elem_bytes


def quadratic_share(N: int, d: int) -> float:
    """Share N^2 / (N^2 + N d) of the naive path's traffic that is quadratic."""
    return N * N / (N * N + N * d)
