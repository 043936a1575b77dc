"""Seeded synthetic inputs for the attention forward pass.

This module only draws random numbers and names workload shapes; it holds none
of the attention arithmetic.  Both the HIP path and the fp64 oracle are fed
from it, with the same 16-bit bit patterns.

Recipe: a CPU ``torch.Generator`` seeded with ``seed`` draws
``randn((B,H,N,d), float32)`` for q, then k, then v (i.i.d. N(0,1)).  For the
"peaky" workload q and k are multiplied by ``qk_gain`` in fp32; each tensor is
then cast once, round-to-nearest-even, to the 16-bit dtype.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np
import torch

_TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f16" or "bf16"
    causal: bool
    qk_gain: float = 1.0
    note: str = ""
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def scale(self) -> float:
        """1/sqrt(d), as the fp32 value handed to the kernel."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def flops(self) -> float:
        """4*B*H*N^2*d, halved when causal (the metric's FLOP convention)."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five workloads of the forward-pass study, plus the ragged variant of the
# second one and non-causal long-sequence extras at d=128.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 256, 64, "f16", False,
                     note="B1 H2 N256 d64 fp16, non-causal"),
    "n1k": Workload("n1k", 4, 16, 1024, 128, "bf16", False,
                    note="B4 H16 N1024 d128 bf16, non-causal"),
    "n1000": Workload("n1000", 4, 16, 1000, 128, "bf16", False,
                      note="B4 H16 N1000 d128 bf16, non-causal (ragged tail)"),
    "n4k_causal": Workload("n4k_causal", 2, 16, 4096, 128, "bf16", True,
                           note="B2 H16 N4096 d128 bf16, causal"),
    "n8k_causal_peaky": Workload("n8k_causal_peaky", 1, 32, 8192, 128, "bf16", True,
                                 qk_gain=3.0,
                                 note="B1 H32 N8192 d128 bf16, causal, Q,K x3"),
    "n16k_d64": Workload("n16k_d64", 1, 4, 16384, 64, "f16", False,
                         note="B1 H4 N16384 d64 fp16, non-causal, few heads"),
    "n4k_full": Workload("n4k_full", 2, 16, 4096, 128, "bf16", False,
                         note="extra: B2 H16 N4096 d128 bf16, non-causal"),
    "n8k_full": Workload("n8k_full", 1, 32, 8192, 128, "bf16", False,
                         note="extra: B1 H32 N8192 d128 bf16, non-causal"),
    "n4k_h4_causal": Workload("n4k_h4_causal", 1, 4, 4096, 128, "bf16", True,
                              note="extra: B1 H4 N4096 d128 bf16, causal (64 Q blocks)"),
}


def make_qkv(B: int, H: int, N: int, d: int, dtype: str, seed: int = 0,
             qk_gain: float = 1.0):
    """Return CPU tensors (q, k, v) of shape [B,H,N,d] in ``dtype``."""
    if dtype not in _TORCH_DTYPES:
        raise ValueError(f"dtype must be one of {sorted(_TORCH_DTYPES)}")
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if qk_gain != 1.0:
        q.mul_(np.float32(qk_gain).item())
        k.mul_(np.float32(qk_gain).item())
    t = _TORCH_DTYPES[dtype]
    return q.to(t), k.to(t), v.to(t)


def varlen_offsets(n_seq: int, lo: int, hi: int, seed: int = 0):
    """Cumulative starts [0, L_0, L_0+L_1, ...] of n_seq packed sequences
    with lengths drawn uniformly from [lo, hi] by a seeded numpy generator."""
    lens = np.random.default_rng(seed).integers(lo, hi + 1, size=n_seq)
    return [0] + np.cumsum(lens).astype(int).tolist()


def make_workload(w: Workload, seed: int = 0):
    return make_qkv(w.B, w.H, w.N, w.d, w.dtype, seed=seed, qk_gain=w.qk_gain)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of a CPU fp16/bf16 tensor, as numpy.uint16."""
    if t.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("expected an fp16 or bf16 tensor")
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
