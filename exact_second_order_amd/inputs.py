"""Seeded synthetic inputs for BoB workloads (shared by tests, smoke and bench).

This module only draws random numbers and casts them; it holds none of the
method's arithmetic. Both the HIP path and the fp64 oracle consume exactly the
tensors it returns (the oracle upcasts the cast values to float64).

Recipe: a CPU torch.Generator seeded with `seed` draws, in this order, Q, K, V,
dO, gQ, gK, gV, each iid N(0, 1) float32 of shape [B, H, N, d]; optional
factors are applied in float32; then every tensor is cast (round to nearest
even) to the workload dtype.
"""

import math
from dataclasses import dataclass

import torch

NAMES = ("Q", "K", "V", "dO", "gQ", "gK", "gV")


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: torch.dtype
    qk_factor: float = 1.0  # multiplies Q and K before the cast

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> float:
        """Algorithmic flops of one BoB call: 34 B H N^2 d (17 N x N x d products)."""
        return 34.0 * self.B * self.H * float(self.N) * float(self.N) * self.d

    @property
    def dtype_name(self) -> str:
        return {torch.float32: "f32", torch.bfloat16: "bf16"}[self.dtype]


# The five workloads. Sizes follow the method's reported regime: 16384 is the
# length where materialising baselines run out of memory, 262144 the longest
# length reported for one GPU.
WORKLOADS = (
    Workload("bob_b1h1n128d64_f32", 1, 1, 128, 64, torch.float32),
    Workload("bob_b2h8n4096d64_bf16_qk0.5", 2, 8, 4096, 64, torch.bfloat16, 0.5),
    Workload("bob_b1h8n16384d128_bf16", 1, 8, 16384, 128, torch.bfloat16),
    Workload("bob_b1h4n65536d64_bf16", 1, 4, 65536, 64, torch.bfloat16),
    Workload("bob_b1h1n262144d64_bf16", 1, 1, 262144, 64, torch.bfloat16),
)


def make_inputs(B, H, N, d, dtype, seed, qk_factor=1.0, H_kv=None):
    """Return the seven input tensors (CPU, `dtype`) as a dict keyed by NAMES.

    H_kv (default H) gives K, V, gK, gV that many heads (grouped-query
    attention); the draw order and distribution are unchanged.
    """
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    hkv = H if H_kv is None else H_kv
    out = {}
    for name in NAMES:
        heads = hkv if name in ("K", "V", "gK", "gV") else H
        x = torch.randn((B, heads, N, d), generator=g, dtype=torch.float32)
        if name in ("Q", "K") and qk_factor != 1.0:
            x.mul_(qk_factor)
        out[name] = x.to(dtype)
    return out


def workload_inputs(w: Workload, seed=None):
    """Inputs of workload `w`; the default seed is the workload's index."""
    if seed is None:
        seed = WORKLOADS.index(w)
    return make_inputs(w.B, w.H, w.N, w.d, w.dtype, seed, w.qk_factor)
