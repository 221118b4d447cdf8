"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and casts them to the storage types the
kernels consume; it contains none of the attention arithmetic, so both the HIP
path and the oracle can be fed from it without sharing any of the method.

Recipe (the pages benchmark on random synthetic tensors, no dataset):
  * numpy ``Generator(PCG64(seed))``; ``standard_normal`` float32 draws in the
    order Q, K, V (then dO when a gradient is needed), each ``[B, H, N, d]``
    contiguous;
  * outlier workloads: after the three normal draws, one ``random()`` uniform
    per entry of Q, then K, then V from the same stream; entries with
    ``u < 1e-3`` are multiplied by 20;
  * bf16 tensors are the float32 draws rounded to nearest-even by torch's cast;
    the oracle receives the exact fp64 upcast of the bf16 values;
  * the +-1 signs of the Hadamard rotation come from their own stream (seed 103);
  * merge workloads: partial outputs and LSEs drawn on the device with a seeded
    torch generator (O ~ N(0, 1) as bf16, LSE ~ 7 + 2 N(0, 1), about the LSE of
    a 1024-key shard of N(0, 1) scores).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f32", "bf16", "fp8"
    causal: bool
    seed: int
    outliers: bool = False
    backward: bool = False
    parts: int = 0          # > 0: merge of this many partial results

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    @property
    def flops(self) -> float:
        """Forward FLOPs 4*B*H*N^2*d (two products); a backward workload counts
        10*B*H*N^2*d (five products: S, dP, dV, dK, dQ); halved when causal."""
        f = (10.0 if self.backward else 4.0) * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f

    @property
    def merge_bytes(self) -> int:
        """HBM bytes a merge must move: every part's O and LSE read once, O and
        LSE written once (bf16 O, fp32 LSE)."""
        rows = self.B * self.H * self.N
        return (self.parts + 1) * (rows * self.d * 2 + rows * 4)


# The workloads the benchmark targets and parity cases are built on.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 1, 128, 64, "f32", False, 0),
    "bf16_n2048_d64": Workload("bf16_n2048_d64", 4, 16, 2048, 64, "bf16", False, 1),
    "bf16_causal_n8192_d128": Workload("bf16_causal_n8192_d128", 2, 16, 8192, 128, "bf16", True, 2),
    "fp8_n8192_d128": Workload("fp8_n8192_d128", 2, 16, 8192, 128, "fp8", False, 3, outliers=True),
    # the fp8 path under the causal mask (not one of the pages' configurations)
    "fp8_causal_n8192_d128": Workload("fp8_causal_n8192_d128", 2, 16, 8192, 128, "fp8", True, 8, outliers=True),
    "bf16_bwd_causal_n4096_d128": Workload("bf16_bwd_causal_n4096_d128", 2, 16, 4096, 128, "bf16",
                                           True, 4, backward=True),
    # the fp32 path at a size that fills the chip (not one of the pages' configurations)
    "f32_causal_n4096_d128": Workload("f32_causal_n4096_d128", 2, 16, 4096, 128, "f32", True, 6),
    "f32_bwd_causal_n4096_d128": Workload("f32_bwd_causal_n4096_d128", 2, 16, 4096, 128, "f32",
                                          True, 7, backward=True),
    # combine step of the headline shape sharded over 8 key ranges
    "merge_bf16_s8_n8192_d128": Workload("merge_bf16_s8_n8192_d128", 2, 16, 8192, 128, "bf16", False, 5,
                                         parts=8),
}


def normal_qkv(B, H, N, d, seed, outliers=False, with_dout=False):
    """float32 numpy arrays (Q, K, V[, dO]) with the recipe above."""
    g = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, N, d)
    xs = [g.standard_normal(shape, dtype=np.float32) for _ in range(3)]
    if with_dout:
        xs.append(g.standard_normal(shape, dtype=np.float32))
    if outliers:
        for x in xs[:3]:
            u = g.random(shape, dtype=np.float32)
            x[u < 1e-3] *= 20.0
    return xs


def page_outlier_qkv(B, H, N, d, seed):
    """The FP8 error study's own input model: N(0,1) + N(0,100)*Bernoulli(0.001)
    per entry (variance 100, i.e. sigma 10), for context runs only."""
    g = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, N, d)
    out = []
    for _ in range(3):
        base = g.standard_normal(shape, dtype=np.float32)
        big = g.standard_normal(shape, dtype=np.float32) * 10.0
        bern = g.random(shape, dtype=np.float32) < 1e-3
        out.append(base + big * bern)
    return out


def hadamard_signs(d, seed=103):
    """+-1 int8 vector of length d for the random diagonal of the rotation."""
    g = np.random.Generator(np.random.PCG64(seed))
    return np.where(g.random(d) < 0.5, -1, 1).astype(np.int8)


def to_bf16(x):
    """(torch bf16 CPU tensor, exact fp64 numpy upcast) of a float32 array."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)
    return t, t.to(torch.float64).numpy()


def sample_rows(B, H, N, count, seed):
    """Seeded flat row ids (b*H + h)*N + i, always including rows 0, 1 and N-1
    of the first and last head, sorted and unique."""
    g = np.random.Generator(np.random.PCG64(seed + 7919))
    total = B * H * N
    fixed = [0, min(1, N - 1), N - 1, (B * H - 1) * N, (B * H - 1) * N + N - 1]
    rnd = g.integers(0, total, size=max(count - len(fixed), 0))
    return np.unique(np.concatenate([np.asarray(fixed, np.int64), rnd.astype(np.int64)]))


def merge_parts(w, device):
    """Seeded device tensors (o_parts bf16 [S, B, H, N, d], lse_parts fp32
    [S, B, H, N]) for a merge workload."""
    import torch
    gen = torch.Generator(device=device).manual_seed(w.seed)
    o = torch.randn((w.parts, w.B, w.H, w.N, w.d), generator=gen, device=device).to(torch.bfloat16)
    lse = 7.0 + 2.0 * torch.randn((w.parts, w.B, w.H, w.N), generator=gen, device=device)
    return o, lse
