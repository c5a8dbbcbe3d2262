"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and rounds them to the storage
precision of each workload; it performs none of the attention arithmetic.
Both the fp64 oracle (through the tests) and the GPU path (through the tests
and the benchmark) consume its arrays, so the two sides see identical inputs.

Recipe (one entry of ``WORKLOADS`` per workload):

* values are iid N(0, 1), drawn as float32 by ``numpy.random.Generator(PCG64(seed))``
  in the order Q, K, V, each of shape [B, H, N, d] in C order;
* workloads with outliers then, for Q, K and V in turn, draw a Bernoulli mask
  ``rng.random(shape) < outlier_rate`` from the same generator and multiply the
  selected entries by ``outlier_scale``;
* bf16 / fp8 workloads round the float32 values to bfloat16 (round to nearest
  even) -- that bfloat16 tensor *is* the input both sides consume;
* the random sign vector of the orthogonal rotation used by the fp8 workload is
  drawn from ``PCG64(seed + 1)`` as ``integers(0, 2, d) * 2 - 1``.
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str  # "f32", "bf16" or "fp8" (fp8: bf16 inputs, quantised on the device)
    B: int
    H: int
    N: int
    d: int
    causal: bool
    seed: int
    outlier_rate: float = 0.0
    outlier_scale: float = 1.0

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def flops(self) -> float:
        """Counted attention FLOPs: 4*B*H*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if self.causal else f


# The five workloads: a tiny fp32 case, bf16 causal at N=2048, bf16 d=64 with
# many workgroups, bf16 causal long-sequence (the sequence-parallel case) and
# fp8 causal with 0.1 % x50 outliers.  seed = 1000 + position in this list.
WORKLOADS = [
    Workload("f32_tiny_b1h2n256d64", "f32", 1, 2, 256, 64, False, 1000),
    Workload("bf16_causal_b4h16n2048d128", "bf16", 4, 16, 2048, 128, True, 1001),
    Workload("bf16_b16h16n1024d64", "bf16", 16, 16, 1024, 64, False, 1002),
    Workload("bf16_causal_b1h32n16384d128", "bf16", 1, 32, 16384, 128, True, 1003),
    Workload("fp8_causal_b2h16n8192d128_outliers", "fp8", 2, 16, 8192, 128, True, 1004,
             outlier_rate=1e-3, outlier_scale=50.0),
]


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    for w in WORKLOADS:
        if w.name == name_or_index:
            return w
    raise KeyError(name_or_index)


def draw_qkv(B, H, N, d, seed, dtype="bf16", outlier_rate=0.0, outlier_scale=1.0):
    """Return (q, k, v) as CPU torch tensors (float32 for "f32", bfloat16 otherwise)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, N, d)
    arrs = [rng.standard_normal(shape, dtype=np.float32) for _ in range(3)]
    if outlier_rate > 0.0:
        for a in arrs:
            mask = rng.random(shape) < outlier_rate
            a[mask] *= np.float32(outlier_scale)
    out = []
    for a in arrs:
        t = torch.from_numpy(a)
        if dtype != "f32":
            t = t.to(torch.bfloat16)
        out.append(t)
    return tuple(out)


def draw_signs(d, seed) -> np.ndarray:
    """Random +-1 sign vector (int8) for the orthogonal rotation of Q and K."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.integers(0, 2, d) * 2 - 1).astype(np.int8)


def workload_inputs(w: Workload):
    """(q, k, v) for a workload, plus the rotation signs for fp8 workloads (else None)."""
    q, k, v = draw_qkv(w.B, w.H, w.N, w.d, w.seed, w.dtype, w.outlier_rate, w.outlier_scale)
    signs = draw_signs(w.d, w.seed + 1) if w.dtype == "fp8" else None
    return q, k, v, signs


def sha256(t) -> str:
    a = t.view(torch.int16).numpy() if isinstance(t, torch.Tensor) and t.dtype == torch.bfloat16 else (
        t.numpy() if isinstance(t, torch.Tensor) else np.asarray(t))
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
