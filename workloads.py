"""Seeded synthetic KDA inputs, shared by the tests, the benchmark and smoke().

This module holds no part of the method's arithmetic: it only draws random
tensors with the shapes and distributions of the workloads and packs
sequence lengths.  Both the HIP path and the oracle receive the same bytes.

Shapes follow the forward call's argument list ("Debajo del capó: CUTLASS en
Hopper", 7minutos.es): q, k, g [B,T,H,K] bf16; v [B,T,H,V] bf16; beta logits
[B,T,H] bf16; A_log [H] fp32; dt_bias [H,K] fp32; lower_bound a scalar in
[-5, 0]; optional initial/final states [N,H,K,V] in bf16 or fp32; optional
int64 cu_seqlens [N+1].  The kernel supports K = V = 128 only.

Recipe (one numpy PCG64 stream per workload, seed = 1000 + index):
  q, k, v, g, beta ~ N(mean, 1) drawn in that order as float32, then rounded
  to bf16 (round-to-nearest-even); g's mean is 0 except where stated;
  A_log[h] = log(U(1, 16)); dt_bias ~ N(0, 0.1^2); initial state ~ N(0, 0.1^2)
  fp32; scale = 1/sqrt(K).  Varlen lengths come from a separate PCG64 stream
  (seed + 100): L = round(exp(U(ln lo, ln hi))), bumped by one when a multiple
  of 64, appended until the total is reached, the last one trimmed, a short
  remainder merged into the shortest sequence.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

K_DIM = 128
V_DIM = 128
CHUNK = 64


@dataclass
class Workload:
    name: str
    B: int
    T: int
    H: int
    K: int
    V: int
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    beta: torch.Tensor
    A_log: torch.Tensor
    dt_bias: torch.Tensor
    lower_bound: float
    scale: float
    initial_state: Optional[torch.Tensor]
    final_state_dtype: Optional[torch.dtype]
    cu_seqlens: Optional[torch.Tensor]
    seqlens: List[int] = field(default_factory=list)

    @property
    def N(self) -> int:
        return self.B if self.cu_seqlens is None else self.cu_seqlens.numel() - 1

    @property
    def tokens(self) -> int:
        return self.B * self.T

    def to(self, device) -> "Workload":
        mv = lambda t: None if t is None else t.to(device)
        return Workload(self.name, self.B, self.T, self.H, self.K, self.V,
                        mv(self.q), mv(self.k), mv(self.v), mv(self.g), mv(self.beta),
                        mv(self.A_log), mv(self.dt_bias), self.lower_bound, self.scale,
                        mv(self.initial_state), self.final_state_dtype, mv(self.cu_seqlens),
                        list(self.seqlens))

    def head_slice(self, heads) -> "Workload":
        """The same workload restricted to a subset of heads (heads are independent)."""
        idx = torch.as_tensor(list(heads), dtype=torch.long)
        sel = lambda t, dim: t.index_select(dim, idx.to(t.device)).contiguous()
        h0 = None if self.initial_state is None else sel(self.initial_state, 1)
        return Workload(self.name + "[heads]", self.B, self.T, len(idx), self.K, self.V,
                        sel(self.q, 2), sel(self.k, 2), sel(self.v, 2), sel(self.g, 2),
                        sel(self.beta, 2), sel(self.A_log, 0), sel(self.dt_bias, 0),
                        self.lower_bound, self.scale, h0, self.final_state_dtype,
                        self.cu_seqlens, list(self.seqlens))


def _normal_bf16(rng: np.random.Generator, shape, mean: float = 0.0, std: float = 1.0) -> torch.Tensor:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return torch.from_numpy(x).to(torch.bfloat16)


def varlen_lengths(total: int, lo: int, hi: int, seed: int) -> List[int]:
    """Log-uniform lengths in [lo, hi], none a multiple of CHUNK, summing to total."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens: List[int] = []
    while sum(lens) < total:
        L = int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
        if L % CHUNK == 0:
            L += 1
        lens.append(L)
    lens[-1] -= sum(lens) - total
    if lens[-1] < lo and len(lens) > 1:
        rem = lens.pop()
        i = int(np.argmin(lens))
        lens[i] += rem
    for i, L in enumerate(lens):  # keep every length off a chunk multiple
        if L % CHUNK == 0:
            j = (i + 1) % len(lens)
            lens[i] += 1
            lens[j] -= 1
    assert sum(lens) == total and all(L > 0 for L in lens)
    return lens


def make(name: str, B: int, T: int, H: int, seed: int, *, lower_bound: float = -5.0,
         g_mean: float = 0.0, init: Optional[str] = None, final: Optional[str] = "fp32",
         seqlens: Optional[List[int]] = None, K: int = K_DIM, V: int = V_DIM,
         beta_std: float = 1.0) -> Workload:
    """Draw one workload.  ``init``/``final`` are None, "fp32" or "bf16".
    With ``seqlens`` the batch is packed (B must be 1, T = sum(seqlens))."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if seqlens is not None:
        assert B == 1 and T == sum(seqlens)
    q = _normal_bf16(rng, (B, T, H, K))
    k = _normal_bf16(rng, (B, T, H, K))
    v = _normal_bf16(rng, (B, T, H, V))
    g = _normal_bf16(rng, (B, T, H, K), mean=g_mean)
    beta = _normal_bf16(rng, (B, T, H), std=beta_std)
    A_log = torch.from_numpy(np.log(rng.uniform(1.0, 16.0, size=H)).astype(np.float32))
    dt_bias = torch.from_numpy((0.1 * rng.standard_normal(size=(H, K))).astype(np.float32))
    N = B if seqlens is None else len(seqlens)
    h0 = None
    if init is not None:
        h0 = torch.from_numpy((0.1 * rng.standard_normal(size=(N, H, K, V), dtype=np.float32)))
        if init == "bf16":
            h0 = h0.to(torch.bfloat16)
    cu = None
    if seqlens is not None:
        cu = torch.tensor([0] + list(np.cumsum(seqlens)), dtype=torch.int64)
    fdt = {None: None, "fp32": torch.float32, "bf16": torch.bfloat16}[final]
    return Workload(name, B, T, H, K, V, q, k, v, g, beta, A_log, dt_bias,
                    float(np.float32(lower_bound)), float(np.float32(1.0 / math.sqrt(K))),
                    h0, fdt, cu, list(seqlens) if seqlens is not None else [T] * B)


def loss_grads(w: Workload, seed: int, final: Optional[str] = "fp32"):
    """Seeded loss gradients for the backward pass of workload ``w``: d_out ~ N(0, 1)
    bf16 [B, T, H, V] and d_final ~ N(0, 1) [N, H, K, V] ("fp32", "bf16" or None)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    d_out = _normal_bf16(rng, (w.B, w.T, w.H, w.V))
    d_fin = None
    if final is not None:
        d_fin = torch.from_numpy(rng.standard_normal(size=(w.N, w.H, w.K, w.V), dtype=np.float32))
        if final == "bf16":
            d_fin = d_fin.to(torch.bfloat16)
    return d_out, d_fin


# The five workloads the library is measured and checked on.
CONFIG_NAMES = [
    "tiny_T512_H4",
    "batch4_T2048_H32",
    "long_T8192_H32",
    "varlen_32K_H32",
    "long_T131072_H32",
]


def config(i: int) -> Workload:
    seed = 1000 + i
    if i == 0:
        return make(CONFIG_NAMES[0], 1, 512, 4, seed, lower_bound=-5.0, init=None, final="fp32")
    if i == 1:
        return make(CONFIG_NAMES[1], 4, 2048, 32, seed, lower_bound=-5.0, init="fp32", final="fp32")
    if i == 2:
        return make(CONFIG_NAMES[2], 1, 8192, 32, seed, lower_bound=-5.0, init=None, final="bf16")
    if i == 3:
        lens = varlen_lengths(32768, 37, 8192, seed + 100)
        return make(CONFIG_NAMES[3], 1, 32768, 32, seed, lower_bound=-3.0, init="fp32",
                    final="fp32", seqlens=lens)
    if i == 4:
        return make(CONFIG_NAMES[4], 1, 131072, 32, seed, lower_bound=-5.0, g_mean=-1.0,
                    init="fp32", final="fp32")
    raise ValueError("config index must be 0..4")


# The pages' own benchmark shapes: T = 8192 tokens, head dim 128, H = 96 and
# H = 64, as one fixed-length sequence and as eight packed sequences of 1024
# tokens (the uniform-varlen scenario).  The pages do not state the initial
# state, lower bound or gate statistics of these runs; the recipe of the
# T = 8192 workload above is reused (no initial state, lower_bound = -5,
# fp32 final state).
PAGES_NAMES = ["pages_H96_fixed8192", "pages_H96_varlen1024x8", "pages_H64_fixed8192", "pages_H64_varlen1024x8"]


def pages_workload(name: str) -> Workload:
    i = PAGES_NAMES.index(name)
    H = 96 if i < 2 else 64
    seed = 2000 + i
    if i % 2 == 0:
        return make(name, 1, 8192, H, seed, lower_bound=-5.0, init=None, final="fp32")
    return make(name, 1, 8192, H, seed, lower_bound=-5.0, init=None, final="fp32", seqlens=[1024] * 8)


# One long sequence with few heads: the state chains alone occupy few CUs, so
# the forward pass splits them into segments.  Same recipe as the 128K-token
# workload above (g ~ N(-1, 1), lower_bound = -5, fp32 initial and final
# states) with H = 4.
SPLIT_NAMES = ["long_T131072_H4"]


def split_workload(name: str) -> Workload:
    i = SPLIT_NAMES.index(name)
    return make(name, 1, 131072, 4, 3000 + i, lower_bound=-5.0, g_mean=-1.0, init="fp32", final="fp32")


def by_name(name: str) -> Workload:
    """Any workload by name: CONFIG_NAMES, PAGES_NAMES or SPLIT_NAMES."""
    if name in CONFIG_NAMES:
        return config(CONFIG_NAMES.index(name))
    if name in SPLIT_NAMES:
        return split_workload(name)
    return pages_workload(name)


def config_shape(i: int) -> dict:
    """Shapes of a workload without drawing it."""
    shapes = {0: (1, 512, 4), 1: (4, 2048, 32), 2: (1, 8192, 32), 3: (1, 32768, 32), 4: (1, 131072, 32)}
    B, T, H = shapes[i]
    return {"B": B, "T": T, "H": H, "K": K_DIM, "V": V_DIM}
