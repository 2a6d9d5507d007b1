"""Seeded synthetic inputs for the GEMM workloads.

This module draws random matrices and rounds them to fp16/bf16.  It holds
none of the product's arithmetic and is the only code shared between the
GPU tests and the CPU oracle: both receive the same tensors from here.

Recipe (all draws on the CPU with ``torch.Generator().manual_seed(seed)``,
so every run and every machine sees the same bits):

* ``uniform``: u ~ U[0, 1) in fp32, x = lo + (hi - lo) * u, times an
  optional ``scale``, rounded to the 16-bit type to nearest even.  With
  ``nonzero`` every entry that rounds to +-0 is drawn again from the same
  generator until none is left.
* ``normal``: x = std * n with n ~ N(0, 1) in fp32, rounded the same way
  (``std`` is the standard deviation).

The workload table below gives the five GEMM shapes the library is tested
and measured on, with their value recipes and seeds; ``ATTENTION`` holds the
attention workloads (head dimension 256, the pages' SDP kernel) in the same
form.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

_TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16}


def uniform(shape, seed: int, lo: float = -1.0, hi: float = 1.0, scale: float = 1.0,
            dtype: str = "f16", nonzero: bool = False) -> torch.Tensor:
    """CPU tensor of ``dtype`` with entries lo + (hi-lo)*U[0,1), scaled."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    td = _TORCH_DTYPE[dtype]

    def draw(n_or_shape):
        u = torch.rand(n_or_shape, generator=g, dtype=torch.float32)
        x = lo + (hi - lo) * u
        if scale != 1.0:
            x = x * scale
        return x.to(td)

    out = draw(tuple(shape))
    if nonzero:
        flat = out.view(-1)
        while True:
            zeros = (flat == 0).nonzero().view(-1)
            if zeros.numel() == 0:
                break
            flat[zeros] = draw(zeros.numel())
    return out


def normal(shape, seed: int, std: float, dtype: str = "bf16") -> torch.Tensor:
    """CPU tensor of ``dtype`` with entries std * N(0, 1)."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    n = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    return (n * std).to(_TORCH_DTYPE[dtype])


def small_integers(shape, seed: int, lo: int = -2, hi: int = 2, dtype: str = "f16") -> torch.Tensor:
    """Integers drawn uniformly from [lo, hi], exactly representable in the
    16-bit type.  Products and partial sums of these stay exact integers in
    fp32 while |sum| < 2^24, so any correct summation order gives the same
    bits."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    x = torch.randint(lo, hi + 1, tuple(shape), generator=g, dtype=torch.int32)
    return x.to(_TORCH_DTYPE[dtype])


def bits(t: torch.Tensor):
    """The 16-bit patterns of a CPU fp16/bf16 tensor as a numpy uint16 array."""
    import numpy as np
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@dataclass(frozen=True)
class Workload:
    """One GEMM workload: shapes, types, value recipe and seeds."""
    name: str
    dtype: str              # input type: "f16" or "bf16"
    batch: int
    M: int
    N: int
    K: int
    out_fp32: bool
    a_recipe: dict = field(default_factory=dict)
    b_recipe: dict = field(default_factory=dict)
    base_seed: int = 0
    rotating: int = 1       # distinct (A, B) sets cycled through when timing
    rotate_a: bool = True   # False: one A shared by all rotating sets

    @property
    def flops(self) -> int:
        return 2 * self.batch * self.M * self.N * self.K

    @property
    def compulsory_bytes(self) -> int:
        """Each operand read once and C written once."""
        cb = 4 if self.out_fp32 else 2
        return self.batch * (2 * self.M * self.K + 2 * self.K * self.N + cb * self.M * self.N)

    def seed(self, j: int) -> int:
        """Seed of rotating set j (A is drawn with it, B with it + 500)."""
        return self.base_seed * 1000 + j

    def _draw(self, recipe: dict, shape, seed: int) -> torch.Tensor:
        kind = recipe.get("kind", "uniform")
        if kind == "uniform":
            return uniform(shape, seed, lo=recipe.get("lo", -1.0), hi=recipe.get("hi", 1.0),
                           scale=recipe.get("scale", 1.0), dtype=self.dtype,
                           nonzero=recipe.get("nonzero", False))
        if kind == "normal":
            return normal(shape, seed, std=recipe["std"], dtype=self.dtype)
        raise ValueError(kind)

    def a_shape(self):
        return (self.batch, self.M, self.K) if self.batch > 1 else (self.M, self.K)

    def b_shape(self):
        return (self.batch, self.K, self.N) if self.batch > 1 else (self.K, self.N)

    def c_shape(self):
        return (self.batch, self.M, self.N) if self.batch > 1 else (self.M, self.N)

    def make_a(self, j: int = 0) -> torch.Tensor:
        return self._draw(self.a_recipe, self.a_shape(), self.seed(j if self.rotate_a else 0))

    def make_b(self, j: int = 0) -> torch.Tensor:
        return self._draw(self.b_recipe, self.b_shape(), self.seed(j) + 500)


WORKLOADS = {
    # small correctness shape, finishes in well under a second on the CPU
    "f16_256": Workload("f16_256", "f16", 1, 256, 256, 256, False,
                        {"kind": "uniform", "nonzero": True}, {"kind": "uniform", "nonzero": True},
                        base_seed=101, rotating=8),
    # the headline compute-bound shape
    "f16_4096": Workload("f16_4096", "f16", 1, 4096, 4096, 4096, False,
                         {"kind": "uniform", "nonzero": True}, {"kind": "uniform", "nonzero": True},
                         base_seed=102, rotating=8),
    # long K loop, bf16 in, fp32 out
    "bf16_4096x4096x16384": Workload("bf16_4096x4096x16384", "bf16", 1, 4096, 4096, 16384, True,
                                     {"kind": "normal", "std": 1.0 / math.sqrt(16384)},
                                     {"kind": "normal", "std": 1.0 / math.sqrt(16384)},
                                     base_seed=103, rotating=4),
    # attention-score shape: 64 independent 4096x256 . 256x4096 products
    "f16_batched_64x4096x4096x256": Workload("f16_batched_64x4096x4096x256", "f16", 64, 4096, 4096,
                                             256, False,
                                             {"kind": "uniform", "lo": -0.5, "hi": 0.5},
                                             {"kind": "uniform", "lo": -0.5, "hi": 0.5},
                                             base_seed=104, rotating=2),
    # decode-like memory-bound shape; 16 rotating B (weight) buffers, one A
    "f16_skinny_64x8192x8192": Workload("f16_skinny_64x8192x8192", "f16", 1, 64, 8192, 8192, False,
                                        {"kind": "uniform"},
                                        {"kind": "uniform", "scale": 1.0 / math.sqrt(8192)},
                                        base_seed=105, rotating=16, rotate_a=False),
}


@dataclass(frozen=True)
class AttentionWorkload:
    """One attention workload O = softmax(scale Q K^T) V: BH independent
    (batch x head) problems of Sq query rows, Skv keys and head dimension D,
    with Q, K, V drawn by ``recipe`` (Q with seed(j), K with seed(j) + 500,
    V with seed(j) + 700) and scale 1/sqrt(D)."""
    name: str
    dtype: str
    BH: int
    Sq: int
    Skv: int
    D: int
    out_fp32: bool
    recipe: dict = field(default_factory=dict)
    base_seed: int = 0
    rotating: int = 1

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def flops(self) -> int:
        """Both products: Q K^T and P V, 2 flops per multiply-add each."""
        return 4 * self.BH * self.Sq * self.Skv * self.D

    @property
    def compulsory_bytes(self) -> int:
        ob = 4 if self.out_fp32 else 2
        return self.BH * self.D * (2 * self.Sq + 4 * self.Skv + ob * self.Sq)

    def seed(self, j: int) -> int:
        return self.base_seed * 1000 + j

    def _draw(self, shape, seed):
        r = self.recipe
        return uniform(shape, seed, lo=r.get("lo", -1.0), hi=r.get("hi", 1.0), dtype=self.dtype)

    def make_q(self, j: int = 0) -> torch.Tensor:
        return self._draw((self.BH, self.Sq, self.D), self.seed(j))

    def make_k(self, j: int = 0) -> torch.Tensor:
        return self._draw((self.BH, self.Skv, self.D), self.seed(j) + 500)

    def make_v(self, j: int = 0) -> torch.Tensor:
        return self._draw((self.BH, self.Skv, self.D), self.seed(j) + 700)


ATTENTION = {
    # small shape the oracle forms whole in about a second
    "attn_f16_2x512x512x256": AttentionWorkload("attn_f16_2x512x512x256", "f16", 2, 512, 512, 256, False,
                                                {"lo": -0.5, "hi": 0.5}, base_seed=201, rotating=2),
    # the attention the batched 64 x 4096x256 . 256x4096 product is the first
    # half of: 64 heads of 4096 queries and keys, head dimension 256, values
    # as that product's operands
    "attn_f16_64x4096x4096x256": AttentionWorkload("attn_f16_64x4096x4096x256", "f16", 64, 4096, 4096, 256,
                                                   False, {"lo": -0.5, "hi": 0.5}, base_seed=202, rotating=2),
    # the same at head dimension 128
    "attn_f16_64x4096x4096x128": AttentionWorkload("attn_f16_64x4096x4096x128", "f16", 64, 4096, 4096, 128,
                                                   False, {"lo": -0.5, "hi": 0.5}, base_seed=203, rotating=2),
}
