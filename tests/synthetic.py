"""Seeded synthetic inputs for the fused linear cross-entropy workloads.

This module holds no loss arithmetic: it only draws inputs.  Both the oracle
side and the GPU side of a test read the same arrays from here.

Recipe (one numpy Generator per workload, draws in this order):
  hidden  ~ N(0, 1)                        [n_tok][d_model]
  weight  ~ N(0, sigma_w^2)                [vocab][d_model] row-major
  targets ~ uniform ids in [0, vocab), or Zipf(s) ids by inverse CDF
  mask    : exactly round(frac * n_tok) tokens masked, chosen by a seeded
            permutation; 1 = counted
bf16 and fp16 workloads draw in fp32 and round to the 16-bit type (round to
nearest even, done by torch); the oracle reads exactly those values widened to
fp64.
Distillation: student ~ N(0, 4^2), teacher = student + N(0, 1), both rounded
to the workload dtype after the sum.
Label cross-entropy from logits: logits ~ N(0, 4^2) rounded to the dtype,
then targets uniform in [0, vocab), then the mask.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch


@dataclass(frozen=True)
class CEWorkload:
    name: str
    n_tok: int
    d_model: int
    vocab: int
    chunk: int
    dtype: str            # "f64", "bf16" or "f16"
    sigma_w: float
    z_coef: float
    mask_frac: float
    targets: str          # "uniform" or "zipf1.1"
    seed: int


@dataclass(frozen=True)
class DistillWorkload:
    name: str
    n_tok: int
    vocab: int
    dtype: str
    temperature: float
    z_coef: float
    mask_frac: float
    seed: int


# The five workloads: a tiny fp64 case, the Qwen3-0.6B-shaped LM head in fp64
# and in bf16 (the headline), a large bf16 LM head, and logit distillation.
TINY_F64 = CEWorkload("tiny_f64_64x64x1000", 64, 64, 1000, 16, "f64", 1.0 / 8.0, 0.0, 0.0,
                      "uniform", 1)
QWEN_F64 = CEWorkload("qwen06b_head_f64_2048x1024x151936", 2048, 1024, 151936, 256, "f64",
                      0.02, 0.0, 0.0, "uniform", 2)
QWEN_BF16 = CEWorkload("qwen06b_head_bf16_2048x1024x151936", 2048, 1024, 151936, 256, "bf16",
                       0.02, 1e-4, 0.05, "uniform", 3)
LARGE_BF16 = CEWorkload("large_head_bf16_8192x4096x128256", 8192, 4096, 128256, 512, "bf16",
                        0.02, 1e-4, 0.0, "zipf1.1", 4)
DISTILL_BF16 = DistillWorkload("distill_bf16_4096x151936", 4096, 151936, "bf16", 2.0, 1e-4,
                               0.10, 5)


@dataclass(frozen=True)
class LabelWorkload:
    name: str
    n_tok: int
    vocab: int
    dtype: str
    z_coef: float
    mask_frac: float
    seed: int


# Label cross-entropy over materialized logits at the distillation shape.
LABEL_BF16 = LabelWorkload("label_ce_bf16_4096x151936", 4096, 151936, "bf16", 1e-4, 0.10, 6)


def torch_dtype(name: str):
    return {"bf16": torch.bfloat16, "f16": torch.float16, "f64": torch.float64,
            "f32": torch.float32}[name]


def _normal(rng: np.random.Generator, shape, sigma: float, dtype: str) -> torch.Tensor:
    if dtype == "f64":
        return torch.from_numpy(rng.standard_normal(shape, dtype=np.float64) * sigma)
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return torch.from_numpy(x).to(torch_dtype(dtype))


def zipf_ids(rng: np.random.Generator, n: int, vocab: int, s: float) -> np.ndarray:
    """Ids k in [0, vocab) with P(k) proportional to (k+1)^-s, by inverse CDF."""
    p = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    u = rng.random(n)
    return np.minimum(np.searchsorted(cdf, u, side="right"), vocab - 1).astype(np.int64)


def exact_mask(rng: np.random.Generator, n: int, frac: float) -> Optional[np.ndarray]:
    """1 = counted.  Exactly round(frac*n) tokens are masked; None if frac == 0."""
    if frac <= 0.0:
        return None
    k = int(round(frac * n))
    m = np.ones(n, dtype=np.uint8)
    m[rng.permutation(n)[:k]] = 0
    return m


@dataclass
class CEInputs:
    hidden: torch.Tensor      # CPU tensor in the workload dtype
    weight: torch.Tensor
    targets: np.ndarray       # int64
    mask: Optional[np.ndarray]

    def hidden64(self) -> np.ndarray:
        return self.hidden.to(torch.float64).numpy()

    def weight64(self) -> np.ndarray:
        return self.weight.to(torch.float64).numpy()


def ce_inputs(w: CEWorkload, n_tok: Optional[int] = None, d_model: Optional[int] = None,
              vocab: Optional[int] = None, seed: Optional[int] = None) -> CEInputs:
    """Inputs for workload w; the shape or seed can be overridden for small cases."""
    n = n_tok or w.n_tok
    D = d_model or w.d_model
    V = vocab or w.vocab
    rng = np.random.default_rng(w.seed if seed is None else seed)
    H = _normal(rng, (n, D), 1.0, w.dtype)
    W = _normal(rng, (V, D), w.sigma_w, w.dtype)
    if w.targets == "uniform":
        y = rng.integers(0, V, size=n, dtype=np.int64)
    elif w.targets.startswith("zipf"):
        y = zipf_ids(rng, n, V, float(w.targets[4:]))
    else:
        raise ValueError(w.targets)
    m = exact_mask(rng, n, w.mask_frac)
    return CEInputs(H, W, y, m)


@dataclass
class DistillInputs:
    student: torch.Tensor
    teacher: torch.Tensor
    mask: Optional[np.ndarray]


def distill_inputs(w: DistillWorkload, n_tok: Optional[int] = None,
                   vocab: Optional[int] = None, seed: Optional[int] = None,
                   dtype: Optional[str] = None) -> DistillInputs:
    n = n_tok or w.n_tok
    V = vocab or w.vocab
    dt = dtype or w.dtype
    rng = np.random.default_rng(w.seed if seed is None else seed)
    if dt == "f64":
        s = rng.standard_normal((n, V), dtype=np.float64) * 4.0
        u = s + rng.standard_normal((n, V), dtype=np.float64)
        S, U = torch.from_numpy(s), torch.from_numpy(u)
    else:
        s = rng.standard_normal((n, V), dtype=np.float32)
        s *= np.float32(4.0)
        u = rng.standard_normal((n, V), dtype=np.float32)
        u += s
        S, U = torch.from_numpy(s).to(torch_dtype(dt)), torch.from_numpy(u).to(torch_dtype(dt))
    m = exact_mask(rng, n, w.mask_frac)
    return DistillInputs(S, U, m)


@dataclass
class LabelInputs:
    logits: torch.Tensor      # CPU tensor in the workload dtype
    targets: np.ndarray       # int64
    mask: Optional[np.ndarray]


def label_inputs(w: LabelWorkload, n_tok: Optional[int] = None, vocab: Optional[int] = None,
                 seed: Optional[int] = None, dtype: Optional[str] = None) -> LabelInputs:
    n = n_tok or w.n_tok
    V = vocab or w.vocab
    dt = dtype or w.dtype
    rng = np.random.default_rng(w.seed if seed is None else seed)
    if dt == "f64":
        Z = torch.from_numpy(rng.standard_normal((n, V), dtype=np.float64) * 4.0)
    else:
        z = rng.standard_normal((n, V), dtype=np.float32)
        z *= np.float32(4.0)
        Z = torch.from_numpy(z).to(torch_dtype(dt))
    y = rng.integers(0, V, n, dtype=np.int64)
    m = exact_mask(rng, n, w.mask_frac)
    return LabelInputs(Z, y, m)
