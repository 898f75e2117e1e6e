"""Seeded synthetic workloads for the QLoRA NF4 linear layer.

This module only draws random inputs; it holds none of the method's
arithmetic.  Both the oracle-side tests and the GPU-side tests and benchmark
take their inputs from here, so both sides see the same bytes.

Recipe (stated once, used everywhere):
  * linear j of a workload draws from numpy.random.default_rng([seed, j]),
    with the workload's own seed (0 for the 1024x1024 parity linear, 1 for
    the LLaMA-7B linears, 2 for the 65B decode shapes, 3 for the 33B
    linears) unless a test picks another seed; linears are numbered in the
    order q, k, v, o, gate, up, down;
  * per linear the draws are, in this order:
      W   float32 [N, K], standard normal x 0.02
      an outlier mask, uniform(0,1) < 0.001, and W *= 10 on the mask
      X   [M, K] standard normal, rounded to bf16 (x_kind "relu" keeps
          max(x, 0) of the same draw, "shifted" adds 1: non-zero-mean
          activations such as a ReLU-family layer feeds its down
          projection)
      A   [K, r] normal with standard deviation 1/r, rounded to bf16
      B   [r, N] normal with standard deviation b_std (0.01), rounded to bf16
      dY  [M, N] standard normal, rounded to bf16
  * bf16 rounding is torch's float32 -> bfloat16 conversion on the CPU
    (round to nearest even); tensors travel as uint16 bit patterns.

The shapes stand in for LLaMA-7B, -33B and -65B linear layers (the pages'
models), with token counts from the batch and sequence sizes the pages quote.
"""
from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np


@dataclass(frozen=True)
class Linear:
    name: str
    N: int   # out features (rows of W_lin)
    K: int   # in features


@dataclass(frozen=True)
class Workload:
    key: str
    seed: int
    name: str
    linears: Tuple[Linear, ...]
    M: Tuple[int, ...]
    r: int
    alpha: float
    note: str = ""

    @property
    def s(self) -> float:
        return self.alpha / self.r if self.r else 0.0


def _llama_layer(hidden: int, ffn: int) -> Tuple[Linear, ...]:
    return (Linear("q", hidden, hidden), Linear("k", hidden, hidden),
            Linear("v", hidden, hidden), Linear("o", hidden, hidden),
            Linear("gate", ffn, hidden), Linear("up", ffn, hidden),
            Linear("down", hidden, ffn))


WORKLOADS = {
    "parity_1k": Workload("parity_1k", 0, "single linear 1024x1024, M=16, r=16 (parity case)",
                          (Linear("w", 1024, 1024),), (16,), 16, 16.0),
    "llama7b": Workload("llama7b", 1, "LLaMA-7B layer linears, M=2048 tokens, r=64",
                        _llama_layer(4096, 11008), (2048,), 64, 16.0),
    "decode_65b": Workload("decode_65b", 2, "65B-shaped decode sweep, M in {1,4,16}, r=64",
                           (Linear("qkvo", 8192, 8192), Linear("up", 22016, 8192),
                            Linear("down", 8192, 22016)), (1, 4, 16), 64, 16.0,
                           "alpha not given for this sweep; alpha=16 assumed (s=0.25)"),
    "llama33b_recompute": Workload("llama33b_recompute", 3,
                                   "33B-shaped layer linears, M=4096 tokens, r=64, "
                                   "recompute bwd", _llama_layer(6656, 17920), (4096,), 64, 16.0),
    "stack_65b": Workload("stack_65b", 4, "65B-shaped stack, 80 layers x 7 linears, M=2048, r=64",
                          _llama_layer(8192, 22016) * 80, (2048,), 64, 16.0),
}


def to_bf16_bits(a) -> np.ndarray:
    """float32 -> bf16 bit patterns via torch's CPU conversion (RNE)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def draw_weight(rng, N: int, K: int) -> np.ndarray:
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    mask = rng.random((N, K)) < 0.001
    W[mask] *= np.float32(10.0)
    return W


@dataclass
class LinearInputs:
    W: np.ndarray            # float32 [N, K]
    X: np.ndarray            # bf16 bits [M, K]
    A: np.ndarray            # bf16 bits [K, r]
    B: np.ndarray            # bf16 bits [r, N]
    dY: np.ndarray = None    # bf16 bits [M, N]
    extra: dict = field(default_factory=dict)


X_KINDS = ("normal", "relu", "shifted")


def draw_activations(rng, M: int, K: int, x_kind: str = "normal") -> np.ndarray:
    """[M, K] float32 activations: standard normal, its positive part
    ("relu") or the standard normal plus 1 ("shifted"); one draw either way."""
    if x_kind not in X_KINDS:
        raise ValueError(f"x_kind must be one of {X_KINDS}")
    x = rng.standard_normal((M, K), dtype=np.float32)
    if x_kind == "relu":
        x = np.maximum(x, np.float32(0.0))
    elif x_kind == "shifted":
        x = x + np.float32(1.0)
    return x


def draw_linear(rng, N: int, K: int, M: int, r: int, b_std: float = 0.01,
                with_grad: bool = True, x_kind: str = "normal") -> LinearInputs:
    W = draw_weight(rng, N, K)
    X = to_bf16_bits(draw_activations(rng, M, K, x_kind))
    a_std = np.float32(1.0 / r) if r else np.float32(0.0)
    A = to_bf16_bits(rng.standard_normal((K, r), dtype=np.float32) * a_std)
    B = to_bf16_bits(rng.standard_normal((r, N), dtype=np.float32) * np.float32(b_std))
    dY = (to_bf16_bits(rng.standard_normal((M, N), dtype=np.float32))
          if with_grad else None)
    return LinearInputs(W, X, A, B, dY)


def linear_rng(wl_seed: int, lin_idx: int, seed: int = None):
    return np.random.default_rng([wl_seed if seed is None else seed, lin_idx])


def workload_inputs(key: str, M: int = None, seed: int = None,
                    linears: List[int] = None, with_grad: bool = True):
    """Yield (Linear, LinearInputs) for the linears of a workload, in order.

    Each linear has its own generator, so a subset yields the same bytes as
    the full workload for those linears.
    """
    wl = WORKLOADS[key]
    m = wl.M[0] if M is None else M
    idxs = range(len(wl.linears)) if linears is None else linears
    for i in idxs:
        lin = wl.linears[i]
        yield lin, draw_linear(linear_rng(wl.seed, i, seed), lin.N, lin.K, m, wl.r,
                               with_grad=with_grad)


def device_weight(torch, dev, N: int, K: int, seed: int):
    """The 65B stack's weights, drawn on the device (the 65B stack is too large
    to draw on the host): torch.Generator(device).manual_seed(seed), W =
    standard normal x 0.02, outliers (uniform < 0.001) x 10, float32 [N, K]."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    W = torch.randn((N, K), generator=g, device=dev, dtype=torch.float32) * 0.02
    mask = torch.rand((N, K), generator=g, device=dev) < 0.001
    # (where(), not masked indexing: the latter fails beyond 2^31 elements)
    return torch.where(mask, W * 10.0, W)


def device_adapters(torch, dev, N: int, K: int, r: int, seed: int, b_std: float = 0.01):
    """A [K, r] ~ N(0, 1/r) and B [r, N] ~ N(0, b_std), bf16, drawn on the
    device with torch.Generator(device).manual_seed(seed)."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    A = (torch.randn((K, r), generator=g, device=dev) / r).to(torch.bfloat16)
    B = (torch.randn((r, N), generator=g, device=dev) * b_std).to(torch.bfloat16)
    return A, B


def device_activations(torch, dev, M: int, K: int, seed: int):
    """X [M, K] standard normal, bf16, drawn on the device."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)

