"""Seeded synthetic inputs for the Lighthouse Attention layer.

This module only draws random tensors and casts them to the layer's dtype; it
holds none of the layer's arithmetic, so both the CPU oracle (through the
tests) and the HIP path can consume the same arrays.

The workload table mirrors the shapes the pages quote: a 530M Llama-3-style
attention layer at 98,304 tokens (page "gist.science/paper/2605.06554",
Experimental Results; page "skillsmp.com ... lighthouse-attention", results
table) and the 512K extreme-length measurement (same pages, speedup section).
The pages train on C4 text through a trained model; neither is available, so
Q, K and V are i.i.d. normal, optionally scaled per token by a lognormal factor
so that the l2-norm scores spread the way trained activations do.

Draw order per workload (fixed): Q, K, V ~ N(0,1) float32 [B,H,N,d] from
numpy PCG64(seed); then, when ``lognormal`` is set, one factor
m = exp(0.5 * N(0,1)) per (b,h,t) from the same generator, applied to that
token's q, k and v rows; then a cast to the workload dtype with
round-to-nearest-even.  The upstream gradient dO ~ N(0,1) comes from its own
generator PCG64(seed + 1000).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f32" or "bf16"
    p: int
    L: int
    k: int
    seed: int
    lognormal: bool

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # Single head, small: the size every oracle check finishes in seconds.
    "tiny_f32": Workload("tiny_f32", 1, 1, 4096, 64, "f32", 4, 3, 64, 1, False),
    # L = 1: no selection, so the layer must equal dense causal attention.
    "dense_check_f32": Workload("dense_check_f32", 1, 1, 256, 64, "f32", 4, 1, 1, 11, False),
    "mid_bf16": Workload("mid_bf16", 1, 8, 32768, 128, "bf16", 4, 4, 256, 2, True),
    # 530M Llama-3-style layer at 98K context (16 heads of 64).
    "llama530m_98k_k1536": Workload("llama530m_98k_k1536", 1, 16, 98304, 64, "bf16", 4, 4, 1536, 3, True),
    "llama530m_98k_k6144": Workload("llama530m_98k_k6144", 1, 16, 98304, 64, "bf16", 4, 4, 6144, 3, True),
    # Same shapes with clustered high-norm spans and exact ties (built in tests).
    "llama530m_98k_adversarial": Workload("llama530m_98k_adversarial", 1, 16, 98304, 64, "bf16", 4, 4, 1536, 4, True),
    "extreme_512k": Workload("extreme_512k", 1, 16, 524288, 64, "bf16", 4, 6, 1536, 5, True),
    # The ablation optimum of the technical summary (Experimental Results): p = 2, L = 3, k = 1536,
    # on the same 98K layer (S = 30720).
    "ablation_p2_L3_98k": Workload("ablation_p2_L3_98k", 1, 16, 98304, 64, "bf16", 2, 3, 1536, 6, True),
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(x)
    if dtype == "f32":
        return t.contiguous()
    if dtype == "bf16":
        return t.to(torch.bfloat16).contiguous()   # round-to-nearest-even
    raise ValueError(f"unknown dtype {dtype!r}")


def make_qkv(w: Workload):
    """Q, K, V as CPU torch tensors of the workload dtype, shape [B,H,N,d]."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    shape = (w.B, w.H, w.N, w.d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if w.lognormal:
        m = np.exp(np.float32(0.5) * rng.standard_normal((w.B, w.H, w.N, 1), dtype=np.float32))
        q *= m
        k *= m
        v *= m
    return _cast(q, w.dtype), _cast(k, w.dtype), _cast(v, w.dtype)


def make_dout(w: Workload) -> torch.Tensor:
    """Upstream gradient dO ~ N(0,1), [B,H,N,d], workload dtype."""
    rng = np.random.Generator(np.random.PCG64(w.seed + 1000))
    return _cast(rng.standard_normal((w.B, w.H, w.N, w.d), dtype=np.float32), w.dtype)


def make_proj_inputs(B: int, N: int, Dm: int, H: int, d: int, seed: int):
    """Layer input x ~ N(0,1) [B,N,Dm], projection weights w ~ N(0, 1/Dm)
    [3Hd, Dm] (the usual fan-in scaling), and upstream gradients dq, dk, dv
    ~ N(0,1) [B,H,N,d]; all bf16 (round-to-nearest-even), CPU tensors."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((B, N, Dm), dtype=np.float32)
    w = rng.standard_normal((3 * H * d, Dm), dtype=np.float32) * np.float32(1.0 / np.sqrt(Dm))
    rg = np.random.Generator(np.random.PCG64(seed + 1000))
    g = [rg.standard_normal((B, H, N, d), dtype=np.float32) for _ in range(3)]
    return _cast(x, "bf16"), _cast(w, "bf16"), [_cast(a, "bf16") for a in g]


def make_random(shape, seed: int, dtype: str, scale: float = 1.0) -> torch.Tensor:
    """Generic N(0, scale^2) tensor for small ad-hoc cases."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    return _cast(x, dtype)
