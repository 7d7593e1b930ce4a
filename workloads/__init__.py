"""Seeded synthetic inputs for the attention path.

This module only draws numbers: shapes, random values, masks, position ids,
edit points and page permutations.  It performs none of the attention or cache
arithmetic, so both the float64 oracle and the GPU library can take their
inputs from here without sharing any of the method's code.

Every generator is deterministic in its seed.  Floating-point tensors are
returned as CPU torch tensors of the storage dtype (float32, or bfloat16 made
by round-to-nearest-even from float32 draws); callers move them to the device
or upcast them for the oracle.

Workloads (the shapes of the source pages' examples and of the sizes they
discuss for Llama-3-8B- and Grok-1-shaped attention):

* ``tiny``      B=1, n=4, Hq=2, Hkv=1, d=4, fp32, no rotation, U(-0.2, 0.2)
                from ``random.Random(7)`` (the toy decoder's generator family),
                then 3 single-token decode steps.
* ``ragged``    B=4, n=128, lengths U{1..128}, Hq=8, Hkv=2, d=64, bf16 N(0,1),
                theta 1e4, 16 decode steps.
* ``llama``     B=8, n=2048, Hq=32, Hkv=8, d=128, bf16, theta 5e5, page pool
                handed out in a seeded random order, 64 decode steps.
* ``grok``      B=1, n=8192, Hq=48, Hkv=8, d=128, bf16, theta 1e4; decode at
                T=8192 over a 64-layer cache.
* ``serving``   64 sequences with cached lengths log-uniform in [512, 32768]
                (Hq=32, Hkv=8, d=128), one batched decode step.
* ``edit``      16 sequences of n=4096; an edit at m ~ U{1..4095}; truncate to
                m and re-prefill the regenerated suffix.
"""
from __future__ import annotations

import math
import random
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "AttnShape", "PrefillInputs", "DecodeStep",
    "normal", "uniform_tiny", "right_padded_mask", "positions_for",
    "prefill_inputs", "decode_step_inputs", "page_order",
    "tiny", "ragged", "llama", "grok", "serving_lengths", "edit_points",
    "WORKED_2D",
]

# The two-dimensional worked example of the second page ("手算一次 Attention"):
# one query against two keys.
WORKED_2D = {
    "q": [1.0, 0.0],
    "k": [[1.0, 0.0], [0.0, 1.0]],
    "v": [[10.0, 0.0], [0.0, 20.0]],
}


@dataclass(frozen=True)
class AttnShape:
    B: int
    n: int
    Hq: int
    Hkv: int
    d: int
    dtype: torch.dtype          # storage dtype of Q/K/V and of the cache
    theta: float                # rotation base; 0 means no rotation
    page_size: int = 16


@dataclass
class PrefillInputs:
    shape: AttnShape
    Q: torch.Tensor             # [B, Hq, n, d]
    K: torch.Tensor             # [B, Hkv, n, d]
    V: torch.Tensor             # [B, Hkv, n, d]
    mask: torch.Tensor          # uint8 [B, n]
    positions: torch.Tensor     # int32 [B, n]; -1 where the mask is 0
    lengths: list = field(default_factory=list)   # valid tokens per row


@dataclass
class DecodeStep:
    q: torch.Tensor             # [B, Hq, 1, d]
    k: torch.Tensor             # [B, Hkv, 1, d]
    v: torch.Tensor             # [B, Hkv, 1, d]


def _to_storage(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(dtype)


def normal(shape, seed, dtype=torch.bfloat16) -> torch.Tensor:
    """N(0,1) draws from numpy PCG64(seed), stored in ``dtype`` (RNE)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _to_storage(rng.standard_normal(shape, dtype=np.float32), dtype)


def uniform_tiny(rng: random.Random, shape) -> torch.Tensor:
    """U(-0.2, 0.2) doubles drawn in C order, rounded to float32."""
    count = int(np.prod(shape))
    vals = [rng.uniform(-0.2, 0.2) for _ in range(count)]
    return torch.tensor(np.array(vals, dtype=np.float64).astype(np.float32).reshape(shape))


def right_padded_mask(lengths, n) -> torch.Tensor:
    m = torch.zeros((len(lengths), n), dtype=torch.uint8)
    for b, nb in enumerate(lengths):
        m[b, :nb] = 1
    return m


def positions_for(mask: torch.Tensor, start) -> torch.Tensor:
    """Position ids: c_b, c_b+1, ... over the valid tokens of each row, -1 elsewhere."""
    B, n = mask.shape
    pos = torch.full((B, n), -1, dtype=torch.int32)
    for b in range(B):
        c = int(start[b]) if not isinstance(start, int) else start
        idx = torch.nonzero(mask[b]).flatten()
        pos[b, idx] = torch.arange(c, c + idx.numel(), dtype=torch.int32)
    return pos


def prefill_inputs(shape: AttnShape, seed: int, lengths=None, start=0,
                   poison_padding: bool = False) -> PrefillInputs:
    """Q, K, V ~ N(0,1) for every rectangular row, right-padded validity mask.

    ``start`` is the cache length each row continues from (an int or a list).
    With ``poison_padding`` every padded row of Q, K and V holds NaN, which a
    correct implementation must never let reach a valid output.
    """
    B, n = shape.B, shape.n
    if lengths is None:
        lengths = [n] * B
    Q = normal((B, shape.Hq, n, shape.d), seed, shape.dtype)
    K = normal((B, shape.Hkv, n, shape.d), seed + 100_000, shape.dtype)
    V = normal((B, shape.Hkv, n, shape.d), seed + 200_000, shape.dtype)
    mask = right_padded_mask(lengths, n)
    if poison_padding:
        for b, nb in enumerate(lengths):
            for t in (Q, K, V):
                t[b, :, nb:, :] = float("nan")
    pos = positions_for(mask, start if not isinstance(start, int) else [start] * B)
    return PrefillInputs(shape, Q, K, V, mask, pos, list(lengths))


def decode_step_inputs(shape: AttnShape, seed: int, step: int) -> DecodeStep:
    """Fresh q, k, v ~ N(0,1) for one single-token step, seeded by (seed, step)."""
    s = seed * 1000 + 500 + step
    return DecodeStep(
        q=normal((shape.B, shape.Hq, 1, shape.d), s, shape.dtype),
        k=normal((shape.B, shape.Hkv, 1, shape.d), s + 100_000, shape.dtype),
        v=normal((shape.B, shape.Hkv, 1, shape.d), s + 200_000, shape.dtype),
    )


def page_order(num_pages: int, seed) -> list:
    """Initial free-page order: identity for ``seed is None``, else a PCG64 permutation."""
    if seed is None:
        return list(range(num_pages))
    rng = np.random.Generator(np.random.PCG64(seed))
    return [int(x) for x in rng.permutation(num_pages)]


# ---------------------------------------------------------------- workloads

def tiny():
    """B=1, n=4, Hq=2, Hkv=1, d=4 fp32 from random.Random(7); 3 decode steps."""
    shape = AttnShape(B=1, n=4, Hq=2, Hkv=1, d=4, dtype=torch.float32, theta=0.0)
    rng = random.Random(7)
    Q = uniform_tiny(rng, (1, 2, 4, 4))
    K = uniform_tiny(rng, (1, 1, 4, 4))
    V = uniform_tiny(rng, (1, 1, 4, 4))
    mask = right_padded_mask([4], 4)
    pre = PrefillInputs(shape, Q, K, V, mask, positions_for(mask, [0]), [4])
    steps = []
    for _ in range(3):
        steps.append(DecodeStep(q=uniform_tiny(rng, (1, 2, 1, 4)),
                                k=uniform_tiny(rng, (1, 1, 1, 4)),
                                v=uniform_tiny(rng, (1, 1, 1, 4))))
    return pre, steps


def ragged_lengths(B=4, n=128, seed=1002):
    rng = np.random.Generator(np.random.PCG64(seed))
    return [int(x) for x in rng.integers(1, n + 1, size=B)]


def ragged(poison_padding=False, seed=1002):
    shape = AttnShape(B=4, n=128, Hq=8, Hkv=2, d=64, dtype=torch.bfloat16, theta=1e4)
    lengths = ragged_lengths(4, 128, seed)
    return prefill_inputs(shape, seed, lengths, 0, poison_padding)


LLAMA = AttnShape(B=8, n=2048, Hq=32, Hkv=8, d=128, dtype=torch.bfloat16, theta=5e5)
GROK = AttnShape(B=1, n=8192, Hq=48, Hkv=8, d=128, dtype=torch.bfloat16, theta=1e4)
SERVING = AttnShape(B=64, n=1, Hq=32, Hkv=8, d=128, dtype=torch.bfloat16, theta=5e5)
EDIT = AttnShape(B=16, n=4096, Hq=32, Hkv=8, d=128, dtype=torch.bfloat16, theta=5e5)


def llama(seed=1003):
    return prefill_inputs(LLAMA, seed)


def grok(seed=1004):
    return prefill_inputs(GROK, seed)


def serving_lengths(B=64, lo=512, hi=32768, seed=1005):
    """L_b = floor(exp(U(ln lo, ln hi))), clamped to [lo, hi]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    u = rng.uniform(math.log(lo), math.log(hi), size=B)
    return [min(hi, max(lo, int(math.floor(math.exp(x))))) for x in u]


def edit_points(B=16, n=4096, seed=1006):
    """Edit positions m_b ~ U{1..n-1}, 0-based: tokens [0, m_b) are kept."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return [int(x) for x in rng.integers(1, n, size=B)]


def normal_device(shape, seed, dtype=torch.bfloat16, device="cuda") -> torch.Tensor:
    """N(0,1) drawn on the device by torch's seeded generator (for fills too
    large to draw on the host quickly); stored in ``dtype``."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(dtype)
