"""Rotary position transform of q and k, test infrastructure.

Source: page "KV Cache 与 Prefill/Decode 推理路径", prefix-equality proof, RoPE
paragraph: the query and key at position p are each multiplied by a rotation
fixed by the position id, so their inner product depends only on the distance
between the two positions.  The page's own formulas did not survive extraction;
page 1 (section 2.3) only requires that the rotated q and k are the ones used in
the dot product and (section 2.5) that the cache holds the rotated keys.

Reading fixed for this library (the pages leave it open):

* pairing: dimension i is rotated together with dimension i + d/2, i < d/2;
* frequency of pair i: theta ** (-2 i / d), angle = p * frequency, in double;
* c = float32(cos(angle)), s = float32(sin(angle)) from the C library;
* rotation in float32 with one rounding per product and per sum (no fused
  multiply-add):  x' = (x*c) - (y*s),  y' = (x*s) + (y*c);
* then rounded to the storage dtype (bfloat16 by nearest-even).

theta == 0 means "no position transform" (the toy decoder of page 2).
"""
import functools
import math

import numpy as np


def inv_freq(theta: float, d: int) -> list:
    return [math.pow(theta, -2.0 * i / d) for i in range(d // 2)]


@functools.lru_cache(maxsize=None)
def _row(theta: float, d: int, p: int) -> tuple:
    """(cos, sin) of every pair at position p, each rounded once to float32."""
    c, s = [], []
    for fi in inv_freq(theta, d):
        a = float(p) * fi
        c.append(math.cos(a))
        s.append(math.sin(a))
    return np.array(c, dtype=np.float32), np.array(s, dtype=np.float32)


def cos_sin(theta: float, d: int, positions) -> tuple:
    """float32 cos and sin tables, shape [len(positions), d/2]."""
    pos = [int(p) for p in positions]
    c = np.empty((len(pos), d // 2), dtype=np.float32)
    s = np.empty((len(pos), d // 2), dtype=np.float32)
    for r, p in enumerate(pos):
        c[r], s[r] = _row(float(theta), int(d), p)
    return c, s


def rotate(x, positions, theta: float) -> np.ndarray:
    """Rotate float32 rows x[..., t, :] by positions[t]; returns float32.

    Every product and every sum is a separate float32 operation, so the
    result is bit-determined by (x, c, s).
    """
    x = np.asarray(x, dtype=np.float32)
    if theta == 0:
        return x.copy()
    d = x.shape[-1]
    if d % 2:
        raise ValueError("rotation needs an even head dimension")
    c, s = cos_sin(theta, d, positions)           # [T, d/2]
    h = d // 2
    a = x[..., :h]
    b = x[..., h:]
    ac = np.multiply(a, c, dtype=np.float32)
    bs = np.multiply(b, s, dtype=np.float32)
    as_ = np.multiply(a, s, dtype=np.float32)
    bc = np.multiply(b, c, dtype=np.float32)
    out = np.empty_like(x)
    out[..., :h] = np.subtract(ac, bs, dtype=np.float32)
    out[..., h:] = np.add(as_, bc, dtype=np.float32)
    return out
