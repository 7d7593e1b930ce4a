"""Masked causal grouped-query attention, written out in numpy float64.

Test infrastructure.  Definitions from page "Prefill：整层状态演化与 KV 建立":

* section 2.2, mask M: for a valid query row i of sequence b, M[b,i,j] = 0 when
  both i and j are valid tokens and j <= i, and -inf otherwise.  Invalid query
  rows never enter the softmax; their output is discarded (here: set to 0).
* section 2.3, head map: query head h reads KV head g(h) = floor(h*Hkv/Hq),
  which needs Hkv to divide Hq.
* section 2.3, scores: S = <q_used, k_used> / sqrt(d_h) + M.
* section 2.3, softmax: subtract the maximum over the finite scores of the
  row; the denominator sums the exponentials of the finite scores only.  A valid
  row must hold at least one finite score.
* section 2.3, output: O = sum_j A[j] * V[g(h), j].

With a cache the keys are slots 0..T-1 whose slot number equals the token
position (incremental prefill, page "KV Cache 与 Prefill/Decode 推理路径",
multi-turn lesson: the old prefix is wholly visible and the new block is
lower-triangular).  A query at position p may read the slots j <= p, which is
the same rule as section 2.2 once slot = position.

Sliding window (page "KV Cache 与 Prefill/Decode 推理路径", sliding-window
lesson): the visible range is the latest W positions, the current one
included, so a query at position p reads the slots p - W < j <= p.  W = 0
means no window.
"""
import numpy as np

NEG_INF = float("-inf")


def head_map(h: int, Hq: int, Hkv: int) -> int:
    """g(h) = floor(h * Hkv / Hq)."""
    return (h * Hkv) // Hq


def rect_mask(G) -> np.ndarray:
    """Section 2.2 mask for one prefill with no prior cache.

    G: [B, n] 0/1 validity.  Returns M [B, n, n] float64 with 0 / -inf; a row
    whose query is invalid is all -inf (it never enters the softmax).
    """
    G = np.asarray(G).astype(bool)
    B, n = G.shape
    M = np.full((B, n, n), NEG_INF)
    for b in range(B):
        for i in range(n):
            if not G[b, i]:
                continue
            for j in range(n):
                if G[b, j] and j <= i:
                    M[b, i, j] = 0.0
    return M


def slot_mask(q_pos, T: int) -> np.ndarray:
    """M[i, j] = 0 for cache slots j <= q_pos[i], -inf for later slots; j < T."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    j = np.arange(T, dtype=np.int64)
    return np.where(j[None, :] <= q_pos[:, None], 0.0, NEG_INF)


def window_mask(q_pos, T: int, W: int) -> np.ndarray:
    """M[i, j] = 0 for cache slots q_pos[i] - W < j <= q_pos[i], -inf otherwise
    (W = 0: every slot j <= q_pos[i]); j < T."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    j = np.arange(T, dtype=np.int64)[None, :]
    visible = j <= q_pos[:, None]
    if W > 0:
        visible &= j > q_pos[:, None] - W
    return np.where(visible, 0.0, NEG_INF)


def finite_score_count(M) -> int:
    return int(np.isfinite(np.asarray(M)).sum())


def softmax_finite(S) -> np.ndarray:
    """Row-wise softmax over the finite entries of S (float64)."""
    S = np.asarray(S, dtype=np.float64)
    finite = np.isfinite(S)
    if not finite.any(axis=-1).all():
        raise ValueError("a valid query row has no finite score")
    m = np.max(np.where(finite, S, NEG_INF), axis=-1, keepdims=True)
    E = np.where(finite, np.exp(np.where(finite, S, 0.0) - m), 0.0)
    Z = E.sum(axis=-1, keepdims=True)
    return E / Z


def attend(q_used, k_used, v, M) -> np.ndarray:
    """O for one sequence.

    q_used: [Hq, nq, d]; k_used, v: [Hkv, T, d]; M: [nq, T] (0 / -inf).
    Returns O [Hq, nq, d] float64.
    """
    q_used = np.asarray(q_used, dtype=np.float64)
    k_used = np.asarray(k_used, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Hq, nq, d = q_used.shape
    Hkv = k_used.shape[0]
    if Hq % Hkv:
        raise ValueError("Hkv must divide Hq")
    O = np.zeros((Hq, nq, d))
    if nq == 0:
        return O
    for h in range(Hq):
        g = head_map(h, Hq, Hkv)
        S = (q_used[h] @ k_used[g].T) / np.sqrt(d) + M
        A = softmax_finite(S)
        O[h] = A @ v[g]
    return O


def attend_positions(q_used, q_pos, k_used, v, row_chunk: int = 1024, window: int = 0) -> np.ndarray:
    """O for queries at absolute positions q_pos against cache slots 0..T-1
    (only the latest ``window`` of them when window > 0).

    Rows are independent, so they are evaluated ``row_chunk`` at a time only to
    bound memory; each row's arithmetic is the same as in ``attend``.  A chunk
    only takes the slots that some row of it can see, [lo, hi): every slot
    outside them has M = -inf for every row of the chunk, so it carries zero
    weight and adds nothing to a row's maximum or denominator (section 2.2).
    """
    q_used = np.asarray(q_used, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    out = np.zeros(q_used.shape)
    for r0 in range(0, q_used.shape[1], row_chunk):
        r1 = min(q_used.shape[1], r0 + row_chunk)
        p = q_pos[r0:r1]
        hi = int(p.max()) + 1
        lo = max(0, int(p.min()) - window + 1) if window else 0
        M = window_mask(p - lo, hi - lo, window) if window else slot_mask(p, hi)
        out[:, r0:r1] = attend(q_used[:, r0:r1], k_used[:, lo:hi], v[:, lo:hi], M)
    return out
