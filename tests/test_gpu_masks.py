"""GPU parity of general validity masks: padding before, after and between the
valid tokens of a row.

Valid tokens take consecutive positions (and cache slots) in row order;
padding rows may hold NaN and must come out as exact zeros.  Outputs are
compared with the float64 oracle per row, the cache bit for bit, and the same
tokens laid out with different padding must give bit-identical outputs.
"""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from harness import Pair, as_f32, compare_rows, gather

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_gqa_attention_attn_amd  # noqa: F401  (fails loudly if the library is missing)


def _holey(shape, seed, rows_per_b, starts):
    """Q, K, V ~ N(0,1) with NaN in every padding row; mask and positions for the
    given valid rows of each batch row (positions start_b, start_b + 1, ...)."""
    B, n = shape.B, shape.n
    Q = W.normal((B, shape.Hq, n, shape.d), seed, shape.dtype)
    K = W.normal((B, shape.Hkv, n, shape.d), seed + 100_000, shape.dtype)
    V = W.normal((B, shape.Hkv, n, shape.d), seed + 200_000, shape.dtype)
    mask = torch.zeros((B, n), dtype=torch.uint8)
    pos = torch.full((B, n), -1, dtype=torch.int32)
    for b, rows in enumerate(rows_per_b):
        rows = torch.tensor(rows, dtype=torch.long)
        mask[b, rows] = 1
        pos[b, rows] = torch.arange(starts[b], starts[b] + len(rows), dtype=torch.int32)
        pad = torch.ones(n, dtype=torch.bool)
        pad[rows] = False
        for t in (Q, K, V):
            t[b][:, pad] = float("nan")
    return Q, K, V, mask, pos


def _check(O, ref, mask, Hq, dtype):
    valid = mask.numpy().astype(bool)[:, None, :].repeat(Hq, 1)
    compare_rows(O, ref, dtype, rows_mask=valid)
    assert np.all(as_f32(O)[~valid] == 0.0), "padding rows must be written as 0"


def _patterns(n, rng):
    """Rows with holes: several runs, left + right padding, a single token, none."""
    runs = sorted(rng.choice(np.arange(n), size=n // 2, replace=False).tolist())
    return [runs,
            [0, 1, 2, 7, 8, n - 3, n - 1],
            list(range(5, n - 9)) + [n - 4],
            [n // 2],
            []]


@pytest.mark.parametrize("dtype,Hq,Hkv,d", [(torch.bfloat16, 32, 8, 128), (torch.bfloat16, 8, 2, 64),
                                            (torch.float32, 4, 2, 32)])
def test_masks_with_holes(dtype, Hq, Hkv, d):
    """A prefill, a second prefill continuing each cache with holes again, decode
    steps, and gqa_attention on holey rows inside the cache."""
    import causal_gqa_attention_attn_amd as lib
    say(f"case: masks with holes, {dtype} Hq={Hq} Hkv={Hkv} d={d}")
    rng = np.random.default_rng(31)
    n = 150
    rows = _patterns(n, rng)
    B = len(rows)
    shape = W.AttnShape(B=B, n=n, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, theta=1e4)
    pair = Pair(1, Hkv, d, 128, B, 24, dtype, 1e4, free_order=W.page_order(128, 32))
    ids = list(range(B))
    Q, K, V, mask, pos = _holey(shape, 900, rows, [0] * B)
    O, ref = pair.prefill(0, ids, Q, K, V, mask, pos)
    _check(O, ref, mask, Hq, dtype)
    pair.check_cache(ids)
    lens = [len(r) for r in rows]
    rows2 = [_patterns(n, rng)[(b + 1) % B] for b in range(B)]
    Q, K, V, mask, pos = _holey(shape, 901, rows2, lens)
    O, ref = pair.prefill(0, ids, Q, K, V, mask, pos)
    _check(O, ref, mask, Hq, dtype)
    pair.check_cache(ids)
    live = [b for b in ids if lens[b] + len(rows2[b]) > 0]
    for step in range(2):
        o, r = pair.step(0, live, W.decode_step_inputs(W.AttnShape(B=len(live), n=1, Hq=Hq, Hkv=Hkv, d=d,
                                                                   dtype=dtype, theta=1e4), 902, step))
        compare_rows(o, r, dtype)
    # queries inside the cache: a holey row of 12 tokens at positions 20..31 of sequence 0
    Qm = W.normal((1, Hq, 20, d), 903, dtype)
    sel = [0, 1, 4, 5, 6, 9, 10, 11, 14, 16, 17, 19]
    m = torch.zeros((1, 20), dtype=torch.uint8)
    m[0, sel] = 1
    p = torch.full((1, 20), -1, dtype=torch.int32)
    p[0, sel] = torch.arange(20, 32, dtype=torch.int32)
    Om = torch.full((1, Hq, 20, d), float("nan"), dtype=dtype, device="cuda")
    lib.gqa_attention(pair.gpu.handle, 0, [0], Qm.cuda(), m, p, Om)
    torch.cuda.synchronize()
    refm = pair.ref.prefill_rows(0, 0, as_f32(Qm[0][:, sel]), list(range(20, 32)))
    compare_rows(Om[0][:, sel], refm, dtype)
    pad = [i for i in range(20) if i not in sel]
    assert np.all(as_f32(Om[0][:, pad]) == 0.0)


def test_padding_placement_gives_identical_outputs():
    """The same 70 tokens right-padded, left-padded and scattered with holes:
    identical cache bytes and bit-identical outputs on their rows ([P1] 2.11:
    an unmasked padding key would make a sample's result depend on the layout)."""
    say("case: one sequence's tokens under three padding layouts")
    rng = np.random.default_rng(33)
    n, nv, Hq, Hkv, d = 128, 70, 32, 8, 128
    shape = W.AttnShape(B=1, n=nv, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=5e5)
    base = W.prefill_inputs(shape, 904)
    layouts = [list(range(nv)), list(range(n - nv, n)), sorted(rng.choice(n, size=nv, replace=False).tolist())]
    outs, caches = [], []
    for rows in layouts:
        Q = torch.full((1, Hq, n, d), float("nan"), dtype=torch.bfloat16)
        K = torch.full((1, Hkv, n, d), float("nan"), dtype=torch.bfloat16)
        V = torch.full((1, Hkv, n, d), float("nan"), dtype=torch.bfloat16)
        Q[0][:, rows], K[0][:, rows], V[0][:, rows] = base.Q[0], base.K[0], base.V[0]
        mask = torch.zeros((1, n), dtype=torch.uint8)
        mask[0, rows] = 1
        pos = torch.full((1, n), -1, dtype=torch.int32)
        pos[0, rows] = torch.arange(nv, dtype=torch.int32)
        pair = Pair(1, Hkv, d, 16, 1, 16, torch.bfloat16, 5e5)
        O, _ = pair.prefill(0, [0], Q, K, V, mask, pos, oracle=False)
        outs.append(O[0][:, rows].cpu())
        caches.append(gather(pair.gpu, 0, 0))
        pad = [i for i in range(n) if i not in rows]
        assert np.all(as_f32(O[0][:, pad]) == 0.0)
    for o, (k, v) in zip(outs[1:], caches[1:]):
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
        assert torch.equal(k.view(torch.int16), caches[0][0].view(torch.int16))
        assert torch.equal(v.view(torch.int16), caches[0][1].view(torch.int16))


def test_holey_chunk_with_workspace_takes_the_tiled_kernel():
    """A short chunk whose rows have holes, passed with a workspace: still exact
    (the split-T kernel takes single runs only, so the tiled kernel runs)."""
    say("case: 8-row chunk with holes and a workspace")
    Hq, Hkv, d = 32, 8, 128
    pair = Pair(1, Hkv, d, 256, 2, 128, torch.bfloat16, 1e4)
    inp = W.prefill_inputs(W.AttnShape(B=2, n=1500, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=1e4), 905,
                           lengths=[1500, 700])
    pair.prefill(0, [0, 1], inp.Q, inp.K, inp.V, inp.mask, inp.positions, oracle=False)
    shape = W.AttnShape(B=2, n=8, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=1e4)
    Q, K, V, mask, pos = _holey(shape, 906, [[0, 2, 3, 7], [1, 6]], [1500, 700])
    O, ref = pair.prefill(0, [0, 1], Q, K, V, mask, pos, workspace=pair.chunk_workspace(2, Hq, 8))
    _check(O, ref, mask, Hq, torch.bfloat16)
    pair.check_cache([0, 1])


@pytest.mark.parametrize("dtype,Hq,Hkv,d", [(torch.bfloat16, 8, 2, 64), (torch.float32, 4, 2, 32)])
def test_many_rows_and_runs_span_launches(dtype, Hq, Hkv, d):
    """70 batch rows, most with two or three runs of valid rows: more rows and
    runs than one attention launch takes, so the entries are cut into several
    launches; then a decode step over all 70 sequences."""
    say(f"case: 70 rows with holes over several launches, {dtype} Hq={Hq} Hkv={Hkv} d={d}")
    rng = np.random.default_rng(35)
    B, n = 70, 40
    rows = []
    for b in range(B):
        k = int(rng.integers(0, 4))
        rows.append(sorted(rng.choice(n, size=int(rng.integers(1, n)), replace=False).tolist()) if k else
                    list(range(int(rng.integers(1, n)))))
    shape = W.AttnShape(B=B, n=n, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, theta=1e4)
    pair = Pair(1, Hkv, d, B * 4, B, 4, dtype, 1e4, free_order=W.page_order(B * 4, 36))
    ids = list(range(B))
    Q, K, V, mask, pos = _holey(shape, 907, rows, [0] * B)
    O, ref = pair.prefill(0, ids, Q, K, V, mask, pos)
    _check(O, ref, mask, Hq, dtype)
    pair.check_cache(ids)
    o, r = pair.step(0, ids, W.decode_step_inputs(W.AttnShape(B=B, n=1, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype,
                                                              theta=1e4), 908, 0))
    compare_rows(o, r, dtype)


@pytest.mark.parametrize("Hq,Hkv,d,window", [(32, 8, 128, 0), (8, 2, 64, 0), (16, 4, 128, 48)])
def test_short_runs_take_32_token_tiles(Hq, Hkv, d, window):
    """Rows whose valid tokens come in runs of at most 32 (here 1 to 12 tokens
    between padding): with 4 dividing Hq/Hkv the launch uses 32-token query
    tiles of four heads.  Two such prefills continue each cache (the second
    one's queries also see the first one's keys), with and without a window."""
    say(f"case: runs of 1..12 tokens, bf16 Hq={Hq} Hkv={Hkv} d={d} window={window}")
    rng = np.random.default_rng(37 + window)
    B, n = 5, 150
    shape = W.AttnShape(B=B, n=n, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=1e4)
    pages = B * 24
    pair = Pair(1, Hkv, d, pages, B, 24, torch.bfloat16, 1e4, max_position=1024,
                free_order=W.page_order(pages, 38), window=window)
    ids = list(range(B))
    lens = [0] * B

    def fragmented():
        rows_per_b = []
        for b in range(B):
            rows, r = [], int(rng.integers(0, 4))
            while r < n:
                k = int(rng.integers(1, 13))
                rows.extend(range(r, min(n, r + k)))
                r += k + int(rng.integers(1, 6))
            rows_per_b.append(rows if b != 3 else rows[:1])
        return rows_per_b

    for rnd in range(2):
        rows = fragmented()
        Q, K, V, mask, pos = _holey(shape, 910 + rnd, rows, lens)
        O, ref = pair.prefill(0, ids, Q, K, V, mask, pos)
        _check(O, ref, mask, Hq, torch.bfloat16)
        lens = [a + len(r) for a, r in zip(lens, rows)]
    pair.check_cache(ids)
