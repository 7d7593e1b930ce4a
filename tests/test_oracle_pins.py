"""Pins of the float64 oracle against facts fixed outside it.

Each check ties one part of the oracle to something it does not compute
itself: values printed on the source pages, closed forms, an independent
library routine (torch's scaled-dot-product attention and bfloat16
conversion, numpy complex arithmetic), pure-Python brute force, or counts the
pages print.  The checks are plain functions so that ``test_oracle_mutants``
can plant mistakes in the oracle and see them caught.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention, brute, rope
from oracle.bf16 import round_f32_to_bf16
from oracle.cache_model import CacheModel, OracleError

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = [float(v) for v in vals]
    return out


# ------------------------------------------------------------------ worked example

def _worked_inputs():
    q = np.array([[[1.0, 0.0]]])                       # [Hq=1, 1, 2]
    k = np.array([[[1.0, 0.0], [0.0, 1.0]]])           # [Hkv=1, 2, 2]
    v = np.array([[[10.0, 0.0], [0.0, 20.0]]])
    return q, k, v


def check_worked_example():
    g = read_golden("worked_2d.txt")
    q, k, v = _worked_inputs()
    # second position: both keys visible
    o = attention.attend_positions(q, [1], k, v)[0, 0]
    A = attention.softmax_finite(np.array([[1 / math.sqrt(2), 0.0]]))[0]
    w1, w2, tol = g["weights_both"]
    assert abs(A[0] - w1) <= tol and abs(A[1] - w2) <= tol
    o1, o2, tol = g["output_both"]
    assert abs(o[0] - o1) <= tol and abs(o[1] - o2) <= tol
    # closed form: p1 = 1 / (1 + exp(-1/sqrt(2)))
    p1 = 1.0 / (1.0 + math.exp(-1.0 / math.sqrt(2.0)))
    assert abs(o[0] - 10 * p1) < 1e-12 and abs(o[1] - 20 * (1 - p1)) < 1e-12
    # first position: only k1 visible -> exactly v1
    o_first = attention.attend_positions(q, [0], k, v)[0, 0]
    f1, f2, _ = g["output_first"]
    assert o_first[0] == f1 and o_first[1] == f2


def test_worked_example():
    check_worked_example()


def test_worked_example_brute():
    g = read_golden("worked_2d.txt")
    q, k, v = _worked_inputs()
    o = brute.attend_brute(q.tolist(), [1], k.tolist(), v.tolist())[0][0]
    o1, o2, tol = g["output_both"]
    assert abs(o[0] - o1) <= tol and abs(o[1] - o2) <= tol
    assert brute.attend_brute(q.tolist(), [0], k.tolist(), v.tolist())[0][0] == [10.0, 0.0]


def test_worked_example_gqa_two_heads():
    """Two query heads with the same q on one KV head give the same output twice."""
    q, k, v = _worked_inputs()
    q2 = np.concatenate([q, q], axis=0)
    o = attention.attend_positions(q2, [1], k, v)
    p1 = 1.0 / (1.0 + math.exp(-1.0 / math.sqrt(2.0)))
    for h in range(2):
        assert abs(o[h, 0, 0] - 10 * p1) < 1e-12 and abs(o[h, 0, 1] - 20 * (1 - p1)) < 1e-12


# ------------------------------------------------------------------ closed forms

def check_single_key_and_uniform():
    rng = np.random.default_rng(11)
    k = rng.standard_normal((1, 5, 8))
    v = rng.standard_normal((1, 5, 8))
    q = rng.standard_normal((2, 1, 8))
    # the query at position 0 sees one key: its output is that value row exactly
    o = attention.attend_positions(q, [0], k, v)
    assert np.array_equal(o[0, 0], v[0, 0]) and np.array_equal(o[1, 0], v[0, 0])
    # a zero query gives equal weights: the mean of the visible values
    qz = np.zeros((1, 5, 8))
    o = attention.attend_positions(qz, np.arange(5), k, v)
    for i in range(5):
        assert np.allclose(o[0, i], v[0, :i + 1].mean(axis=0), rtol=0, atol=1e-13)


def test_single_key_and_uniform():
    check_single_key_and_uniform()


def check_against_textbook_sdpa():
    """GQA equals multi-head attention with each KV head repeated for its group.

    The reference is torch's scaled_dot_product_attention (float64, CPU, causal)
    on K/V expanded with repeat_interleave: the textbook form of g(h).
    """
    rng = np.random.default_rng(5)
    for (Hq, Hkv, n, d) in [(4, 2, 9, 8), (6, 2, 7, 16), (8, 8, 5, 4), (6, 1, 12, 6)]:
        q = rng.standard_normal((Hq, n, d))
        k = rng.standard_normal((Hkv, n, d))
        v = rng.standard_normal((Hkv, n, d))
        o = attention.attend_positions(q, np.arange(n), k, v)
        G = Hq // Hkv
        kt = torch.from_numpy(k).repeat_interleave(G, dim=0)
        vt = torch.from_numpy(v).repeat_interleave(G, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None], kt[None], vt[None], is_causal=True)[0].numpy()
        assert np.max(np.abs(o - ref)) < 1e-12, (Hq, Hkv, n, d)


def test_against_textbook_sdpa():
    check_against_textbook_sdpa()


def check_brute_force():
    """numpy oracle == pure-Python loops on tiny ragged shapes with a cache prefix."""
    rng = np.random.default_rng(3)
    for (Hq, Hkv, T, nq, d) in [(2, 1, 4, 4, 4), (4, 2, 7, 3, 5), (6, 3, 9, 5, 2), (3, 1, 6, 1, 3)]:
        k = rng.standard_normal((Hkv, T, d))
        v = rng.standard_normal((Hkv, T, d))
        q = rng.standard_normal((Hq, nq, d))
        pos = np.arange(T - nq, T)
        o = attention.attend_positions(q, pos, k, v)
        ob = np.array(brute.attend_brute(q.tolist(), pos.tolist(), k.tolist(), v.tolist()))
        assert np.max(np.abs(o - ob)) < 1e-12


def test_brute_force():
    check_brute_force()


# ------------------------------------------------------------------ mask and counts

def check_mask_counts():
    g = read_golden("counts.txt")
    layers, heads = 2, 2
    full = sum(layers * heads * attention.finite_score_count(attention.rect_mask(np.ones((1, n))))
               for n in (4, 5, 6, 7))
    assert full == g["score_pairs_full"][0]
    cached = layers * heads * attention.finite_score_count(attention.slot_mask(np.arange(4), 4))
    for T in (5, 6, 7):
        cached += layers * heads * attention.finite_score_count(attention.slot_mask([T - 1], T))
    assert cached == g["score_pairs_cached"][0]


def test_mask_counts():
    check_mask_counts()


def test_rect_mask_matches_slot_mask():
    """Section 2.2's mask over a right-padded prefill equals the slot form on valid rows."""
    G = np.array([[1, 1, 1, 0, 0], [1, 1, 1, 1, 1]])
    M = attention.rect_mask(G)
    for b in range(2):
        nb = int(G[b].sum())
        S = attention.slot_mask(np.arange(nb), nb)
        assert np.array_equal(M[b, :nb, :nb], S)
        assert np.all(np.isneginf(M[b, :nb, nb:]))
        assert np.all(np.isneginf(M[b, nb:, :]))


def test_no_finite_score_rejected():
    with pytest.raises(ValueError):
        attention.softmax_finite(np.array([[float("-inf"), float("-inf")]]))


# ------------------------------------------------------------------ bf16 and rotation

def check_bf16_rounding():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 20000),
        # exact ties: 1 + 2^-8 (odd neighbour below? no: 1.0 is even) and 1 + 3*2^-8
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3.3895314e38, -3.3895314e38,
                  1e-45, 0.0, -0.0, np.inf, -np.inf], dtype=np.float32),
    ]).astype(np.float32)
    ours = round_f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    assert np.isnan(round_f32_to_bf16(np.array([np.nan], dtype=np.float32)))[0]


def test_bf16_rounding():
    check_bf16_rounding()


def check_rotation():
    rng = np.random.default_rng(1)
    d, theta = 16, 10000.0
    x = rng.standard_normal((3, 40, d)).astype(np.float32)
    pos = np.arange(40) * 37
    r = rope.rotate(x, pos, theta)
    # complex-number form: (a + i b) * exp(i * p * theta^(-2k/d)), pairs (k, k + d/2)
    h = d // 2
    z = x[..., :h].astype(np.float64) + 1j * x[..., h:].astype(np.float64)
    ang = pos[:, None].astype(np.float64) * theta ** (-2.0 * np.arange(h) / d)[None, :]
    zr = z * np.exp(1j * ang)
    assert np.max(np.abs(r[..., :h] - zr.real)) < 1e-5
    assert np.max(np.abs(r[..., h:] - zr.imag)) < 1e-5
    # position 0 is the identity, bit for bit
    r0 = rope.rotate(x[:, :1], [0], theta)
    assert np.array_equal(r0.view(np.uint32), x[:, :1].view(np.uint32))
    # inner products depend only on the position difference
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, d)).astype(np.float32)
    dots = []
    for p in (5, 100, 1000):
        qa = rope.rotate(q, [p], theta).astype(np.float64)
        ka = rope.rotate(k, [p + 7], theta).astype(np.float64)
        dots.append(float((qa * ka).sum()))
    assert max(dots) - min(dots) < 1e-4


def test_rotation():
    check_rotation()


def test_rotation_disabled_is_identity():
    x = np.random.default_rng(2).standard_normal((2, 3, 4)).astype(np.float32)
    assert np.array_equal(rope.rotate(x, [0, 1, 2], 0.0), x)


# ------------------------------------------------------------------ cache model

def _model(**kw):
    cfg = dict(num_layers=1, num_kv_heads=1, head_dim=4, page_size=16, num_pages=64,
               max_seqs=4, max_pages_per_seq=16, dtype="f32", rope_theta=0.0)
    cfg.update(kw)
    return CacheModel(**cfg)


def _append(m, layer, seqs, n_tokens, start, rng, Hkv=1, d=4):
    B = len(seqs)
    n = max(n_tokens)
    K = rng.standard_normal((B, Hkv, n, d)).astype(np.float32)
    V = rng.standard_normal((B, Hkv, n, d)).astype(np.float32)
    mask = np.zeros((B, n), np.uint8)
    pos = -np.ones((B, n), np.int32)
    for b, nb in enumerate(n_tokens):
        mask[b, :nb] = 1
        pos[b, :nb] = np.arange(start[b], start[b] + nb)
    m.append(layer, seqs, K, V, mask, pos)
    return K, V


def check_cache_counts():
    g = read_golden("counts.txt")
    rng = np.random.default_rng(0)
    # section 2.8 ledger: B=1, n=12, L=2, Hkv=1, d_h=4
    m = _model(num_layers=2)
    for layer in range(2):
        _append(m, layer, [0], [12], [0], rng)
    assert m.logical_elements() == g["ledger_scalars"][0]
    # paging: 18 tokens at 16 per page -> 2 pages, 14 free slots in the last
    m = _model()
    _append(m, 0, [0], [int(g["paging_tokens"][0])], [0], rng)
    pages = m.page_table(0)
    assert len(pages) == g["paging_pages"][0]
    assert len(pages) * 16 - 18 == g["paging_free_slots"][0]
    # the tail never wastes more than P-1 slots
    for n in range(1, 70):
        m = _model(max_pages_per_seq=8)
        _append(m, 0, [0], [n], [0], rng)
        assert 0 <= len(m.page_table(0)) * 16 - n <= 15
    # Grok-1 sizing: 2 * 64 * 8192 * 8 * 128 elements of 2 bytes
    elements = 2 * 64 * 1 * 8192 * 8 * 128
    assert elements * 2 == g["grok_cache_bytes"][0] == 2 ** 31


def test_cache_counts():
    check_cache_counts()


def test_allocator_order_and_truncate():
    rng = np.random.default_rng(0)
    order = [5, 3, 9, 1, 0, 2, 4, 6, 7, 8, 10, 11]
    m = _model(num_pages=12, free_order=order)
    _append(m, 0, [1, 0], [20, 40], [0, 0], rng)     # seq 1 takes 2 pages, then seq 0 takes 3
    assert m.page_table(1) == [5, 3] and m.page_table(0) == [9, 1, 0]
    m.truncate(0, 17)                               # keeps 2 pages, frees logical page 2 (phys 0)
    assert m.page_table(0) == [9, 1] and list(m.free)[-1] == 0
    assert m.cache_length(0, 0) == 17
    m.truncate(0, 0)
    assert m.page_table(0) == [] and list(m.free)[-2:] == [9, 1]
    assert m.check() == []


def check_prefix_sharing():
    """Prefix-sharing lesson of "KV Cache 与 Prefill/Decode 推理路径": requests with
    the same first m tokens have the same per-layer K/V there, so the second
    one references the first one's blocks instead of prefilling them again; a
    shared block goes back to the pool only when no request references it; a
    fork inside a block (its 18-token, two-block example) needs the block
    copied before either branch writes into it."""
    rng = np.random.default_rng(11)
    m = _model(num_layers=2, num_pages=10, max_seqs=3)
    for layer in range(2):
        _append(m, layer, [0], [18], [0], rng)
    assert m.page_table(0) == [0, 1]
    m.fork(0, 1, 18)
    assert m.page_table(1) == [0, 1], "the fork references the prefix blocks"
    assert len(m.free) == 8 and m.ref[:2] == [2, 2] and m.copies == []
    for layer in range(2):
        assert np.array_equal(m.keys(1, layer), m.keys(0, layer))
        assert np.array_equal(m.values(1, layer), m.values(0, layer))
    # branch 1 writes slot 18, inside shared block 1: copied first, to the next free page
    suffix = []
    for layer in range(2):
        suffix.append(_append(m, layer, [1], [3], [18], rng))
    assert m.page_table(1) == [0, 2] and m.copies == [(1, 2)]
    assert m.ref[:3] == [2, 1, 1]
    # branch 0 writes slot 18 too: block 1 has one reference left, written in place
    for layer in range(2):
        _append(m, layer, [0], [5], [18], rng)
    assert m.page_table(0) == [0, 1] and m.copies == [(1, 2)]
    for layer in range(2):
        assert np.array_equal(m.keys(1, layer)[:, :18], m.keys(0, layer)[:, :18])
        assert np.array_equal(m.keys(1, layer)[:, 18:], suffix[layer][0][0])
        assert np.array_equal(m.values(1, layer)[:, 18:], suffix[layer][1][0])
    assert m.check() == []
    # releasing branch 0 frees only its own block; the shared block 0 stays
    m.truncate(0, 0)
    assert list(m.free)[-1] == 1 and 0 not in m.free and m.ref[0] == 1
    m.truncate(1, 0)
    assert list(m.free)[-2:] == [0, 2] and m.check() == []
    # a fork at a block boundary shares whole blocks only and needs no copy
    for layer in range(2):
        _append(m, layer, [2], [32], [0], rng)
    m.fork(2, 0, 16)
    for layer in range(2):
        _append(m, layer, [0], [4], [16], rng)
    assert len(m.page_table(0)) == 2 and m.page_table(0)[0] == m.page_table(2)[0]
    assert m.copies == [(1, 2)] and m.check() == []


def check_fork_then_suffix_equals_full_prefill():
    """A forked request that prefills only its own suffix gets the outputs a full
    prefill of the whole sequence gets (position i depends on tokens 0..i only)."""
    rng = np.random.default_rng(12)
    Hq, Hkv, d, n, mfork = 4, 2, 8, 40, 21
    Q = rng.standard_normal((1, Hq, n, d)).astype(np.float32)
    K = rng.standard_normal((1, Hkv, n, d)).astype(np.float32)
    V = rng.standard_normal((1, Hkv, n, d)).astype(np.float32)
    pos = np.arange(n)[None].astype(np.int32)
    full = _model(num_kv_heads=Hkv, head_dim=d, rope_theta=1e4, max_seqs=3)
    O_full = full.prefill(0, [0], Q, K, V, np.ones((1, n), np.uint8), pos)
    m = _model(num_kv_heads=Hkv, head_dim=d, rope_theta=1e4, max_seqs=3)
    other = rng.standard_normal((1, Hkv, n, d)).astype(np.float32)
    head = np.ones((1, n), np.uint8)
    head[:, mfork:] = 0
    m.prefill(0, [0], Q, K, V, head, pos)                    # the shared prefix, as request 0
    tail = np.concatenate([K[:, :, :mfork], other[:, :, mfork:]], axis=2)
    m.append(0, [0], tail, tail, 1 - head, pos)              # request 0 continues differently
    m.fork(0, 1, mfork)
    O_sfx = m.prefill(0, [1], Q, K, V, 1 - head, pos)
    assert np.allclose(O_sfx[:, :, mfork:], O_full[:, :, mfork:], rtol=0, atol=1e-12)
    assert m.check() == []


def check_padding_placement_invariance():
    """Section 2.2 (padding never becomes visible history) and section 2.11 (an
    unmasked padding key makes a sample's result depend on the batch layout):
    the same valid tokens, right-padded, left-padded or with holes between
    them, give the same cache and the same outputs on their rows, and zeros on
    every padding row."""
    rng = np.random.default_rng(13)
    Hq, Hkv, d, nv, n = 4, 2, 8, 9, 16
    Qv = rng.standard_normal((Hq, nv, d)).astype(np.float32)
    Kv = rng.standard_normal((Hkv, nv, d)).astype(np.float32)
    Vv = rng.standard_normal((Hkv, nv, d)).astype(np.float32)
    layouts = [list(range(nv)), list(range(n - nv, n)), [0, 2, 3, 6, 7, 8, 11, 14, 15]]
    outs, caches = [], []
    for rows in layouts:
        Q = rng.standard_normal((1, Hq, n, d)).astype(np.float32) * 50   # padding: any values
        K = rng.standard_normal((1, Hkv, n, d)).astype(np.float32) * 50
        V = rng.standard_normal((1, Hkv, n, d)).astype(np.float32) * 50
        Q[0][:, rows], K[0][:, rows], V[0][:, rows] = Qv, Kv, Vv
        mask = np.zeros((1, n), np.uint8)
        mask[0, rows] = 1
        pos = np.full((1, n), -7, np.int32)
        pos[0, rows] = np.arange(3, 3 + nv)
        m = _model(num_kv_heads=Hkv, head_dim=d, rope_theta=1e4)
        _append(m, 0, [0], [3], [0], rng, Hkv=Hkv, d=d)
        m.K[(0, 0)][:] = 0.25                                       # the same 3-token prefix everywhere
        m.V[(0, 0)][:] = -0.5
        O = m.prefill(0, [0], Q, K, V, mask, pos)
        pad = np.ones(n, bool)
        pad[rows] = False
        assert np.all(O[0][:, pad] == 0.0)
        outs.append(O[0][:, rows])
        caches.append((m.keys(0, 0).copy(), m.values(0, 0).copy()))
    for o, (k, v) in zip(outs[1:], caches[1:]):
        assert np.array_equal(o, outs[0])
        assert np.array_equal(k, caches[0][0]) and np.array_equal(v, caches[0][1])


def check_sliding_window():
    """Sliding-window lesson of "KV Cache 与 Prefill/Decode 推理路径": the window
    holds the latest W positions, the current one included (its W = 4 example:
    the 4th token reads tokens 1..4).  Pinned by special cases (W >= T is plain
    causal attention; W = 1 returns the query's own value), by slicing the
    history instead of masking it, and by pure-Python loops."""
    import math
    rng = np.random.default_rng(14)
    Hq, Hkv, d, T = 4, 2, 8, 12
    q = rng.standard_normal((Hq, T, d))
    k = rng.standard_normal((Hkv, T, d))
    v = rng.standard_normal((Hkv, T, d))
    pos = np.arange(T)
    full = attention.attend_positions(q, pos, k, v)
    assert np.array_equal(attention.attend_positions(q, pos, k, v, window=T), full)
    own = attention.attend_positions(q, pos, k, v, window=1)
    for h in range(Hq):
        assert np.allclose(own[h], v[attention.head_map(h, Hq, Hkv)], rtol=0, atol=1e-15)
    W = 4
    win = attention.attend_positions(q, pos, k, v, window=W)
    for p in range(T):
        lo = max(0, p - W + 1)
        sl = attention.attend(q[:, p:p + 1], k[:, lo:p + 1], v[:, lo:p + 1], np.zeros((1, p + 1 - lo)))
        assert np.allclose(win[:, p:p + 1], sl, rtol=0, atol=1e-12)
        for h in range(Hq):                          # loops and math.fsum
            g = (h * Hkv) // Hq
            sc = [math.fsum(q[h, p, e] * k[g, j, e] for e in range(d)) / math.sqrt(d) for j in range(lo, p + 1)]
            mx = max(sc)
            ex = [math.exp(x - mx) for x in sc]
            z = math.fsum(ex)
            for e in range(d):
                o = math.fsum(ex[i] * v[g, lo + i, e] for i in range(len(ex))) / z
                assert abs(o - win[h, p, e]) <= 1e-12


def check_ring_cache():
    """Ring of R pages for a window W: logical page L in entry L mod R, reused in
    place once the ring is full; a call whose window and new tokens need more
    than R pages is refused; a ring sequence is only released or kept."""
    rng = np.random.default_rng(15)
    m = _model(num_pages=8, max_pages_per_seq=3, window=20, max_position=256)
    _append(m, 0, [0], [48], [0], rng)
    assert m.page_table(0) == [0, 1, 2] and len(m.free) == 5
    _append(m, 0, [0], [1], [48], rng)              # logical page 3 reuses entry 0 (page 0)
    assert m.page_table(0) == [0, 1, 2] and len(m.free) == 5
    assert m.resident_from(0, 0) == 16
    with pytest.raises(OracleError) as e:            # keys 30..88 span logical pages 1..5
        _append(m, 0, [0], [40], [49], rng)
    assert e.value.code == "OUT_OF_PAGES"
    _append(m, 0, [0], [14], [49], rng)
    assert m.check() == [] and m.cache_length(0, 0) == 63
    with pytest.raises(OracleError) as e:
        m.truncate(0, 50)
    assert e.value.code == "UNSUPPORTED"
    with pytest.raises(OracleError) as e:
        m.fork(0, 1, 10)
    assert e.value.code == "UNSUPPORTED"
    assert m.resident_from(0, 0) == 16                # logical pages 1..3 remain
    with pytest.raises(OracleError) as e:            # position 30's window starts at 11 < 16
        m.prefill_rows(0, 0, np.zeros((1, 1, 4), np.float32), [30])
    assert e.value.code == "POSITION"
    m.prefill_rows(0, 0, np.zeros((1, 1, 4), np.float32), [35])
    short = _model(num_pages=8, max_pages_per_seq=3, window=20, max_position=256)
    _append(short, 0, [0], [10], [0], rng)
    short.prefill_rows(0, 0, np.zeros((1, 1, 4), np.float32), [5])   # window starts before 0: nothing lost
    m.truncate(0, 0)
    assert m.page_table(0) == [] and list(m.free)[-3:] == [0, 1, 2] and m.check() == []
    with pytest.raises(OracleError) as e:
        _model(max_pages_per_seq=2, window=20)        # a window of 20 may span 3 pages
    assert e.value.code == "UNSUPPORTED"


def test_sliding_window():
    check_sliding_window()
    check_ring_cache()


def test_padding_placement_invariance():
    check_padding_placement_invariance()


def test_prefix_sharing():
    check_prefix_sharing()
    check_fork_then_suffix_equals_full_prefill()


def test_remap_keeps_logical_content():
    rng = np.random.default_rng(0)
    m = _model(num_pages=8)
    _append(m, 0, [0], [30], [0], rng)
    k_before = m.keys(0, 0).copy()
    src = m.page_table(0)
    m.remap(src, [6, 7])
    assert m.page_table(0) == [6, 7]
    assert np.array_equal(m.keys(0, 0), k_before)
    assert list(m.free)[-2:] == src
    with pytest.raises(OracleError) as e:
        m.remap([6], [7])                            # 7 is in use
    assert e.value.code == "CACHE"


def test_failure_table():
    """Section 2.11 rows that a call can detect, each rejected before any change."""
    rng = np.random.default_rng(0)
    m = _model(num_layers=2)
    _append(m, 0, [0], [5], [0], rng)
    K = np.zeros((1, 1, 3, 4), np.float32)
    # position ids restarting at 0 after reuse
    with pytest.raises(OracleError) as e:
        m.append(0, [0], K, K, np.ones((1, 3), np.uint8), np.array([[0, 1, 2]]))
    assert e.value.code == "POSITION"
    assert m.cache_length(0, 0) == 5
    # validity entries outside {0, 1} (section 2.2)
    with pytest.raises(OracleError) as e:
        m.append(0, [0], K, K, np.array([[1, 2, 1]], np.uint8), np.array([[5, 6, 7]]))
    assert e.value.code == "MASK"
    # a hole: the valid tokens still take consecutive positions, so 5, 6 (not 5, 7)
    with pytest.raises(OracleError) as e:
        m.append(0, [0], K, K, np.array([[1, 0, 1]], np.uint8), np.array([[5, 6, 7]]))
    assert e.value.code == "POSITION"
    # Hkv must divide Hq
    m2 = _model(num_kv_heads=2)
    Q = np.zeros((1, 3, 2, 4), np.float32)
    K2 = np.zeros((1, 2, 2, 4), np.float32)
    with pytest.raises(OracleError) as e:
        m2.prefill(0, [0], Q, K2, K2, np.ones((1, 2), np.uint8), np.array([[0, 1]]))
    assert e.value.code == "SHAPE"
    # decode with a valid length that differs from the cache length
    q = np.zeros((1, 2, 1, 4), np.float32)
    with pytest.raises(OracleError) as e:
        m.decode(0, [0], q, [4])
    assert e.value.code == "CACHE"
    # the pool runs out: nothing changes
    m3 = _model(num_pages=2)
    with pytest.raises(OracleError) as e:
        _append(m3, 0, [0, 1], [20, 20], [0, 0], rng)
    assert e.value.code == "OUT_OF_PAGES" and m3.page_table(0) == [] and len(m3.free) == 2
    # layer lengths differ across layers -> the invariant check reports it
    assert any("differ" in s for s in m.check())


def test_padding_and_batch_composition():
    """Padding (even NaN) never reaches valid outputs; batch mates never change a row."""
    rng = np.random.default_rng(4)
    Hq, Hkv, d, n = 4, 2, 8, 6
    lengths = [6, 3, 0]
    Q = rng.standard_normal((3, Hq, n, d)).astype(np.float32)
    K = rng.standard_normal((3, Hkv, n, d)).astype(np.float32)
    V = rng.standard_normal((3, Hkv, n, d)).astype(np.float32)
    mask = np.zeros((3, n), np.uint8)
    pos = -np.ones((3, n), np.int64)
    for b, nb in enumerate(lengths):
        mask[b, :nb] = 1
        pos[b, :nb] = np.arange(nb)
    Qp, Kp, Vp = Q.copy(), K.copy(), V.copy()
    for b, nb in enumerate(lengths):
        Qp[b, :, nb:] = Kp[b, :, nb:] = Vp[b, :, nb:] = np.nan
    kw = dict(num_layers=1, num_kv_heads=Hkv, head_dim=d, page_size=16, num_pages=8,
              max_seqs=3, max_pages_per_seq=2, dtype="f32", rope_theta=100.0)
    o = CacheModel(**kw).prefill(0, [0, 1, 2], Q, K, V, mask, pos)
    op = CacheModel(**kw).prefill(0, [0, 1, 2], Qp, Kp, Vp, mask, pos)
    assert np.array_equal(o, op) and not np.isnan(op).any()
    assert np.all(op[1, :, 3:] == 0) and np.all(op[2] == 0)
    alone = CacheModel(**kw).prefill(0, [1], Q[1:2, :, :3], K[1:2, :, :3], V[1:2, :, :3],
                                     mask[1:2, :3], pos[1:2, :3])
    assert np.array_equal(alone[0], o[1, :, :3])


def test_cached_decode_equals_full_recompute():
    """The toy's check: every cached step equals a full recompute within 1e-12."""
    import workloads
    pre, steps = workloads.tiny()
    kw = dict(num_layers=1, num_kv_heads=1, head_dim=4, page_size=16, num_pages=4,
              max_seqs=1, max_pages_per_seq=4, dtype="f32", rope_theta=0.0)
    m = CacheModel(**kw)
    m.prefill(0, [0], pre.Q.numpy(), pre.K.numpy(), pre.V.numpy(), pre.mask.numpy(), pre.positions.numpy())
    Qs, Ks, Vs = [pre.Q.numpy()], [pre.K.numpy()], [pre.V.numpy()]
    for t, st in enumerate(steps):
        T = 4 + t + 1
        one = np.ones((1, 1), np.uint8)
        m.append(0, [0], st.k.numpy(), st.v.numpy(), one, np.array([[T - 1]]))
        o = m.decode(0, [0], st.q.numpy(), [T])
        Qs.append(st.q.numpy()); Ks.append(st.k.numpy()); Vs.append(st.v.numpy())
        full = CacheModel(**kw).prefill(0, [0], np.concatenate(Qs, 2), np.concatenate(Ks, 2),
                                        np.concatenate(Vs, 2), np.ones((1, T), np.uint8),
                                        np.arange(T)[None])
        assert np.max(np.abs(o[0, :, 0] - full[0, :, T - 1])) < 1e-12


def test_prefix_unchanged_by_suffix_edit():
    """Edit at m: prefix outputs and prefix cache stay exactly as they were."""
    rng = np.random.default_rng(9)
    Hq, Hkv, d, n, m_edit = 4, 2, 8, 40, 23
    kw = dict(num_layers=1, num_kv_heads=Hkv, head_dim=d, page_size=16, num_pages=8,
              max_seqs=1, max_pages_per_seq=4, dtype="bf16", rope_theta=1e4)
    r = lambda *s: round_f32_to_bf16(rng.standard_normal(s).astype(np.float32))
    Q, K, V = r(1, Hq, n, d), r(1, Hkv, n, d), r(1, Hkv, n, d)
    model = CacheModel(**kw)
    O = model.prefill(0, [0], Q, K, V, np.ones((1, n), np.uint8), np.arange(n)[None])
    k_prefix = model.keys(0, 0)[:, :m_edit].copy()
    model.truncate(0, m_edit)
    Q2, K2, V2 = r(1, Hq, n - m_edit, d), r(1, Hkv, n - m_edit, d), r(1, Hkv, n - m_edit, d)
    O2 = model.prefill(0, [0], Q2, K2, V2, np.ones((1, n - m_edit), np.uint8),
                       np.arange(m_edit, n)[None])
    assert np.array_equal(model.keys(0, 0)[:, :m_edit], k_prefix)
    # the edited sequence from scratch: prefix rows equal, suffix rows equal the re-prefill
    Qf, Kf, Vf = (np.concatenate([a[:, :, :m_edit], b], 2) for a, b in ((Q, Q2), (K, K2), (V, V2)))
    Of = CacheModel(**kw).prefill(0, [0], Qf, Kf, Vf, np.ones((1, n), np.uint8), np.arange(n)[None])
    assert np.array_equal(Of[:, :, :m_edit], O[:, :, :m_edit])
    assert np.max(np.abs(Of[:, :, m_edit:] - O2)) < 1e-12
