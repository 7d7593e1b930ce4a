"""GPU parity of sliding-window attention over ring caches.

A cache created with window W attends each query at position p to the keys
p-W+1..p, and holds each sequence in a ring of max_pages_per_seq pages (logical
page L in table entry L mod R).  Prefill chunks, decode steps, verify chunks on
the split-T kernel and queries inside the cache are compared with the float64
oracle; the resident part of the cache and the block tables bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from harness import Pair, as_f32, compare_rows

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_gqa_attention_attn_amd  # noqa: F401  (fails loudly if the library is missing)


def _ring_pages(win, chunk):
    return -(-win // 16) + 1 + -(-chunk // 16)


def _chunk(pair, layer, ids, shape, seed, lengths, starts, workspace=None, check=True):
    inp = W.prefill_inputs(shape, seed, lengths=lengths, start=starts, poison_padding=True)
    O, ref = pair.prefill(layer, ids, inp.Q, inp.K, inp.V, inp.mask, inp.positions, workspace=workspace,
                          oracle=check)
    if check:
        valid = inp.mask.numpy().astype(bool)[:, None, :].repeat(shape.Hq, 1)
        compare_rows(O, ref, shape.dtype, rows_mask=valid)
        assert np.all(as_f32(O)[~valid] == 0.0)


@pytest.mark.parametrize("win", [1, 37, 100, 300])
@pytest.mark.parametrize("dtype,Hq,Hkv,d", [(torch.bfloat16, 32, 8, 128), (torch.bfloat16, 8, 2, 64),
                                            (torch.float32, 4, 2, 32)])
def test_window_prefill_and_decode(dtype, Hq, Hkv, d, win):
    """Three sequences prefilled in ragged chunks of up to 160 tokens until the
    ring has wrapped, then fused and unfused decode steps."""
    say(f"case: window {win}, {dtype} Hq={Hq} Hkv={Hkv} d={d}")
    chunk = 160
    R = _ring_pages(win, chunk)
    pair = Pair(1, Hkv, d, 3 * R + 4, 3, R, dtype, 1e4, max_position=4096,
                free_order=W.page_order(3 * R + 4, 41), window=win)
    pair.gpu.k_pool.fill_(float("nan"))
    pair.gpu.v_pool.fill_(float("nan"))
    ids = [0, 1, 2]
    lens = [0, 0, 0]
    rng = np.random.default_rng(42)
    for rnd in range(5):
        add = [int(x) for x in rng.integers(1, chunk + 1, size=3)]
        add[rnd % 3] = chunk
        shape = W.AttnShape(B=3, n=max(add), Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, theta=1e4)
        _chunk(pair, 0, ids, shape, 500 + rnd, add, lens)
        lens = [a + b for a, b in zip(lens, add)]
    pair.check_cache(ids)
    assert max(lens) > R * 16 or win >= 300, "the ring should have wrapped"
    dshape = W.AttnShape(B=3, n=1, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, theta=1e4)
    for step in range(3):
        o, r = pair.step(0, ids, W.decode_step_inputs(dshape, 520, step))
        compare_rows(o, r, dtype)
        o, r = pair.step_fused(0, ids, W.decode_step_inputs(dshape, 530, step))
        compare_rows(o, r, dtype)
    pair.check_cache(ids)


@pytest.mark.parametrize("win", [1, 5, 100])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (24, 8)])
def test_window_odd_group_sizes(Hq, Hkv, win):
    """Odd Hq/Hkv (MHA, three heads per group) takes 128-token query tiles, whose
    last rows can start their windows two key tiles after the first row's.  A
    256-token chunk at position 0, then one of 200 at 256 and one of 130 at 456:
    the second query tile of each chunk has rows whose window lies wholly in the
    third key tile its workgroup reads."""
    say(f"case: window {win}, odd group Hq={Hq} Hkv={Hkv}, 128-token query tiles")
    d = 128
    chunks = [256, 200, 130]
    R = _ring_pages(win, max(chunks)) + 1
    pair = Pair(1, Hkv, d, R + 4, 1, R, torch.bfloat16, 1e4, max_position=1024,
                free_order=W.page_order(R + 4, 43), window=win)
    pair.gpu.k_pool.fill_(float("nan"))
    pair.gpu.v_pool.fill_(float("nan"))
    c = 0
    for i, n in enumerate(chunks):
        shape = W.AttnShape(B=1, n=n, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=1e4)
        _chunk(pair, 0, [0], shape, 560 + i, [n], [c])
        c += n
    pair.check_cache([0])


@pytest.mark.parametrize("win", [1, 5, 100])
def test_window_odd_group_large_negative_logits(win):
    """Every score of every row far below zero (q close to -4u, k close to 4u for
    a fixed u, no rotation: logits near -180): the softmax must still be exact
    for rows whose window starts two key tiles after their workgroup's first
    row, where a reference that misses the row's keys would underflow every
    probability."""
    say(f"case: window {win}, Hq=Hkv=8, all logits near -180")
    Hq = Hkv = 8
    d, n = 128, 256
    R = _ring_pages(win, n) + 1
    pair = Pair(1, Hkv, d, R + 4, 1, R, torch.bfloat16, 0.0, max_position=1024, window=win)
    u = W.normal((1, 1, 1, d), 580, torch.float32)
    Q = (-4.0 * u + 0.1 * W.normal((1, Hq, n, d), 581, torch.float32)).to(torch.bfloat16)
    K = (4.0 * u + 0.1 * W.normal((1, Hkv, n, d), 582, torch.float32)).to(torch.bfloat16)
    V = W.normal((1, Hkv, n, d), 583, torch.bfloat16)
    mask = torch.ones((1, n), dtype=torch.uint8)
    pos = torch.arange(n, dtype=torch.int32)[None]
    O, ref = pair.prefill(0, [0], Q, K, V, mask, pos)
    compare_rows(O, ref, torch.bfloat16)
    pair.check_cache([0])


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (8, 8)])
def test_window_prefill_second_pass_on_score_overflow(Hq, Hkv):
    """Window 100: one key (position 150) whose score dwarfs every other, seen
    by rows 150..249 only.  Its probability against the tile reference passes
    2^64, so the windowed kernel takes its exact-maximum pass, which must keep
    the window's lower edge: rows 160..249 of the pointing heads return that
    key's value, rows 250.. do not see it.  64- and 128-token query tiles."""
    win, n, d = 100, 300, 128
    G = Hq // Hkv
    say(f"case: window {win}, Hq={Hq} Hkv={Hkv}, a spike key at 150 (exact-maximum pass)")
    shape = W.AttnShape(B=1, n=n, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=0.0)
    inp = W.prefill_inputs(shape, 905)
    direction = torch.zeros(d)
    direction[3] = 1.0
    inp.K[0, 0, 150] = (40.0 * direction).to(torch.bfloat16)
    inp.Q[0, :G, 160:] = (40.0 * direction).to(torch.bfloat16)
    R = _ring_pages(win, n) + 1
    pair = Pair(1, Hkv, d, R + 4, 1, R, torch.bfloat16, 0.0, max_position=1024, window=win)
    O, ref = pair.prefill(0, [0], inp.Q, inp.K, inp.V, inp.mask, inp.positions)
    compare_rows(O, ref, torch.bfloat16)
    o = O.float().cpu()
    for h in range(G):
        assert torch.allclose(o[0, h, 200], inp.V[0, 0, 150].float(), atol=1e-2), "row 200 must return the spike's value"
        assert not torch.allclose(o[0, h, 260], inp.V[0, 0, 150].float(), atol=1e-1), "row 260 is past the spike's window"
    pair.check_cache([0])


def test_window_long_ring_many_wraps():
    """One sequence, W = 512 on a 50-page ring: 4096 prompt tokens in chunks of
    256, then 64 decode steps, the ring wrapping five times."""
    say("case: W=512, 50-page ring, 4096 tokens in 256-token chunks + 64 decode steps")
    Hq, Hkv, d, win = 32, 8, 128, 512
    pair = Pair(1, Hkv, d, 56, 1, 50, torch.bfloat16, 5e5, max_position=8192, window=win)
    shape = W.AttnShape(B=1, n=256, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=5e5)
    for c in range(16):
        _chunk(pair, 0, [0], shape, 600 + c, [256], [256 * c], check=c in (0, 1, 2, 9, 15))
    pair.check_cache([0])
    dshape = W.AttnShape(B=1, n=1, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=5e5)
    for step in range(64):
        o, r = pair.step_fused(0, [0], W.decode_step_inputs(dshape, 640, step))
        compare_rows(o, r, torch.bfloat16)
    pair.check_cache([0])


def test_window_verify_chunks_and_rows_inside_the_ring():
    """Short chunks on the split-T kernel with a window (several splits), and
    gqa_attention on positions whose window the ring still holds."""
    import causal_gqa_attention_attn_amd as lib
    say("case: W=700 ring, 8-token verify chunks with a workspace; rows inside the ring")
    Hq, Hkv, d, win = 32, 8, 128, 700
    R = _ring_pages(win, 512)
    pair = Pair(1, Hkv, d, 2 * R + 4, 2, R, torch.bfloat16, 1e4, max_position=8192, window=win)
    ids = [0, 1]
    shape = W.AttnShape(B=2, n=512, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=1e4)
    lens = [0, 0]
    for c in range(5):
        add = [512, 300]
        _chunk(pair, 0, ids, shape, 700 + c, add, lens, check=False)
        lens = [a + b for a, b in zip(lens, add)]
    ws = pair.chunk_workspace(2, Hq, 8)
    cshape = W.AttnShape(B=2, n=8, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=1e4)
    for r in range(3):
        _chunk(pair, 0, ids, cshape, 720 + r, [8, 5], lens, workspace=ws)
        lens = [lens[0] + 8, lens[1] + 5]
    pair.check_cache(ids)
    # rows inside the ring: the last 100 positions of sequence 0
    n0 = lens[0]
    rows = list(range(n0 - 100, n0))
    Qm = W.normal((1, Hq, 100, d), 730, torch.bfloat16)
    Om = torch.full((1, Hq, 100, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lib.gqa_attention(pair.gpu.handle, 0, [0], Qm.cuda(), torch.ones((1, 100), dtype=torch.uint8),
                      torch.tensor([rows], dtype=torch.int32), Om)
    torch.cuda.synchronize()
    ref = pair.ref.prefill_rows(0, 0, as_f32(Qm[0]), rows)
    compare_rows(Om[0], ref, torch.bfloat16)
    # a query whose window starts before what the ring holds
    first = pair.ref.resident_from(0, 0)
    bad = first + win - 2
    with pytest.raises(lib.GqaError) as e:
        lib.gqa_attention(pair.gpu.handle, 0, [0], Qm[:, :, :1].cuda(), torch.ones((1, 1), dtype=torch.uint8),
                          torch.tensor([[bad]], dtype=torch.int32), Om[:, :, :1])
    assert e.value.name == "POSITION"


def test_window_rejections_match_oracle():
    """Ring rules: a chunk too long for the ring, a mid-sequence truncate, a fork."""
    import causal_gqa_attention_attn_amd as lib
    say("case: ring rejections")
    pair = Pair(1, 2, 64, 16, 2, 4, torch.bfloat16, 1e4, max_position=1024, window=40)
    shape = W.AttnShape(B=1, n=30, Hq=4, Hkv=2, d=64, dtype=torch.bfloat16, theta=1e4)
    _chunk(pair, 0, [0], shape, 800, [30], [0])
    big = W.prefill_inputs(W.AttnShape(B=1, n=60, Hq=4, Hkv=2, d=64, dtype=torch.bfloat16, theta=1e4), 801,
                           start=30)
    with pytest.raises(lib.GqaError) as e:
        lib.kv_cache_append(pair.gpu.handle, 0, [0], big.K.cuda(), big.V.cuda(), big.mask, big.positions)
    assert e.value.name == "OUT_OF_PAGES"
    with pytest.raises(Exception) as eo:
        pair.ref.append(0, [0], as_f32(big.K), as_f32(big.V), big.mask.numpy(), big.positions.numpy())
    assert eo.value.code == "OUT_OF_PAGES"
    for call, code in [(lambda: lib.kv_cache_truncate(pair.gpu.handle, 0, 10), "UNSUPPORTED"),
                       (lambda: lib.kv_cache_fork(pair.gpu.handle, 0, 1, 10), "UNSUPPORTED")]:
        with pytest.raises(lib.GqaError) as e:
            call()
        assert e.value.name == code
    pair.check_cache([0])
    pair.truncate(0, 0)
    pair.check_cache([0])
