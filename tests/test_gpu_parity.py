"""GPU parity: the HIP library through its C ABI against the float64 oracle.

Cache contents and block tables are compared bit for bit, outputs within
1e-5 absolute (float32) or 2e-2 of the row maximum (bfloat16).  Small shapes
span several tiles and ragged tails; the full-size shapes (the Llama-3-8B- and
Grok-1-shaped prefills, the 64-sequence serving decode, the 16-sequence edit)
are checked on every output row, with the oracle's rows spread over a thread
pool.
"""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from concurrent.futures import ThreadPoolExecutor

from threadpoolctl import threadpool_limits

from harness import Pair, as_f32, compare_rows, gather, k_view, oracle_rows, oracle_workers, v_view
from test_oracle_pins import read_golden

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_gqa_attention_attn_amd  # noqa: F401  (fails loudly if the library is missing)


# ------------------------------------------------------------------ tiny / worked example

def test_worked_example_fp32():
    say("case: worked 2-D example, fp32, Hq=1/2, Hkv=1")
    g = read_golden("worked_2d.txt")
    for Hq in (1, 2):
        pair = Pair(1, 1, 2, 4, 1, 2, torch.float32, 0.0)
        Q = torch.tensor([[1.0, 0.0], [1.0, 0.0]]).expand(1, Hq, 2, 2).contiguous()
        K = torch.tensor([[[[1.0, 0.0], [0.0, 1.0]]]])
        V = torch.tensor([[[[10.0, 0.0], [0.0, 20.0]]]])
        mask = torch.ones((1, 2), dtype=torch.uint8)
        pos = torch.tensor([[0, 1]], dtype=torch.int32)
        O, ref = pair.prefill(0, [0], Q, K, V, mask, pos)
        o = as_f32(O)
        for h in range(Hq):
            assert o[0, h, 0, 0] == 10.0 and o[0, h, 0, 1] == 0.0
            o1, o2, tol = g["output_both"]
            assert abs(o[0, h, 1, 0] - o1) <= tol and abs(o[0, h, 1, 1] - o2) <= tol
        compare_rows(O, ref, torch.float32)
        pair.check_cache([0])


def test_tiny_fp32_prefill_and_decode():
    say("case: tiny fp32 B=1 n=4 Hq=2 Hkv=1 d=4, 3 decode steps")
    pre, steps = W.tiny()
    pair = Pair(1, 1, 4, 4, 1, 4, torch.float32, 0.0)
    O, ref = pair.prefill(0, [0], pre.Q, pre.K, pre.V, pre.mask, pre.positions)
    compare_rows(O, ref, torch.float32)
    pair.check_cache([0])
    for st in steps:
        o, r = pair.step(0, [0], st)
        compare_rows(o, r, torch.float32)
    pair.check_cache([0])


def test_fp32_rotated_ragged():
    say("case: fp32 with rotation, ragged, Hq=6 Hkv=2 d=32")
    shape = W.AttnShape(B=3, n=37, Hq=6, Hkv=2, d=32, dtype=torch.float32, theta=1e4)
    inp = W.prefill_inputs(shape, 77, lengths=[37, 20, 1])
    pair = Pair(1, 2, 32, 16, 3, 4, torch.float32, 1e4)
    O, ref = pair.prefill(0, [0, 1, 2], inp.Q, inp.K, inp.V, inp.mask, inp.positions)
    compare_rows(O, ref, torch.float32)
    pair.check_cache([0, 1, 2])
    for t in range(3):
        o, r = pair.step(0, [0, 1, 2], W.decode_step_inputs(shape, 77, t))
        compare_rows(o, r, torch.float32)


# ------------------------------------------------------------------ bf16 prefill + decode

@pytest.mark.parametrize("poison", [False, True])
def test_ragged_bf16(poison):
    say(f"case: ragged bf16 B=4 n=128 Hq=8 Hkv=2 d=64 poison={poison}, 16 decode steps")
    inp = W.ragged(poison_padding=poison)
    pair = Pair(1, 2, 64, 64, 4, 16, torch.bfloat16, 1e4)
    O, ref = pair.prefill(0, [0, 1, 2, 3], inp.Q, inp.K, inp.V, inp.mask, inp.positions)
    valid = inp.mask.numpy().astype(bool)[:, None, :].repeat(8, 1)
    compare_rows(O, ref, torch.bfloat16, rows_mask=valid)
    assert torch.all(O.float().cpu()[~torch.from_numpy(valid)] == 0), "padding rows must be exact zeros"
    pair.check_cache([0, 1, 2, 3])
    for t in range(16):
        o, r = pair.step(0, [0, 1, 2, 3], W.decode_step_inputs(inp.shape, 1002, t))
        compare_rows(o, r, torch.bfloat16)
    pair.check_cache([0, 1, 2, 3])


GQA_SHAPES = [
    # Hq, Hkv, d, lengths, theta
    (8, 2, 64, [130, 77, 1], 1e4),
    (32, 8, 128, [200, 64, 33], 5e5),
    (48, 8, 128, [150, 97], 1e4),
    (8, 8, 128, [70, 5], 1e4),
    (16, 1, 128, [100, 31], 1e4),      # 16 query heads per KV head: two head chunks in prefill
    (12, 1, 64, [90, 129], 1e4),       # 12 per group: a chunk of 8 and one of 4
    (4, 2, 128, [300], 0.0),           # no rotation
]


@pytest.mark.parametrize("Hq,Hkv,d,lengths,theta", GQA_SHAPES)
def test_gqa_shapes_bf16(Hq, Hkv, d, lengths, theta):
    say(f"case: bf16 Hq={Hq} Hkv={Hkv} d={d} lengths={lengths} theta={theta}")
    B, n = len(lengths), max(lengths)
    shape = W.AttnShape(B=B, n=n, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=theta)
    inp = W.prefill_inputs(shape, 4242 + Hq + d, lengths=lengths)
    order = W.page_order(64, 99)
    pair = Pair(1, Hkv, d, 64, B, 24, torch.bfloat16, theta, free_order=order)
    ids = list(range(B))
    O, ref = pair.prefill(0, ids, inp.Q, inp.K, inp.V, inp.mask, inp.positions)
    valid = inp.mask.numpy().astype(bool)[:, None, :].repeat(Hq, 1)
    compare_rows(O, ref, torch.bfloat16, rows_mask=valid)
    pair.check_cache(ids)
    for t in range(3):
        o, r = pair.step(0, ids, W.decode_step_inputs(shape, 4242, t))
        compare_rows(o, r, torch.bfloat16)
    pair.check_cache(ids)


def test_incremental_prefill_and_edit():
    say("case: edit at m, truncate, re-prefill suffix; bf16 Hq=32 Hkv=8 d=128")
    n = 300
    ms = [1, 137, 299]
    B = len(ms)
    shape = W.AttnShape(B=B, n=n, Hq=32, Hkv=8, d=128, dtype=torch.bfloat16, theta=5e5)
    inp = W.prefill_inputs(shape, 31)
    pair = Pair(2, 8, 128, 128, B, 32, torch.bfloat16, 5e5, free_order=W.page_order(128, 5))
    ids = list(range(B))
    for layer in range(2):
        O, ref = pair.prefill(layer, ids, inp.Q, inp.K, inp.V, inp.mask, inp.positions)
        compare_rows(O, ref, torch.bfloat16)
    pair.check_cache(ids)
    prefix = {}
    for s, m in zip(ids, ms):
        prefix[s] = [gather(pair.gpu, s, l) for l in range(2)]
        pair.truncate(s, m)
    lens = [n - m for m in ms]
    suffix = W.prefill_inputs(W.AttnShape(B=B, n=max(lens), Hq=32, Hkv=8, d=128,
                                          dtype=torch.bfloat16, theta=5e5), 2006,
                              lengths=lens, start=ms)
    for layer in range(2):
        O, ref = pair.prefill(layer, ids, suffix.Q, suffix.K, suffix.V, suffix.mask, suffix.positions)
        valid = suffix.mask.numpy().astype(bool)[:, None, :].repeat(32, 1)
        compare_rows(O, ref, torch.bfloat16, rows_mask=valid)
    pair.check_cache(ids)
    for s, m in zip(ids, ms):
        for l in range(2):
            k, v = gather(pair.gpu, s, l)
            k0, v0 = prefix[s][l]
            assert torch.equal(k[:, :m].view(torch.int16), k0[:, :m].view(torch.int16)), "prefix K changed"
            assert torch.equal(v[:, :m].view(torch.int16), v0[:, :m].view(torch.int16)), "prefix V changed"


# ------------------------------------------------------------------ invariants

def _prefill_outputs(order, remap=False):
    shape = W.AttnShape(B=2, n=200, Hq=32, Hkv=8, d=128, dtype=torch.bfloat16, theta=5e5)
    inp = W.prefill_inputs(shape, 555, lengths=[200, 123])
    pair = Pair(1, 8, 128, 64, 2, 16, torch.bfloat16, 5e5, free_order=order)
    O, _ = pair.prefill(0, [0, 1], inp.Q, inp.K, inp.V, inp.mask, inp.positions, oracle=False)
    if remap:
        src = pair.lib.gqa_cache_page_table(pair.gpu.handle, 0)[:3]
        free_now = [p for p in range(64) if p not in set(pair.lib.gqa_cache_page_table(pair.gpu.handle, 0)
                                                         + pair.lib.gqa_cache_page_table(pair.gpu.handle, 1))]
        dst = free_now[-3:]
        pair.lib.kv_cache_remap(pair.gpu.handle, src, dst)
        pair.ref.remap(src, dst)
        pair.lib.gqa_cache_check(pair.gpu.handle)
        pair.check_cache([0, 1])
    st = W.decode_step_inputs(shape, 555, 0)
    o, _ = pair.step(0, [0, 1], st)
    return O.cpu(), o.cpu(), pair


def test_page_permutation_and_remap_invariance():
    say("case: paging invariance (identity vs permuted pool vs remapped pages)")
    O1, o1, _ = _prefill_outputs(None)
    O2, o2, _ = _prefill_outputs(W.page_order(64, 3003))
    O3, o3, _ = _prefill_outputs(W.page_order(64, 3003), remap=True)
    for a, b in ((O1, O2), (o1, o2), (o1, o3)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_batch_composition_invariance():
    say("case: a sequence's output does not depend on its batch mates")
    shape = W.AttnShape(B=3, n=150, Hq=32, Hkv=8, d=128, dtype=torch.bfloat16, theta=5e5)
    inp = W.prefill_inputs(shape, 808, lengths=[150, 40, 99], poison_padding=True)
    pair = Pair(1, 8, 128, 64, 3, 16, torch.bfloat16, 5e5)
    O, _ = pair.prefill(0, [0, 1, 2], inp.Q, inp.K, inp.V, inp.mask, inp.positions, oracle=False)
    solo = Pair(1, 8, 128, 64, 3, 16, torch.bfloat16, 5e5)
    O1, _ = solo.prefill(0, [1], inp.Q[1:2, :, :40], inp.K[1:2, :, :40], inp.V[1:2, :, :40],
                         inp.mask[1:2, :40], inp.positions[1:2, :40], oracle=False)
    assert torch.equal(O[1:2, :, :40].cpu().view(torch.int16), O1.cpu().view(torch.int16))


def test_cached_decode_equals_full_recompute_gpu():
    say("case: GPU incremental cache bytes == GPU fresh prefill cache bytes")
    shape = W.AttnShape(B=1, n=40, Hq=8, Hkv=2, d=64, dtype=torch.bfloat16, theta=1e4)
    inp = W.prefill_inputs(shape, 21)
    a = Pair(1, 2, 64, 16, 1, 8, torch.bfloat16, 1e4)
    a.prefill(0, [0], inp.Q[:, :, :30], inp.K[:, :, :30], inp.V[:, :, :30], inp.mask[:, :30],
              inp.positions[:, :30], oracle=False)
    for t in range(30, 40):
        a.append(0, [0], inp.K[:, :, t:t + 1], inp.V[:, :, t:t + 1], torch.ones((1, 1), dtype=torch.uint8),
                 torch.tensor([[t]], dtype=torch.int32))
    b = Pair(1, 2, 64, 16, 1, 8, torch.bfloat16, 1e4)
    b.prefill(0, [0], inp.Q, inp.K, inp.V, inp.mask, inp.positions, oracle=False)
    ka, va = gather(a.gpu, 0, 0)
    kb, vb = gather(b.gpu, 0, 0)
    assert torch.equal(ka.view(torch.int16), kb.view(torch.int16))
    assert torch.equal(va.view(torch.int16), vb.view(torch.int16))
    a.check_cache([0])


# ------------------------------------------------------------------ error paths on the device build

def test_errors_match_oracle_gpu():
    say("case: rejected calls return the oracle's error class and change nothing")
    import causal_gqa_attention_attn_amd as lib
    from oracle.cache_model import OracleError
    pair = Pair(1, 2, 64, 4, 2, 2, torch.bfloat16, 1e4, max_position=1000)
    shape = W.AttnShape(B=1, n=20, Hq=4, Hkv=2, d=64, dtype=torch.bfloat16, theta=1e4)
    inp = W.prefill_inputs(shape, 1)
    pair.prefill(0, [0], inp.Q, inp.K, inp.V, inp.mask, inp.positions)
    cases = {
        "restart": (inp.mask, inp.positions),
        "hole": (torch.tensor([[1, 0] + [1] * 18], dtype=torch.uint8), inp.positions + 20),
    }
    for name, (mask, pos) in cases.items():
        with pytest.raises(lib.GqaError) as e:
            pair.lib.kv_cache_append(pair.gpu.handle, 0, [0], inp.K.cuda(), inp.V.cuda(), mask, pos)
        with pytest.raises(OracleError) as r:
            pair.ref.append(0, [0], as_f32(inp.K), as_f32(inp.V), mask.numpy(), pos.numpy())
        assert e.value.name == r.value.code, name
    # the pool of 4 pages is exhausted by a second sequence of 60 tokens
    big = W.prefill_inputs(W.AttnShape(B=1, n=60, Hq=4, Hkv=2, d=64, dtype=torch.bfloat16, theta=1e4), 2)
    with pytest.raises(lib.GqaError) as e:
        pair.lib.kv_cache_append(pair.gpu.handle, 0, [1], big.K.cuda(), big.V.cuda(), big.mask, big.positions)
    assert e.value.name == "OUT_OF_PAGES"
    assert lib.gqa_cache_free_pages(pair.gpu.handle) == 2
    pair.check_cache([0, 1])
    lib.gqa_cache_check(pair.gpu.handle)


# ------------------------------------------------------------------ full sizes, every row

def _all_rows(pair, O, inp, seqs, layer=0, starts=None):
    """Every valid row of every listed sequence against the oracle (threaded
    over row blocks); returns the worst row-relative error."""
    Oc = O.cpu()
    jobs, keep = [], []
    for b in seqs:
        nb = int(inp.mask[b].sum())
        c = 0 if starts is None else starts[b]
        jobs.append((b, as_f32(inp.Q[b, :, :nb, :]), np.arange(c, c + nb)))
        keep.append(nb)
    refs = oracle_rows(pair.ref, layer, jobs)
    worst = 0.0
    for b, nb, ref in zip(seqs, keep, refs):
        _, rel = compare_rows(Oc[b, :, :nb, :], ref, torch.bfloat16)
        worst = max(worst, rel)
        assert torch.all(Oc[b, :, nb:, :] == 0), f"padding rows of sequence {b} must be written as 0"
    return worst


def test_llama_full_size():
    """Llama-3-8B-shaped prefill (B=8, n=2048, Hq=32, Hkv=8, d=128, permuted
    page pool): every output row of all 8 sequences, every cache byte and block
    table, then the 64 decode steps on all 8."""
    say("case: Llama-3-8B-shaped prefill B=8 n=2048 Hq=32 Hkv=8 d=128, permuted pages, every row, 64 decode steps")
    inp = W.llama()
    B, n = 8, 2048
    pps = n // 16 + 4
    order = W.page_order(B * pps, 3003)
    pair = Pair(1, 8, 128, B * pps, B, pps, torch.bfloat16, 5e5, free_order=order)
    ids = list(range(B))
    O, _ = pair.prefill(0, ids, inp.Q, inp.K, inp.V, inp.mask, inp.positions, oracle=False)
    worst = _all_rows(pair, O, inp, ids)
    say(f"  worst row-relative error {worst:.3e} over {B * 32 * n} rows")
    pair.check_cache(ids)
    # the 64 decode steps that follow the prefill: even steps append then decode,
    # odd steps append and decode in one launch
    for t in range(64):
        st = W.decode_step_inputs(W.LLAMA, 1003, t)
        o, r = (pair.step_fused if t % 2 else pair.step)(0, ids, st)
        compare_rows(o, r, torch.bfloat16)
    pair.check_cache(ids)
    pair.lib.gqa_workspace_status(pair.gpu.handle, pair.ws)


def test_grok_full_size():
    """Grok-1-shaped prefill (B=1, n=8192, Hq=48, Hkv=8, d=128): all 8192 x 48
    output rows and the whole cache; then a second layer of 8191 tokens, one
    appended token and a decode at T=8192."""
    say("case: Grok-1-shaped prefill B=1 n=8192 Hq=48 Hkv=8 d=128, every row; decode at T=8192")
    inp = W.grok()
    sh = W.GROK
    pps = sh.n // 16 + 4
    pair = Pair(2, sh.Hkv, sh.d, pps, 1, pps, sh.dtype, sh.theta)
    O, _ = pair.prefill(0, [0], inp.Q, inp.K, inp.V, inp.mask, inp.positions, oracle=False)
    worst = _all_rows(pair, O, inp, [0])
    say(f"  worst row-relative error {worst:.3e} over {48 * 8192} rows")
    pair.check_cache([0], invariants=False)
    # second layer holds 8191 tokens, then one appended token and a decode at T=8192
    K2 = W.normal((1, 8, 8191, 128), 7004)
    V2 = W.normal((1, 8, 8191, 128), 7005)
    m = torch.ones((1, 8191), dtype=torch.uint8)
    pair.append(1, [0], K2, V2, m, torch.arange(8191, dtype=torch.int32)[None])
    st = W.decode_step_inputs(W.GROK, 1004, 0)
    pair.append(1, [0], st.k, st.v, torch.ones((1, 1), dtype=torch.uint8), torch.tensor([[8191]], dtype=torch.int32))
    o, r = pair.decode(1, [0], st.q, [8192])
    compare_rows(o, r, torch.bfloat16)
    pair.lib.gqa_workspace_status(pair.gpu.handle, pair.ws)
    pair.check_cache([0])


def test_serving_decode_full_size():
    """Serving decode: 64 sequences with cached lengths log-uniform in
    [512, 32768] (Hq=32, Hkv=8, d=128), one batched append and one decode: the
    output of every sequence and head, every block table and every cache byte."""
    say("case: serving decode, 64 sequences, lengths log-uniform [512, 32768], Hq=32 Hkv=8 d=128, all sequences")
    import causal_gqa_attention_attn_amd as lib
    from oracle.cache_model import CacheModel
    lens = W.serving_lengths()
    B = len(lens)
    pages = sum(-(-(x + 1) // 16) for x in lens) + 8
    order = W.page_order(pages, 1005)
    cache = lib.PagedCache(1, 8, 128, pages, B, 32768 // 16 + 2, dtype=torch.bfloat16, rope_theta=5e5,
                           max_position=32770, free_list_order=order)
    n_max = max(lens)
    # fill in one batched append (batch order fixes the page assignment)
    K = torch.zeros((B, 8, n_max, 128), dtype=torch.bfloat16, device="cuda")
    V = torch.zeros_like(K)
    for b, L in enumerate(lens):
        K[b, :, :L] = W.normal_device((8, L, 128), 91000 + b)
        V[b, :, :L] = W.normal_device((8, L, 128), 92000 + b)
    mask = W.right_padded_mask(lens, n_max)
    pos = W.positions_for(mask, [0] * B)
    lib.kv_cache_append(cache.handle, 0, list(range(B)), K, V, mask, pos)
    del K, V
    st = W.decode_step_inputs(W.SERVING, 1005, 0)
    lib.kv_cache_append(cache.handle, 0, list(range(B)), st.k.cuda(), st.v.cuda(),
                        torch.ones((B, 1), dtype=torch.uint8), torch.tensor([[x] for x in lens], dtype=torch.int32))
    o = torch.empty((B, 32, 1, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(lib.gqa_workspace_size(cache.handle, B, 32), dtype=torch.uint8, device="cuda")
    lib.gqa_decode(cache.handle, 0, list(range(B)), st.q.cuda(), [x + 1 for x in lens], o, ws)
    torch.cuda.synchronize()
    lib.gqa_workspace_status(cache.handle, ws)
    # block tables: a values-free run of the oracle's allocator with the same lengths
    alloc = CacheModel(1, 1, 2, 16, pages, B, 32768 // 16 + 2, dtype="f32", free_order=order)
    z = np.zeros((B, 1, n_max, 2), np.float32)
    alloc.append(0, list(range(B)), z, z, mask.numpy(), pos.numpy())
    alloc.append(0, list(range(B)), np.zeros((B, 1, 1, 2), np.float32), np.zeros((B, 1, 1, 2), np.float32),
                 np.ones((B, 1), np.uint8), np.array([[x] for x in lens]))
    for b in range(B):
        assert lib.gqa_cache_page_table(cache.handle, b) == alloc.page_table(b)
    oc = o.cpu()
    # every sequence: its own oracle cache (rotation and bf16 rounding of its
    # keys), the decode output and the cache bytes; sequences run on a thread pool
    kv = [(W.normal_device((8, L, 128), 91000 + b).cpu(), W.normal_device((8, L, 128), 92000 + b).cpu(),
           gather(cache, b, 0)) for b, L in enumerate(lens)]

    def one(b):
        L = lens[b]
        ref = CacheModel(1, 8, 128, 16, -(-(L + 1) // 16), 1, -(-(L + 1) // 16), dtype="bf16",
                         rope_theta=5e5, max_position=32770)
        kb, vb, (gk, gv) = kv[b]
        k = torch.cat([kb, st.k[b]], dim=1)[None]
        v = torch.cat([vb, st.v[b]], dim=1)[None]
        ref.append(0, [0], as_f32(k), as_f32(v), np.ones((1, L + 1), np.uint8), np.arange(L + 1)[None])
        r = ref.decode(0, [0], as_f32(st.q[b:b + 1]), [L + 1])
        _, rel = compare_rows(oc[b:b + 1], r, torch.bfloat16)
        assert np.array_equal(gk.float().numpy().view(np.uint32), ref.keys(0, 0).view(np.uint32)), f"K of {b}"
        assert np.array_equal(gv.float().numpy().view(np.uint32), ref.values(0, 0).view(np.uint32)), f"V of {b}"
        return rel

    with threadpool_limits(1), ThreadPoolExecutor(max_workers=oracle_workers()) as ex:
        worst = max(ex.map(one, sorted(range(B), key=lambda b: -lens[b])))
    say(f"  worst row-relative error {worst:.3e} over {B} sequences x 32 heads")
    cache.close()


def test_edit_full_size():
    """Prompt edit at full size, in the call the benchmark times: 16 sequences of
    4096 tokens (Hq=32 Hkv=8 d=128) prefilled, each truncated at its seeded edit
    position m_b, then the suffix re-prefilled from new rows (the deep-layer case
    of an edit).  The kept prefix [0, m_b) of every sequence must be byte-identical
    before and after; every suffix row of all 16 sequences is compared with the
    oracle, and all caches and block tables bit for bit."""
    sh = W.EDIT
    say(f"case: edit re-prefill, B={sh.B} n={sh.n} Hq={sh.Hq} Hkv={sh.Hkv} d={sh.d}, every suffix row")
    full = W.prefill_inputs(sh, 1006)
    ms = W.edit_points(sh.B, sh.n)
    lens = [sh.n - m for m in ms]
    suffix = W.prefill_inputs(W.AttnShape(B=sh.B, n=max(lens), Hq=sh.Hq, Hkv=sh.Hkv, d=sh.d, dtype=sh.dtype,
                                          theta=sh.theta), 2006, lengths=lens, start=ms)
    pair = Pair(1, sh.Hkv, sh.d, sh.B * (sh.n // 16) + 16, sh.B, sh.n // 16 + 2, sh.dtype, sh.theta,
                max_position=sh.n + 32, free_order=W.page_order(sh.B * (sh.n // 16) + 16, 1006))
    ids = list(range(sh.B))
    pair.prefill(0, ids, full.Q, full.K, full.V, full.mask, full.positions, oracle=False)
    before = [gather(pair.gpu, b, 0) for b in ids]
    for b, m in zip(ids, ms):
        pair.truncate(b, m)
    Os, _ = pair.prefill(0, ids, suffix.Q, suffix.K, suffix.V, suffix.mask, suffix.positions, oracle=False)
    for b, m in zip(ids, ms):
        k, v = gather(pair.gpu, b, 0)
        assert torch.equal(k[:, :m].view(torch.int16), before[b][0][:, :m].view(torch.int16)), f"prefix K of {b}"
        assert torch.equal(v[:, :m].view(torch.int16), before[b][1][:, :m].view(torch.int16)), f"prefix V of {b}"
    worst = _all_rows(pair, Os, suffix, ids, starts=ms)
    say(f"  worst row-relative error {worst:.3e} over {sum(lens) * sh.Hq} suffix rows")
    pair.check_cache(ids)


def test_attention_half_matches_prefill():
    say("case: kv_cache_append + gqa_attention == gqa_prefill; rows inside a cached sequence")
    import causal_gqa_attention_attn_amd as lib
    shape = W.AttnShape(B=2, n=170, Hq=32, Hkv=8, d=128, dtype=torch.bfloat16, theta=5e5)
    inp = W.prefill_inputs(shape, 313, lengths=[170, 66])
    a = Pair(1, 8, 128, 64, 2, 16, torch.bfloat16, 5e5)
    O, _ = a.prefill(0, [0, 1], inp.Q, inp.K, inp.V, inp.mask, inp.positions, oracle=False)
    b = Pair(1, 8, 128, 64, 2, 16, torch.bfloat16, 5e5)
    b.append(0, [0, 1], inp.K, inp.V, inp.mask, inp.positions)
    O2 = torch.full_like(O, float("nan"))
    lib.gqa_attention(b.gpu.handle, 0, [0, 1], inp.Q.cuda(), inp.mask, inp.positions, O2)
    torch.cuda.synchronize()
    assert torch.equal(O.cpu().view(torch.int16), O2.cpu().view(torch.int16))
    # 40 query rows at positions 100..139 of sequence 0, attending over its cached slots
    Qm = inp.Q[0:1, :, 100:140].contiguous()
    Om = torch.full_like(Qm, float("nan")).cuda()
    lib.gqa_attention(b.gpu.handle, 0, [0], Qm.cuda(), torch.ones((1, 40), dtype=torch.uint8),
                      torch.arange(100, 140, dtype=torch.int32)[None], Om)
    torch.cuda.synchronize()
    ref = b.ref.prefill_rows(0, 0, as_f32(Qm[0]), list(range(100, 140)))
    compare_rows(Om[0], ref, torch.bfloat16)
    with pytest.raises(lib.GqaError) as e:   # queries beyond the cached length
        lib.gqa_attention(b.gpu.handle, 0, [1], Qm.cuda(), torch.ones((1, 40), dtype=torch.uint8),
                          torch.arange(50, 90, dtype=torch.int32)[None], Om)
    assert e.value.name == "POSITION"


def test_decode_graph_replay_matches_eager():
    say("case: HIP-graph replay of append + decode equals the eager calls, replay after replay")
    import causal_gqa_attention_attn_amd as lib
    N, L = 700, 3
    c = lib.PagedCache(L, 8, 128, 64, 1, 64, dtype=torch.bfloat16, rope_theta=1e4, max_position=1024)
    for l in range(L):
        lib.kv_cache_append(c.handle, l, [0], W.normal_device((1, 8, N - 1, 128), 10 + l),
                            W.normal_device((1, 8, N - 1, 128), 20 + l), torch.ones((1, N - 1), dtype=torch.uint8),
                            torch.arange(N - 1, dtype=torch.int32)[None])
    q = [W.normal_device((1, 48, 1, 128), 30 + l) for l in range(L)]
    k = [W.normal_device((1, 8, 1, 128), 40 + l) for l in range(L)]
    v = [W.normal_device((1, 8, 1, 128), 50 + l) for l in range(L)]
    o = [torch.empty_like(x) for x in q]
    ws = torch.zeros(lib.gqa_workspace_size(c.handle, 1, 48), dtype=torch.uint8, device="cuda")
    one = torch.ones((1, 1), dtype=torch.uint8)
    pn = torch.tensor([[N - 1]], dtype=torch.int32)

    def run():
        for l in range(L):
            if l % 2:
                lib.gqa_decode_step(c.handle, l, [0], q[l], k[l], v[l], o[l], ws)
            else:
                lib.kv_cache_append(c.handle, l, [0], k[l], v[l], one, pn)
                lib.gqa_decode(c.handle, l, [0], q[l], [N], o[l], ws)

    run()
    torch.cuda.synchronize()
    eager = [x.clone() for x in o]
    for l in range(L):
        lib.kv_cache_truncate(c.handle, 0, N - 1)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    lib.kv_cache_truncate(c.handle, 0, N - 1)
    for rep in range(3):
        for x in o:
            x.fill_(float("nan"))
        scratch = torch.randn(1 << 20, device="cuda") * 2     # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        del scratch
        for a, b in zip(o, eager):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {rep}"
    c.close()


def test_prefill_second_pass_on_score_overflow():
    say("case: a late key whose score dwarfs the first tile's maximum (forces the prefill's second pass)")
    shape = W.AttnShape(B=1, n=200, Hq=8, Hkv=2, d=128, dtype=torch.bfloat16, theta=0.0)
    inp = W.prefill_inputs(shape, 901)
    # key 150 of kv head 0 and every query of heads 0..3 point the same way with large norm
    direction = torch.zeros(128)
    direction[3] = 1.0
    inp.K[0, 0, 150] = (40.0 * direction).to(torch.bfloat16)
    inp.Q[0, :4, 120:] = (40.0 * direction).to(torch.bfloat16)
    pair = Pair(1, 2, 128, 16, 1, 16, torch.bfloat16, 0.0)
    O, ref = pair.prefill(0, [0], inp.Q, inp.K, inp.V, inp.mask, inp.positions)
    compare_rows(O, ref, torch.bfloat16)
    # rows after the spike are dominated by it: their output is value row 150
    assert torch.allclose(O[0, 0, 160].float().cpu(), inp.V[0, 0, 150].float(), atol=1e-2)


@pytest.mark.parametrize("Hq,Hkv,lengths", [(48, 8, [700]), (32, 8, [33, 320, 1]), (32, 1, [257, 90]),
                                            (8, 2, [16, 47])])
def test_decode_step_fused(Hq, Hkv, lengths):
    say(f"case: gqa_decode_step (append + decode in one launch) Hq={Hq} Hkv={Hkv} lengths={lengths}")
    B = len(lengths)
    d = 128
    shape = W.AttnShape(B=B, n=max(lengths), Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=1e4)
    inp = W.prefill_inputs(shape, 71 + Hq, lengths=lengths)
    a = Pair(1, Hkv, d, 256, B, 64, torch.bfloat16, 1e4, free_order=W.page_order(256, 8))
    b = Pair(1, Hkv, d, 256, B, 64, torch.bfloat16, 1e4, free_order=W.page_order(256, 8))
    ids = list(range(B))
    for p in (a, b):
        p.append(0, ids, inp.K, inp.V, inp.mask, inp.positions)
    for t in range(3):
        st = W.decode_step_inputs(shape, 71, t)
        o1, r1 = a.step_fused(0, ids, st)
        o2, _ = b.step(0, ids, st)
        compare_rows(o1, r1, torch.bfloat16)
        assert torch.equal(o1.cpu().view(torch.int16), o2.cpu().view(torch.int16)), f"step {t}"
    a.check_cache(ids)
    for s in ids:
        ka, va = gather(a.gpu, s, 0)
        kb, vb = gather(b.gpu, s, 0)
        assert torch.equal(ka.view(torch.int16), kb.view(torch.int16))
        assert torch.equal(va.view(torch.int16), vb.view(torch.int16))


@pytest.mark.parametrize("T", [40000, 16 * 16 * 4 + 1, 16 * 16 * 4])
def test_decode_many_splits(T):
    """One long sequence on one kv head: up to 125 splits, several merge rounds
    per lane (running maximum across rounds), and 4- and 5-split merges."""
    say(f"case: decode_step with many splits, T={T}, Hq=8 Hkv=1 d=128")
    import causal_gqa_attention_attn_amd as lib
    from oracle.cache_model import CacheModel
    pages = -(-T // 16) + 2
    cache = lib.PagedCache(1, 1, 128, pages, 1, pages, dtype=torch.bfloat16, rope_theta=1e4,
                           max_position=pages * 16, free_list_order=W.page_order(pages, 77))
    kf = W.normal_device((1, 1, T - 1, 128), 93000 + T)
    vf = W.normal_device((1, 1, T - 1, 128), 94000 + T)
    lib.kv_cache_append(cache.handle, 0, [0], kf, vf, torch.ones((1, T - 1), dtype=torch.uint8),
                        torch.arange(T - 1, dtype=torch.int32)[None])
    shape = W.AttnShape(B=1, n=1, Hq=8, Hkv=1, d=128, dtype=torch.bfloat16, theta=1e4)
    st = W.decode_step_inputs(shape, 95, T)
    o = torch.full((1, 8, 1, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(lib.gqa_workspace_size(cache.handle, 1, 8), dtype=torch.uint8, device="cuda")
    for rep in range(2):                      # second call: flags were left at zero
        if rep:
            lib.kv_cache_truncate(cache.handle, 0, T - 1)
        lib.gqa_decode_step(cache.handle, 0, [0], st.q.cuda(), st.k.cuda(), st.v.cuda(), o, ws)
        torch.cuda.synchronize()
        ref = CacheModel(1, 1, 128, 16, pages, 1, pages, dtype="bf16", rope_theta=1e4, max_position=pages * 16)
        k = torch.cat([kf.cpu(), st.k], dim=2)
        v = torch.cat([vf.cpu(), st.v], dim=2)
        ref.append(0, [0], as_f32(k), as_f32(v), np.ones((1, T), np.uint8), np.arange(T)[None])
        r = ref.decode(0, [0], as_f32(st.q), [T])
        compare_rows(o, r, torch.bfloat16)
    cache.close()


# ------------------------------------------------------------------ stale cache memory

def _poison_stale(pair, seq, layers):
    """NaN into every slot of the sequence's pages at or past its length."""
    lib = pair.lib
    pages = lib.gqa_cache_page_table(pair.gpu.handle, seq)
    kv, vv = k_view(pair.gpu), v_view(pair.gpu)
    for l in layers:
        n = lib.gqa_cache_length(pair.gpu.handle, seq, l)
        for lp, ph in enumerate(pages):
            lo = max(n - lp * 16, 0)
            if lo < 16:
                kv[l, ph, :, lo:, :] = float("nan")
                vv[l, ph, :, :, lo:] = float("nan")


@pytest.mark.parametrize("d,Hq,Hkv", [(128, 32, 8), (64, 8, 2)])
def test_poisoned_cache_memory_never_reaches_outputs(d, Hq, Hkv):
    """Stale and never-written cache slots may hold any bits (NaN here): slots
    past a sequence's length, in its last partly written page, and slots a
    truncate leaves behind.  None of them may reach a valid output."""
    say(f"case: NaN-filled pools, ragged prefill, decode, truncate + re-prefill; d={d} Hq={Hq} Hkv={Hkv}")
    lens = [37, 100, 1, 66]
    B = len(lens)
    n = max(lens)
    shape = W.AttnShape(B=B, n=n, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=1e4)
    inp = W.prefill_inputs(shape, 4242, lengths=lens)
    pair = Pair(1, Hkv, d, 64, B, 16, torch.bfloat16, 1e4, free_order=W.page_order(64, 9))
    pair.gpu.k_pool.fill_(float("nan"))
    pair.gpu.v_pool.fill_(float("nan"))
    ids = list(range(B))
    O, ref = pair.prefill(0, ids, inp.Q, inp.K, inp.V, inp.mask, inp.positions)
    valid = inp.mask.numpy().astype(bool)[:, None, :].repeat(Hq, 1)
    compare_rows(O, ref, torch.bfloat16, rows_mask=valid)
    for step in range(3):
        o, r = pair.step_fused(0, ids, W.decode_step_inputs(shape, 4242, step))
        compare_rows(o, r, torch.bfloat16)
    pair.check_cache(ids)
    # truncate inside a page, poison what it left behind, re-prefill the suffix
    ms = [20, 51, 1, 64]
    for s, m in zip(ids, ms):
        pair.truncate(s, m)
        _poison_stale(pair, s, [0])
    torch.cuda.synchronize()
    sl = [L + 3 - m for L, m in zip(lens, ms)]
    suffix = W.prefill_inputs(W.AttnShape(B=B, n=max(sl), Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=1e4),
                              4343, lengths=sl, start=ms)
    O, ref = pair.prefill(0, ids, suffix.Q, suffix.K, suffix.V, suffix.mask, suffix.positions)
    valid = suffix.mask.numpy().astype(bool)[:, None, :].repeat(Hq, 1)
    compare_rows(O, ref, torch.bfloat16, rows_mask=valid)
    for s in ids:
        _poison_stale(pair, s, [0])
    torch.cuda.synchronize()
    o, r = pair.step_fused(0, ids, W.decode_step_inputs(shape, 4343, 0))
    compare_rows(o, r, torch.bfloat16)
    pair.check_cache(ids)


@pytest.mark.parametrize("scale", [4.0, 8.0])
def test_large_logits_bf16(scale):
    """Queries and keys scaled up (raw scores 16x and 64x those of N(0,1) inputs):
    the softmax must stay within the bf16 tolerance, so the kernel may not round
    anything that multiplies with the score's magnitude (such as a query scaled
    by the softmax factor before its bf16 rounding)."""
    say(f"case: bf16 prefill with Q, K scaled by {scale}")
    shape = W.AttnShape(B=2, n=300, Hq=16, Hkv=4, d=128, dtype=torch.bfloat16, theta=1e4)
    inp = W.prefill_inputs(shape, 777, lengths=[300, 171])
    Q = (inp.Q.float() * scale).to(torch.bfloat16)
    K = (inp.K.float() * scale).to(torch.bfloat16)
    pair = Pair(1, 4, 128, 64, 2, 24, torch.bfloat16, 1e4)
    O, ref = pair.prefill(0, [0, 1], Q, K, inp.V, inp.mask, inp.positions)
    valid = inp.mask.numpy().astype(bool)[:, None, :].repeat(16, 1)
    compare_rows(O, ref, torch.bfloat16, rows_mask=valid)
    o, r = pair.step_fused(0, [0, 1], W.decode_step_inputs(shape, 777, 0))
    compare_rows(o, r, torch.bfloat16)
