"""GPU edge cases against the float64 oracle: empty calls, rows without a valid
token, a decode over a single cached token, positions at the end of the
rotation table, a sequence that fills its block table exactly, a pool that
runs out exactly, and block-table writes spread over several patch launches.
Every rejected call must leave the cache unchanged and match the oracle's
error class."""
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


DTYPES = [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 32)]


@pytest.mark.parametrize("dtype,d", DTYPES)
def test_empty_calls_change_nothing(dtype, d):
    """B = 0 calls and n = 0 prefills are no-ops that return success."""
    import causal_gqa_attention_attn_amd as lib
    say(f"case: empty calls, {dtype} d={d}")
    pair = Pair(1, 2, d, 16, 2, 8, dtype, 1e4)
    shape = W.AttnShape(B=1, n=20, Hq=4, Hkv=2, d=d, dtype=dtype, theta=1e4)
    inp = W.prefill_inputs(shape, 61)
    pair.prefill(0, [0], inp.Q, inp.K, inp.V, inp.mask, inp.positions)
    free = lib.gqa_cache_free_pages(pair.gpu.handle)
    z4 = lambda H, n: torch.zeros((0, H, n, d), dtype=dtype, device="cuda")
    lib.gqa_prefill(pair.gpu.handle, 0, [], z4(4, 5), z4(2, 5), z4(2, 5), np.zeros((0, 5), np.uint8),
                    np.zeros((0, 5), np.int32), z4(4, 5))
    lib.kv_cache_append(pair.gpu.handle, 0, [], z4(2, 5), z4(2, 5), np.zeros((0, 5), np.uint8),
                        np.zeros((0, 5), np.int32))
    lib.gqa_decode(pair.gpu.handle, 0, [], z4(4, 1), [], z4(4, 1))
    lib.gqa_decode_step(pair.gpu.handle, 0, [], z4(4, 1), z4(2, 1), z4(2, 1), z4(4, 1))
    # n = 0 for a real sequence
    e = lambda H: torch.zeros((1, H, 0, d), dtype=dtype, device="cuda")
    lib.gqa_prefill(pair.gpu.handle, 0, [0], e(4), e(2), e(2), np.zeros((1, 0), np.uint8),
                    np.zeros((1, 0), np.int32), e(4))
    torch.cuda.synchronize()
    assert lib.gqa_cache_free_pages(pair.gpu.handle) == free
    assert lib.gqa_cache_length(pair.gpu.handle, 0, 0) == 20
    pair.check_cache([0, 1])


@pytest.mark.parametrize("dtype,d", DTYPES)
def test_rows_without_valid_tokens(dtype, d):
    """Batch rows with no valid token between rows with many: their output rows
    are exact zeros, they take no page, the other rows match the oracle."""
    say(f"case: rows without valid tokens, {dtype} d={d}")
    lengths = [0, 37, 0, 70, 0]
    shape = W.AttnShape(B=5, n=70, Hq=8, Hkv=2, d=d, dtype=dtype, theta=1e4)
    inp = W.prefill_inputs(shape, 62, lengths=lengths, poison_padding=True)
    pair = Pair(1, 2, d, 32, 5, 8, dtype, 1e4, free_order=W.page_order(32, 63))
    ids = [4, 0, 3, 1, 2]
    O, ref = pair.prefill(0, ids, inp.Q, inp.K, inp.V, inp.mask, inp.positions)
    valid = inp.mask.numpy().astype(bool)[:, None, :].repeat(8, 1)
    compare_rows(O, ref, dtype, rows_mask=valid)
    assert np.all(as_f32(O)[~valid] == 0.0), "rows without a valid token must be exact zeros"
    pair.check_cache(ids)
    for s in (4, 3, 2):
        assert pair.lib.gqa_cache_page_table(pair.gpu.handle, s) == []


@pytest.mark.parametrize("dtype,d", DTYPES)
def test_decode_over_one_cached_token(dtype, d):
    """A decode step on an empty cache appends the token and reads T = 1 slot:
    the output is that token's value (one visible key), bit for bit in the
    oracle's rounding; then T = 2."""
    say(f"case: decode at T=1 and T=2, {dtype} d={d}")
    pair = Pair(1, 2, d, 8, 2, 4, dtype, 1e4)
    shape = W.AttnShape(B=2, n=1, Hq=4, Hkv=2, d=d, dtype=dtype, theta=1e4)
    for t in range(2):
        st = W.decode_step_inputs(shape, 64, t)
        o, r = pair.step_fused(0, [0, 1], st)
        compare_rows(o, r, dtype)
        if t == 0:
            # one visible key: softmax weight exactly 1, output = v of g(h)
            v = as_f32(st.v)
            for h in range(4):
                assert np.array_equal(as_f32(o)[:, h, 0], v[:, h // 2, 0]), "T=1 output must equal v"
    pair.check_cache([0, 1])


def test_positions_at_the_end_of_the_rotation_table():
    """Positions up to max_position - 1 are accepted (the last rotation rows);
    one more token is GQA_ERR_POSITION and changes nothing."""
    import causal_gqa_attention_attn_amd as lib
    from oracle.cache_model import OracleError
    say("case: positions at the end of the rotation table (max_position 100)")
    pair = Pair(1, 2, 128, 16, 1, 16, torch.bfloat16, 5e5, max_position=100)
    shape = W.AttnShape(B=1, n=100, Hq=8, Hkv=2, d=128, dtype=torch.bfloat16, theta=5e5)
    inp = W.prefill_inputs(shape, 65)
    O, ref = pair.prefill(0, [0], inp.Q, inp.K, inp.V, inp.mask, inp.positions)
    compare_rows(O, ref, torch.bfloat16)
    st = W.decode_step_inputs(W.AttnShape(B=1, n=1, Hq=8, Hkv=2, d=128, dtype=torch.bfloat16, theta=5e5), 66, 0)
    o = torch.zeros((1, 8, 1, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.GqaError) as e:
        lib.gqa_decode_step(pair.gpu.handle, 0, [0], st.q.cuda(), st.k.cuda(), st.v.cuda(), o)
    assert e.value.name == "POSITION"
    with pytest.raises(OracleError) as r:
        pair.ref.append(0, [0], as_f32(st.k), as_f32(st.v), np.ones((1, 1), np.uint8), np.array([[100]]))
    assert r.value.code == "POSITION"
    assert lib.gqa_cache_length(pair.gpu.handle, 0, 0) == 100
    pair.check_cache([0])


def test_full_block_table_and_exhausted_pool():
    """A sequence filling its block table exactly (8 pages = 128 tokens) decodes
    at T = 128; one more token is GQA_ERR_OUT_OF_PAGES.  A pool used to its
    last page refuses the next page the same way.  Nothing changes on refusal."""
    import causal_gqa_attention_attn_amd as lib
    from oracle.cache_model import OracleError
    say("case: full block table (8 pages), pool of 12 pages used up")
    pair = Pair(1, 2, 64, 12, 2, 8, torch.bfloat16, 1e4, max_position=1024, free_order=W.page_order(12, 67))
    shape = W.AttnShape(B=1, n=127, Hq=4, Hkv=2, d=64, dtype=torch.bfloat16, theta=1e4)
    inp = W.prefill_inputs(shape, 68)
    O, ref = pair.prefill(0, [0], inp.Q, inp.K, inp.V, inp.mask, inp.positions)
    compare_rows(O, ref, torch.bfloat16)
    dshape = W.AttnShape(B=1, n=1, Hq=4, Hkv=2, d=64, dtype=torch.bfloat16, theta=1e4)
    o, r = pair.step_fused(0, [0], W.decode_step_inputs(dshape, 69, 0))      # T = 128: table full
    compare_rows(o, r, torch.bfloat16)
    st = W.decode_step_inputs(dshape, 69, 1)
    oo = torch.zeros((1, 4, 1, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.GqaError) as e:
        lib.gqa_decode_step(pair.gpu.handle, 0, [0], st.q.cuda(), st.k.cuda(), st.v.cuda(), oo)
    assert e.value.name == "OUT_OF_PAGES"
    with pytest.raises(OracleError) as rr:
        pair.ref.append(0, [0], as_f32(st.k), as_f32(st.v), np.ones((1, 1), np.uint8), np.array([[128]]))
    assert rr.value.code == "OUT_OF_PAGES"
    # sequence 1 takes the last 4 pages (64 tokens), then needs a fifth
    s2 = W.prefill_inputs(W.AttnShape(B=1, n=64, Hq=4, Hkv=2, d=64, dtype=torch.bfloat16, theta=1e4), 70)
    pair.prefill(0, [1], s2.Q, s2.K, s2.V, s2.mask, s2.positions)
    assert lib.gqa_cache_free_pages(pair.gpu.handle) == 0
    st1 = W.decode_step_inputs(dshape, 71, 0)
    with pytest.raises(lib.GqaError) as e:
        lib.gqa_decode_step(pair.gpu.handle, 0, [1], st1.q.cuda(), st1.k.cuda(), st1.v.cuda(), oo)
    assert e.value.name == "OUT_OF_PAGES"
    assert lib.gqa_cache_length(pair.gpu.handle, 1, 0) == 64
    pair.check_cache([0, 1])


def test_decode_steps_write_the_pages_they_open():
    """Decode steps that open a page for their token write its block-table entry
    in the decode launch itself.  Three sequences at 14, 15 and 16 tokens take
    20 fused steps (each crosses a page boundary at a different step, one of
    them at once), with a free order that scatters the pages; every step
    against the oracle, then the device block tables bit for bit, then a plain
    decode and a truncate + re-append that read those entries back."""
    say("case: fused decode steps opening pages (block-table entries written in the launch)")
    d, Hq, Hkv = 128, 8, 2
    pair = Pair(1, Hkv, d, 24, 3, 8, torch.bfloat16, 1e4, max_position=1024, free_order=W.page_order(24, 73))
    lengths = [14, 15, 16]
    shape = W.AttnShape(B=3, n=16, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=1e4)
    inp = W.prefill_inputs(shape, 74, lengths=lengths)
    O, ref = pair.prefill(0, [0, 1, 2], inp.Q, inp.K, inp.V, inp.mask, inp.positions)
    dshape = W.AttnShape(B=3, n=1, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=1e4)
    for t in range(20):
        o, r = pair.step_fused(0, [0, 1, 2], W.decode_step_inputs(dshape, 75, t))
        compare_rows(o, r, torch.bfloat16)
    pair.check_cache([0, 1, 2])
    # a decode without append reads every page through the device table
    st = W.decode_step_inputs(dshape, 76, 0)
    lens = [pair.ref.cache_length(s, 0) for s in (0, 1, 2)]
    o, r = pair.decode(0, [0, 1, 2], st.q, lens)
    compare_rows(o, r, torch.bfloat16)
    # free a page again and let the next step open it once more
    pair.truncate(1, 32)
    o, r = pair.step_fused(0, [1], W.decode_step_inputs(W.AttnShape(B=1, n=1, Hq=Hq, Hkv=Hkv, d=d,
                                                                   dtype=torch.bfloat16, theta=1e4), 77, 0))
    compare_rows(o, r, torch.bfloat16)
    pair.check_cache([0, 1, 2])


def test_block_table_patches_split_by_count_and_by_index_span():
    """One append opens 40 x 38 = 1520 block-table entries.  Twenty sequences
    have neighbouring ids (760 entries within 40 960 table indexes: more than
    one patch launch holds), twenty are spread over ids 24..100 (indexes more
    than 65 535 apart: the 16-bit offsets of one launch cannot reach).  The
    device block tables must equal the oracle's bit for bit, and a decode of
    every sequence reads its pages through them."""
    say("case: 1520 block-table entries in one append, split by count and by index span")
    d, Hq, Hkv, L = 64, 4, 2, 600
    ids = list(range(20)) + [24 + 4 * i for i in range(20)]
    pages = len(ids) * 38 + 16
    pair = Pair(1, Hkv, d, pages, max(ids) + 1, 2048, torch.bfloat16, 1e4, max_position=1024,
                free_order=W.page_order(pages, 78))
    shape = W.AttnShape(B=len(ids), n=L, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=1e4)
    inp = W.prefill_inputs(shape, 79)
    pair.append(0, ids, inp.K, inp.V, inp.mask, inp.positions)
    pair.check_cache(ids)
    st = W.decode_step_inputs(W.AttnShape(B=len(ids), n=1, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=1e4),
                              80, 0)
    o, r = pair.decode(0, ids, st.q, [L] * len(ids))
    compare_rows(o, r, torch.bfloat16)
