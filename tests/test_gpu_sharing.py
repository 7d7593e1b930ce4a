"""GPU parity of prefix sharing: kv_cache_fork, copy-on-write, shared-page release.

Sequences that share a prefix reference the same physical pages; a write into
a shared page copies it first.  The library and the float64 oracle run the
same calls; block tables, reference-counted free lists and cache bytes must
agree bit for bit, outputs within 2e-2 of the row maximum (bfloat16) or 1e-5
(float32).
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


def _prefill_all_layers(pair, layers, ids, shape, seed, lengths, start, workspace=None):
    inp = W.prefill_inputs(shape, seed, lengths=lengths, start=start)
    valid = inp.mask.numpy().astype(bool)[:, None, :].repeat(shape.Hq, 1)
    for layer in range(layers):
        O, ref = pair.prefill(layer, ids, inp.Q, inp.K, inp.V, inp.mask, inp.positions, workspace=workspace)
        compare_rows(O, ref, shape.dtype, rows_mask=valid)


@pytest.mark.parametrize("mfork", [0, 16, 37, 300])
@pytest.mark.parametrize("dtype,Hq,Hkv,d", [(torch.bfloat16, 32, 8, 128), (torch.bfloat16, 8, 2, 64),
                                            (torch.float32, 4, 2, 32)])
def test_fork_branches(dtype, Hq, Hkv, d, mfork):
    """A 300-token request, a second one forked from it at mfork that prefills
    its own 50-token suffix, decode steps on both (each branch writing into a
    page the other still references), a third request forked from the second,
    then releasing the first."""
    say(f"case: fork at {mfork}, {dtype} Hq={Hq} Hkv={Hkv} d={d}")
    layers = 2
    pair = Pair(layers, Hkv, d, 96, 3, 32, dtype, 1e4, free_order=W.page_order(96, 77))
    shape = lambda B, n: W.AttnShape(B=B, n=n, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, theta=1e4)
    _prefill_all_layers(pair, layers, [0], shape(1, 300), 501, [300], 0)
    pair.fork(0, 1, mfork)
    pair.check_cache([0, 1], device_tables=False)
    _prefill_all_layers(pair, layers, [1], shape(1, 50), 502, [50], mfork)
    pair.check_cache([0, 1])
    for step in range(2):
        for layer in range(layers):
            o, r = pair.step(layer, [0, 1], W.decode_step_inputs(shape(2, 1), 503 + layer, step))
            compare_rows(o, r, dtype)
    pair.check_cache([0, 1])
    # a third request shares the second one's first 40 + mfork // 2 positions
    m2 = mfork // 2 + 40
    pair.fork(1, 2, m2)
    _prefill_all_layers(pair, layers, [2, 0], shape(2, 20), 504, [20, 7], [m2, 302])
    pair.check_cache([0, 1, 2])
    # the first request ends; the pages the others still reference must stay
    pair.truncate(0, 0)
    pair.check_cache([0, 1, 2], device_tables=False)
    for layer in range(layers):
        o, r = pair.step(layer, [1, 2], W.decode_step_inputs(shape(2, 1), 505 + layer, 0))
        compare_rows(o, r, dtype)
    pair.check_cache([0, 1, 2])


def test_fork_fused_step_copy_on_write_and_remap():
    """gqa_decode_step writes the new token inside the kernel: a shared last
    page must be copied before that launch.  Then a remap moves pages that two
    tables reference; both tables follow."""
    import causal_gqa_attention_attn_amd as lib
    say("case: fused decode step into a shared page; remap of shared pages")
    Hq, Hkv, d = 48, 8, 128
    pair = Pair(1, Hkv, d, 64, 3, 16, torch.bfloat16, 1e4, free_order=W.page_order(64, 78))
    shape = lambda B, n: W.AttnShape(B=B, n=n, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=1e4)
    _prefill_all_layers(pair, 1, [0], shape(1, 45), 601, [45], 0)
    pair.fork(0, 1, 45)
    pair.fork(0, 2, 33)
    for step in range(3):
        o, r = pair.step_fused(0, [1, 0, 2], W.decode_step_inputs(shape(3, 1), 602, step))
        compare_rows(o, r, torch.bfloat16)
        pair.check_cache([0, 1, 2])
    # move every page in use to the free pages at the end of the pool
    used = sorted({p for s in range(3) for p in pair.ref.page_table(s)})
    free = [p for p in pair.ref.free]
    dst = free[-len(used):]
    lib.kv_cache_remap(pair.gpu.handle, used, dst)
    pair.ref.remap(used, dst)
    pair.check_cache([0, 1, 2])
    o, r = pair.step_fused(0, [0, 1, 2], W.decode_step_inputs(shape(3, 1), 603, 0))
    compare_rows(o, r, torch.bfloat16)
    pair.check_cache([0, 1, 2])


def test_forked_verify_chunks_share_a_long_prefix():
    """Four requests forked from one 3000-token prompt (a shared system prompt),
    each then verifying its own 5-token chunk on the split-T kernel."""
    say("case: 4 forks of a 3000-token prompt, 5-token verify chunks")
    Hq, Hkv, d = 32, 8, 128
    pair = Pair(1, Hkv, d, 220, 5, 200, torch.bfloat16, 5e5, free_order=W.page_order(220, 79))
    shape = lambda B, n: W.AttnShape(B=B, n=n, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=5e5)
    inp = W.prefill_inputs(shape(1, 3000), 701)
    pair.prefill(0, [0], inp.Q, inp.K, inp.V, inp.mask, inp.positions, oracle=False)
    for s, m in zip([1, 2, 3, 4], [3000, 2990, 2048, 1]):
        pair.fork(0, s, m)
    pair.check_cache(list(range(5)), device_tables=False)
    ws = pair.chunk_workspace(4, Hq, 5)
    starts = [3000, 2990, 2048, 1]
    ch = W.prefill_inputs(shape(4, 5), 702, start=starts)
    O, ref = pair.prefill(0, [1, 2, 3, 4], ch.Q, ch.K, ch.V, ch.mask, ch.positions, workspace=ws)
    compare_rows(O, ref, torch.bfloat16)
    pair.check_cache(list(range(5)))
    # pages of the prompt: shared by every fork that covers them, stored once
    table0 = pair.ref.page_table(0)
    assert pair.lib.gqa_cache_page_table(pair.gpu.handle, 1)[:187] == table0[:187]
    # page 1 of the prompt: the prompt and the three long forks; page 0 too, since
    # the 1-token fork copied it before writing its slot 1
    assert pair.ref.ref[table0[1]] == 4 and pair.ref.ref[table0[0]] == 4
