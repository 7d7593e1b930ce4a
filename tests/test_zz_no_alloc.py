"""GPU: gqa_decode_step_noalloc (the library's static split scratch, no device
allocation) against gqa_decode_step (the caller's workspace).

Two caches with the same configuration, page order and contents take the same
decode steps, one through each entry point.  Outputs and cache bytes must be
bit-identical (the same kernels read the same inputs), and both within the
bf16 tolerance of the float64 oracle.  The calls run in a row with shrinking
and growing inputs, so the shared scratch is reused with leftovers of a larger
call in it.  A call too large for the scratch is refused and changes nothing.
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


def _noalloc_step(pair, layer, ids, st):
    """One decode step through gqa_decode_step_noalloc; the oracle takes the
    same append and decode."""
    lens = [pair.ref.cache_length(s, layer) for s in ids]
    qd = st.q.to("cuda")
    o = torch.full_like(qd, float("nan"))
    pair.lib.gqa_decode_step_noalloc(pair.gpu.handle, layer, ids, qd, st.k.to("cuda"), st.v.to("cuda"), o)
    torch.cuda.synchronize()
    B = len(ids)
    pair.ref.append(layer, ids, as_f32(st.k), as_f32(st.v), np.ones((B, 1), np.uint8), np.array([[n] for n in lens]))
    return o, pair.ref.decode(layer, ids, as_f32(st.q), [n + 1 for n in lens])


def test_noalloc_decode_step_matches_workspace_path():
    import causal_gqa_attention_attn_amd as lib
    Hq, Hkv, d = 32, 8, 128
    lengths = [3000, 2100, 700, 40]
    say(f"case: no-alloc decode step vs workspace decode step, Hq={Hq} Hkv={Hkv} d={d}, lengths {lengths}")
    shape = W.AttnShape(B=4, n=max(lengths), Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=5e5)
    inp = W.prefill_inputs(shape, 951, lengths=lengths)
    order = W.page_order(800, 952)
    pairs = [Pair(1, Hkv, d, 800, 4, 200, torch.bfloat16, 5e5, free_order=order) for _ in range(2)]
    for p in pairs:
        p.prefill(0, [0, 1, 2, 3], inp.Q, inp.K, inp.V, inp.mask, inp.positions, oracle=False)
    ws_pair, na_pair = pairs
    # calls in a row: all four sequences (several splits each for the long
    # ones), then a smaller call (two sequences, the short ones), then the two
    # longest, then all four again
    calls = [[0, 1, 2, 3], [2, 3], [0, 1], [3, 2, 1, 0]]
    for i, ids in enumerate(calls):
        dshape = W.AttnShape(B=len(ids), n=1, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=5e5)
        st = W.decode_step_inputs(dshape, 960 + i, 0)
        o_ws, r_ws = ws_pair.step_fused(0, ids, st)
        o_na, r_na = _noalloc_step(na_pair, 0, ids, st)
        say(f"  call {i}: sequences {ids}")
        assert torch.equal(o_ws.cpu().view(torch.int16), o_na.cpu().view(torch.int16)), f"call {i}: outputs differ"
        compare_rows(o_na, r_na, torch.bfloat16)
        compare_rows(o_ws, r_ws, torch.bfloat16)
    for s in range(4):
        ka, va = gather(ws_pair.gpu, s, 0)
        kb, vb = gather(na_pair.gpu, s, 0)
        assert torch.equal(ka.view(torch.int16), kb.view(torch.int16)), f"K cache of {s}"
        assert torch.equal(va.view(torch.int16), vb.view(torch.int16)), f"V cache of {s}"
    na_pair.check_cache([0, 1, 2, 3])
    lib.gqa_workspace_status(na_pair.gpu.handle, None)
    lib.gqa_workspace_status(ws_pair.gpu.handle, ws_pair.ws)


def test_noalloc_refuses_calls_beyond_the_scratch():
    """64 kv heads of d = 64 (64 split slots per split), 50 sequences of 300
    tokens (two splits each): 100 splits need 6400 slots, more than the 48 MiB
    scratch holds; the call is refused before anything changes."""
    import causal_gqa_attention_attn_amd as lib
    say("case: no-alloc decode step too large for the static scratch")
    B, n, H, d = 50, 300, 64, 64
    shape = W.AttnShape(B=B, n=n, Hq=H, Hkv=H, d=d, dtype=torch.bfloat16, theta=1e4)
    inp = W.prefill_inputs(shape, 970)
    pair = Pair(1, H, d, B * 20, B, 20, torch.bfloat16, 1e4)
    ids = list(range(B))
    pair.prefill(0, ids, inp.Q, inp.K, inp.V, inp.mask, inp.positions, oracle=False)
    st = W.decode_step_inputs(W.AttnShape(B=B, n=1, Hq=H, Hkv=H, d=d, dtype=torch.bfloat16, theta=1e4), 971, 0)
    o = torch.zeros((B, H, 1, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.GqaError) as e:
        lib.gqa_decode_step_noalloc(pair.gpu.handle, 0, ids, st.q.cuda(), st.k.cuda(), st.v.cuda(), o)
    assert e.value.name == "UNSUPPORTED"
    assert all(lib.gqa_cache_length(pair.gpu.handle, s, 0) == n for s in ids)
    pair.check_cache([0, B - 1])
    # a smaller call on the same caches fits and is correct
    sub = list(range(8))
    st8 = W.decode_step_inputs(W.AttnShape(B=8, n=1, Hq=H, Hkv=H, d=d, dtype=torch.bfloat16, theta=1e4), 972, 0)
    o8, r8 = _noalloc_step(pair, 0, sub, st8)
    compare_rows(o8, r8, torch.bfloat16)
    lib.gqa_workspace_status(pair.gpu.handle, None)


def test_noalloc_decode_step_in_a_hip_graph():
    """The allocation-free decode step captured into a HIP graph (two layers,
    caches long enough for several splits) and replayed three times, with
    eager work of the program between replays: every replay's outputs equal
    the eager call's bit for bit, and the status word stays clear."""
    import causal_gqa_attention_attn_amd as lib
    Hq, Hkv, d, L = 32, 8, 128, 2
    lengths = [2500, 900]
    say(f"case: no-alloc decode step in a HIP graph, {L} layers, lengths {lengths}")
    shape = W.AttnShape(B=2, n=max(lengths), Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=5e5)
    inp = W.prefill_inputs(shape, 981, lengths=lengths)
    pairs = [Pair(L, Hkv, d, 300, 2, 170, torch.bfloat16, 5e5, free_order=W.page_order(300, 982)) for _ in range(2)]
    for p in pairs:
        for layer in range(L):
            p.prefill(layer, [0, 1], inp.Q, inp.K, inp.V, inp.mask, inp.positions, oracle=False)
    eager, graphed = pairs
    dshape = W.AttnShape(B=2, n=1, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=5e5)
    steps = [W.decode_step_inputs(dshape, 983, layer) for layer in range(L)]
    dev = [(s.q.cuda(), s.k.cuda(), s.v.cuda()) for s in steps]
    # eager reference: one decode step per layer on the first cache
    ref = []
    for layer, (q, k, v) in enumerate(dev):
        o = torch.full_like(q, float("nan"))
        lib.gqa_decode_step_noalloc(eager.gpu.handle, layer, [0, 1], q, k, v, o)
        ref.append(o)
    torch.cuda.synchronize()
    # graph: the same steps on the second cache, captured once (the scratch is
    # set up by the earlier eager calls on this device)
    outs = [torch.full_like(q, float("nan")) for q, _, _ in dev]
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            for layer, (q, k, v) in enumerate(dev):
                lib.gqa_decode_step_noalloc(graphed.gpu.handle, layer, [0, 1], q, k, v, outs[layer],
                                            stream=stream.cuda_stream)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device="cuda").sum()      # eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for layer in range(L):
            assert torch.equal(outs[layer].cpu().view(torch.int16), ref[layer].cpu().view(torch.int16)), \
                f"replay {rep}, layer {layer}"
    lib.gqa_workspace_status(graphed.gpu.handle, None)
    for layer in range(L):
        ka, va = gather(eager.gpu, 0, layer)
        kb, vb = gather(graphed.gpu, 0, layer)
        assert torch.equal(ka.view(torch.int16), kb.view(torch.int16))
        assert torch.equal(va.view(torch.int16), vb.view(torch.int16))
