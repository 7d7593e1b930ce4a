"""GPU parity of short query chunks on the split-T kernel (speculative verify).

A bfloat16 gqa_prefill / gqa_attention call with at most GQA_MAX_CHUNK_TOKENS
rectangular rows and a workspace runs on the split-T kernel: one matrix
column per (query token, head), each with its own position, rotation row and
causal limit, split over the cached keys.  Outputs are compared with the
float64 oracle per row (2e-2 of the row maximum), padding rows must be exactly
zero and the cache bit-exact.
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


def _chunk(shape, seed, counts, row0, starts):
    """Q, K, V ~ N(0,1) of [B, H, n, d]; row b holds counts[b] valid tokens from
    rectangular row row0[b] on, at positions starts[b], starts[b] + 1, ...
    Padding rows of Q, K and V are NaN (they must never reach an output)."""
    B, n = shape.B, shape.n
    Q = W.normal((B, shape.Hq, n, shape.d), seed, shape.dtype)
    K = W.normal((B, shape.Hkv, n, shape.d), seed + 100_000, shape.dtype)
    V = W.normal((B, shape.Hkv, n, shape.d), seed + 200_000, shape.dtype)
    mask = torch.zeros((B, n), dtype=torch.uint8)
    pos = torch.zeros((B, n), dtype=torch.int32)
    for b in range(B):
        r, c = row0[b], counts[b]
        mask[b, r:r + c] = 1
        pos[b, r:r + c] = torch.arange(starts[b], starts[b] + c, dtype=torch.int32)
        for t in (Q, K, V):
            t[b, :, :r] = float("nan")
            t[b, :, r + c:] = float("nan")
    return Q, K, V, mask, pos


def _check_chunk_outputs(O, ref, mask, Hq):
    valid = mask.numpy().astype(bool)[:, None, :].repeat(Hq, 1)
    compare_rows(O, ref, torch.bfloat16, rows_mask=valid)
    pad = as_f32(O)[~valid]
    assert np.all(pad == 0.0), "padding rows of O must be written as 0"


def _build_prefix(pair, ids, lens, Hq, seed):
    """Cache prefixes of the given lengths through the tiled prefill (unchecked)."""
    shape = W.AttnShape(B=len(ids), n=max(max(lens), 1), Hq=Hq, Hkv=pair.ref.Hkv, d=pair.ref.d,
                        dtype=torch.bfloat16, theta=pair.ref.theta)
    inp = W.prefill_inputs(shape, seed, lengths=lens)
    pair.prefill(0, ids, inp.Q, inp.K, inp.V, inp.mask, inp.positions, oracle=False)


CHUNK_SHAPES = [(32, 8, 128), (48, 8, 128), (8, 8, 64), (64, 8, 128), (16, 1, 64)]


@pytest.mark.parametrize("n", [1, 4, 7, 16])
@pytest.mark.parametrize("Hq,Hkv,d", CHUNK_SHAPES)
def test_verify_chunks_bf16(Hq, Hkv, d, n):
    """Two verify rounds: a chunk on cached prefixes (empty, inside a page,
    several pages, many splits), a truncate that drops rejected tokens with the
    slots they leave poisoned, then the next chunk."""
    G = Hq // Hkv
    say(f"case: verify chunks n={n} Hq={Hq} Hkv={Hkv} d={d} (G={G}, {n * G} columns per kv head)")
    prefix = [0, 5, 300, 2100]
    B = len(prefix)
    pair = Pair(1, Hkv, d, 4 * 140, B, 140, torch.bfloat16, 1e4, free_order=W.page_order(4 * 140, 21))
    ids = list(range(B))
    _build_prefix(pair, ids, prefix, Hq, 9000 + n)
    ws = pair.chunk_workspace(B, Hq, n)
    shape = W.AttnShape(B=B, n=n, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=1e4)
    # a full chunk, a left-padded run, one token in the last row, an idle sequence
    counts = [n, max(1, n - 2), 1, 0]
    row0 = [0, n - counts[1], n - 1, 0]
    Q, K, V, mask, pos = _chunk(shape, 100 + n, counts, row0, prefix)
    O, ref = pair.prefill(0, ids, Q, K, V, mask, pos, workspace=ws)
    _check_chunk_outputs(O, ref, mask, Hq)
    pair.check_cache(ids)
    # accept about half of each chunk, poison what the truncate leaves, verify again
    lens = [p + c for p, c in zip(prefix, counts)]
    keep = [p + (c + 1) // 2 for p, c in zip(prefix, counts)]
    from test_gpu_parity import _poison_stale
    for s, m in zip(ids, keep):
        pair.truncate(s, m)
        _poison_stale(pair, s, [0])
    torch.cuda.synchronize()
    counts2 = [max(1, n - 1), n, 0, n]
    row02 = [1 if n > 1 else 0, 0, 0, 0]
    Q, K, V, mask, pos = _chunk(shape, 200 + n, counts2, row02, keep)
    O, ref = pair.prefill(0, ids, Q, K, V, mask, pos, workspace=ws)
    _check_chunk_outputs(O, ref, mask, Hq)
    pair.check_cache(ids)
    assert lens != keep or n == 1


def test_chunks_many_splits_and_attention_rows():
    """A 40000-token cache (over a hundred splits per sequence), an 8-token chunk
    on it, then gqa_attention on 12 rows inside the cache on both kernels."""
    import causal_gqa_attention_attn_amd as lib
    say("case: 8-token chunk on a 40000-token cache; gqa_attention rows 20000..20011")
    Hq, Hkv, d = 32, 8, 128
    T0 = 40000
    pair = Pair(1, Hkv, d, 2600, 1, 2600, torch.bfloat16, 5e5)
    _build_prefix(pair, [0], [T0], Hq, 4711)
    ws = pair.chunk_workspace(1, Hq, 16)
    shape = W.AttnShape(B=1, n=8, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=5e5)
    Q, K, V, mask, pos = _chunk(shape, 4712, [8], [0], [T0])
    O, ref = pair.prefill(0, [0], Q, K, V, mask, pos, workspace=ws)
    _check_chunk_outputs(O, ref, mask, Hq)
    pair.check_cache([0])
    # rows inside the cache through gqa_attention: split-T vs oracle, tiled vs oracle
    Qm = W.normal((1, Hq, 12, d), 4713, torch.bfloat16)
    ones = torch.ones((1, 12), dtype=torch.uint8)
    p = torch.arange(20000, 20012, dtype=torch.int32)[None]
    ref = pair.ref.prefill_rows(0, 0, as_f32(Qm[0]), list(range(20000, 20012)))
    for w in (ws, None):
        Om = torch.full((1, Hq, 12, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lib.gqa_attention(pair.gpu.handle, 0, [0], Qm.cuda(), ones, p, Om, w)
        torch.cuda.synchronize()
        compare_rows(Om[0], ref, torch.bfloat16)


def test_shared_workspace_across_call_shapes():
    """One zero-filled workspace, passed with the same size to decode and chunk
    calls of different B, Hq and chunk length in turn: each call must see its
    own flags at zero whatever the previous call left in the record slots."""
    import causal_gqa_attention_attn_amd as lib
    say("case: one workspace shared by decode (B=4, B=1) and chunk (B=2 n=16, B=4 n=3) calls")
    Hkv, d = 8, 128
    prefix = [3000, 700, 5000, 1]
    B = len(prefix)
    pair = Pair(1, Hkv, d, 4 * 340, B, 340, torch.bfloat16, 1e4)
    ids = list(range(B))
    _build_prefix(pair, ids, prefix, 32, 31337)
    nb = max(lib.gqa_attention_workspace_size(pair.gpu.handle, B, 64, 16),
             lib.gqa_workspace_size(pair.gpu.handle, B, 64))
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    lens = list(prefix)
    for step, (kind, sub, Hq, n) in enumerate([("decode", ids, 32, 1), ("chunk", [0, 2], 64, 16),
                                              ("decode", [2], 32, 1), ("chunk", ids, 32, 3),
                                              ("decode", ids, 64, 1), ("chunk", [1, 3], 64, 5)]):
        shape = W.AttnShape(B=len(sub), n=n, Hq=Hq, Hkv=Hkv, d=d, dtype=torch.bfloat16, theta=1e4)
        if kind == "decode":
            st = W.decode_step_inputs(shape, 77 + step, 0)
            qd = st.q.cuda()
            o = torch.full_like(qd, float("nan"))
            lib.gqa_decode_step(pair.gpu.handle, 0, sub, qd, st.k.cuda(), st.v.cuda(), o, ws)
            torch.cuda.synchronize()
            cur = [lens[s] for s in sub]
            pair.ref.append(0, sub, as_f32(st.k), as_f32(st.v), np.ones((len(sub), 1), np.uint8),
                            np.array([[c] for c in cur]))
            ref = pair.ref.decode(0, sub, as_f32(st.q), [c + 1 for c in cur])
            compare_rows(o, ref, torch.bfloat16)
            for s in sub:
                lens[s] += 1
        else:
            Q, K, V, mask, pos = _chunk(shape, 500 + step, [n] * len(sub), [0] * len(sub), [lens[s] for s in sub])
            O, ref = pair.prefill(0, sub, Q, K, V, mask, pos, workspace=ws)
            _check_chunk_outputs(O, ref, mask, Hq)
            for s in sub:
                lens[s] += n
    pair.check_cache(ids)


def test_chunk_workspace_too_small_changes_nothing():
    """A split-T prefill whose workspace is too small fails with GQA_ERR_ARG
    before the cache changes."""
    import causal_gqa_attention_attn_amd as lib
    say("case: chunk prefill with a too-small workspace")
    pair = Pair(1, 8, 128, 200, 1, 200, torch.bfloat16, 1e4)
    _build_prefix(pair, [0], [3000], 32, 5150)
    small = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    shape = W.AttnShape(B=1, n=4, Hq=32, Hkv=8, d=128, dtype=torch.bfloat16, theta=1e4)
    Q, K, V, mask, pos = _chunk(shape, 5151, [4], [0], [3000])
    O = torch.zeros((1, 32, 4, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.GqaError) as e:
        lib.gqa_prefill(pair.gpu.handle, 0, [0], Q.cuda(), K.cuda(), V.cuda(), mask, pos, O, small)
    assert e.value.name == "ARG"
    assert lib.gqa_cache_length(pair.gpu.handle, 0, 0) == 3000
    pair.check_cache([0])
