"""Seeded random sequences of cache operations on the GPU, step by step against
the float64 oracle.

Each step draws one operation: a prefill (ragged lengths, sometimes with
padding between valid tokens), a short chunk on the split-T kernel, decode
steps (fused and not), a fork, a truncate, a remap or a release.  Outputs are
compared after every step, the whole cache (tables, free list, reference
counts, resident bytes) every few steps.  A second run does the same on a
sliding-window ring cache, where forks and edits are not allowed.
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


def _rows(rng, n, count, holes):
    """count valid rows out of n, contiguous from a random start or scattered."""
    if count == 0:
        return []
    if holes and count < n:
        return sorted(rng.choice(n, size=count, replace=False).tolist())
    r0 = int(rng.integers(0, n - count + 1))
    return list(range(r0, r0 + count))


def _inputs(shape, seed, rows_per_b, starts):
    B, n = shape.B, shape.n
    Q = W.normal((B, shape.Hq, n, shape.d), seed, shape.dtype)
    K = W.normal((B, shape.Hkv, n, shape.d), seed + 100_000, shape.dtype)
    V = W.normal((B, shape.Hkv, n, shape.d), seed + 200_000, shape.dtype)
    mask = torch.zeros((B, n), dtype=torch.uint8)
    pos = torch.full((B, n), -1, dtype=torch.int32)
    for b, rows in enumerate(rows_per_b):
        if rows:
            mask[b, rows] = 1
            pos[b, rows] = torch.arange(starts[b], starts[b] + len(rows), dtype=torch.int32)
    return Q, K, V, mask, pos


def _oracle_refuses(pair, call):
    """The oracle's error code for a call on a copy of its state, or None."""
    import copy
    from oracle.cache_model import OracleError
    try:
        call(copy.deepcopy(pair.ref))
    except OracleError as e:
        return e.code
    return None


def _run(seed, window):
    import causal_gqa_attention_attn_amd as lib
    rng = np.random.default_rng(seed)
    Hq, Hkv, d, dtype = 16, 4, 128, torch.bfloat16
    S, R = 6, 48
    pages = S * R // 4          # small enough that some calls run out of pages (and must be refused)
    pair = Pair(1, Hkv, d, pages, S, R, dtype, 1e4, max_position=4096,
                free_order=W.page_order(pages, seed + 1), window=window)
    pair.gpu.k_pool.fill_(float("nan"))
    pair.gpu.v_pool.fill_(float("nan"))
    ws = pair.chunk_workspace(S, Hq, 16)

    def length(s):
        return pair.ref.cache_length(s, 0)

    stale = False          # a fork since the last launch: the device block table catches up at the next one
    for step in range(120):
        op = rng.choice(["prefill", "chunk", "decode", "fork", "truncate", "remap", "release"],
                        p=[0.3, 0.2, 0.2, 0.1, 0.1, 0.05, 0.05])
        if window and op in ("fork", "truncate"):
            op = "decode"
        if op in ("prefill", "chunk"):
            ids = sorted(rng.choice(S, size=int(rng.integers(1, 4)), replace=False).tolist())
            n = int(rng.integers(2, 120)) if op == "prefill" else int(rng.integers(1, 17))
            counts = [int(rng.integers(0, n + 1)) for _ in ids]
            holes = op == "prefill" and rng.random() < 0.4
            rows = [_rows(rng, n, c, holes) for c in counts]
            shape = W.AttnShape(B=len(ids), n=n, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, theta=1e4)
            Q, K, V, mask, pos = _inputs(shape, 1000 * seed + step, rows, [length(s) for s in ids])
            say(f"  step {step}: {op} seqs {ids} n={n} counts={counts} holes={holes}")
            code = _oracle_refuses(pair, lambda m: m.append(0, ids, as_f32(K), as_f32(V), mask.numpy(), pos.numpy()))
            if code:
                with pytest.raises(lib.GqaError) as e:
                    lib.gqa_prefill(pair.gpu.handle, 0, ids, Q.cuda(), K.cuda(), V.cuda(), mask, pos,
                                    torch.empty_like(Q).cuda(), ws if op == "chunk" else None)
                assert e.value.name == code
                say(f"    refused: {code}")
                continue
            O, ref = pair.prefill(0, ids, Q, K, V, mask, pos, workspace=ws if op == "chunk" else None)
            stale = False
            valid = mask.numpy().astype(bool)[:, None, :].repeat(Hq, 1)
            compare_rows(O, ref, dtype, rows_mask=valid)
            assert np.all(as_f32(O)[~valid] == 0.0)
        elif op == "decode":
            ids = [s for s in range(S) if length(s) > 0]
            if not ids:
                continue
            fused = bool(rng.random() < 0.5)
            say(f"  step {step}: decode ({'fused' if fused else 'append + decode'}) seqs {ids}")
            st = W.decode_step_inputs(W.AttnShape(B=len(ids), n=1, Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, theta=1e4),
                                      seed * 100 + step, 0)
            ones = np.ones((len(ids), 1), np.uint8)
            at = np.array([[length(s)] for s in ids], np.int32)
            code = _oracle_refuses(pair, lambda m: m.append(0, ids, as_f32(st.k), as_f32(st.v), ones, at))
            if code:
                with pytest.raises(lib.GqaError) as e:
                    lib.gqa_decode_step(pair.gpu.handle, 0, ids, st.q.cuda(), st.k.cuda(), st.v.cuda(),
                                        torch.empty_like(st.q).cuda(), pair.workspace(len(ids), Hq))
                assert e.value.name == code
                say(f"    refused: {code}")
                continue
            o, r = pair.step_fused(0, ids, st) if fused else pair.step(0, ids, st)
            stale = False
            compare_rows(o, r, dtype)
        elif op == "fork":
            src = [s for s in range(S) if length(s) > 0]
            dst = [s for s in range(S) if length(s) == 0]
            if not src or not dst:
                continue
            a, b = int(rng.choice(src)), int(rng.choice(dst))
            m = int(rng.integers(0, length(a) + 1))
            say(f"  step {step}: fork {a} -> {b} at {m}")
            pair.fork(a, b, m)
            stale = True
        elif op == "truncate":
            live = [s for s in range(S) if length(s) > 0]
            if not live:
                continue
            s = int(rng.choice(live))
            m = int(rng.integers(0, length(s) + 1))
            say(f"  step {step}: truncate {s} to {m}")
            pair.truncate(s, m)
        elif op == "release":
            live = [s for s in range(S) if length(s) > 0]
            if not live:
                continue
            s = int(rng.choice(live))
            say(f"  step {step}: release {s}")
            pair.truncate(s, 0)
        elif op == "remap":
            used = sorted({p for s in range(S) for p in pair.ref.page_table(s)})
            free = list(pair.ref.free)
            k = min(len(used), len(free), 6)
            if k == 0:
                continue
            src = rng.choice(used, size=k, replace=False).tolist()
            dst = rng.choice(free, size=k, replace=False).tolist()
            say(f"  step {step}: remap {src} -> {dst}")
            lib.kv_cache_remap(pair.gpu.handle, src, dst)
            pair.ref.remap(src, dst)
            stale = False
        if step % 10 == 9:
            pair.check_cache(list(range(S)), device_tables=not stale)
    pair.check_cache(list(range(S)), device_tables=False)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_random_operations(seed):
    say(f"case: random operations, seed {seed}")
    _run(seed, 0)


@pytest.mark.parametrize("seed", [4, 5])
def test_random_operations_window(seed):
    say(f"case: random operations on a W=200 ring cache, seed {seed}")
    _run(seed, 200)
