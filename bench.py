#!/usr/bin/env python3
"""Throughput of the attention path on one MI355X, Grok-1-shaped workload.

One step = one pass of the whole path over one batch of synthetic input:
  * kv_cache_truncate of the prompt sequence to 0 (host; frees its pages);
  * prefill of B=1, n=8192, Hq=48, Hkv=8, d=128 (bf16, rotation theta 1e4):
    kv_cache_append (validation, page reservation, block-table patch, fused
    rotation + paged cache write) then gqa_attention (the MFMA causal kernel);
    together these are exactly gqa_prefill;
  * decode at T=8192 over a 64-layer bf16 cache: per layer gqa_decode_step,
    which appends the new token (position 8191) and decodes one query reading
    all 8192 slots, in one launch (2^31 bytes of K/V over the 64 layers).  The 64-layer loop is captured
    once as a HIP graph and replayed, so every step does the same work.

Inputs are resident in HBM before the timed region.  ``value`` is the causal
prefill throughput 2*B*Hq*n^2*d / (append + attention time, HIP events);
``decode`` reports the decode KV-read rate over the 64 layers.  ``roofline``
is the prefill attention kernel: algorithmic flops of one launch over its
event-timed duration, against the bf16 dense MFMA peak (beside it, as
context, the vendor library's 8192^3 bf16 GEMM rate measured in the same run); ``roofline_decode``
is one layer of the decode graph (one decode_bf16_kernel launch: append,
split-T attention and split combine) against HBM.  ``cpu_baseline`` times the float64 oracle on a bounded sample of the
same prefill (query rows spread over the sequence) on this host's cores.
``other_configs`` reports the other measured configurations on the same
GPU, each timed with HIP events around 20 back-to-back calls (host-only
truncates between calls), median and minimum of 5 such batches:
  * Llama-shaped prefill: B=8, n=2048, Hq=32, Hkv=8, d=128 (gqa_prefill);
  * serving decode: one gqa_decode_step of 64 sequences with lengths
    log-uniform in [512, 32768] on one layer (about 2.2 GB of K/V);
  * speculative verify: a 4- and an 8-token chunk appended to and attended
    over each of those 64 caches (gqa_prefill with a workspace, which takes
    the split-T kernel), beside the same call on the tiled prefill kernel;
  * shared prompt: one gqa_decode_step of 64 requests forked from one
    8192-token prompt with 512 tokens of their own (prefix sharing);
  * masks with holes: the Llama-shaped prefill with 1536 valid tokens per
    row in 16 runs separated by padding, beside the same tokens right-padded;
  * sliding window of 4096 positions: the Grok-shaped prefill (flops
    4*Hq*d per visible (query, key) pair) and gqa_decode of the 64 serving
    sequences over ring caches (K/V bytes of the window);
  * edit re-prefill: 16 sequences of 4096 tokens, each truncated at a seeded
    m_b and its suffix re-prefilled (gqa_prefill on a non-empty cache);
    flops 2*Hq*d*(n^2 - m_b^2).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-other-configs]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
B, N, HQ, HKV, D, THETA, LAYERS = 1, 8192, 48, 8, 128, 1e4, 64


def _sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _traffic(kernel_key, source):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the kernel source that is built now; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel_key)
    if not rec or rec.get("source_sha256") != _sha(source):
        return None
    return rec.get("hbm_bytes_per_launch")


def _profiled_us(kernel_key, source):
    """Average duration (us) of a kernel in the committed rocprofv3 kernel trace
    of the same workload, if it was taken on the kernel source built now."""
    path = os.path.join(ROOT, "profiles", "kernels.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel_key)
    if not rec or rec.get("source_sha256") != _sha(source):
        return None
    return rec.get("avg_us")


def _library_gemm(torch, n=8192, reps=10):
    """Dense bf16 GEMM rate of the vendor library (torch.matmul -> hipBLASLt)
    on n x n x n random N(0,1) operands on this GPU: the practical matrix-core
    rate of a plain contraction under the same clock and power limits, reported
    beside the attention kernel's roofline as context (not its peak)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(1234)
    a = torch.randn((n, n), device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn((n, n), device="cuda", dtype=torch.bfloat16, generator=g)
    for _ in range(3):
        c = a @ b
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    return 2.0 * n ** 3 / (ms * 1e-3) / 1e12


def _blas_info():
    """(threads, description) of the BLAS numpy calls into."""
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return (int(i.get("num_threads") or 1),
                        f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer')}, "
                        f"{os.path.basename(i.get('filepath', ''))})")
    except Exception:
        pass
    return os.cpu_count() or 1, "unknown"


def _host():
    """CPU model, physical cores and logical CPUs of this host."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        import psutil
        phys = psutil.cpu_count(logical=False)
    except Exception:
        phys = None
    return {"cpu_model": model, "physical_cores": phys, "logical_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def _oracle_prefill_rate(m, Q, n, Hq, budget_s, block=64):
    """Causal TFLOP/s of the oracle's prefill rows of one sequence (cache m,
    layer 0): blocks of ``block`` query rows interleaved so that any prefix of
    the list is spread over the sequence, heaviest first within each sweep,
    until ``budget_s`` seconds of work.  4*d*(p+1) flops per row and head."""
    stride = 16 * block
    blocks = [r0 for off in range(stride // block) for r0 in range(n - block - block * off, -1, -stride)]
    rows_done, flops, t_used = 0, 0.0, 0.0
    for r0 in blocks:
        rows = list(range(r0, r0 + block))
        t = time.perf_counter()
        m.prefill_rows(0, 0, Q[:, r0:r0 + block], rows)
        t_used += time.perf_counter() - t
        rows_done += block
        flops += sum(4.0 * D * (p + 1) for p in rows) * Hq
        if t_used >= budget_s:
            break
    return flops / t_used / 1e12, rows_done, t_used


def cpu_baseline(inp, budget_s, W):
    """The float64 oracle as it stands, on bounded samples of the benchmark's
    workloads, on this host's cores:
      * value: the Grok-shaped prefill, blocks of 64 query rows spread over the
        sequence (all 48 heads), until ``budget_s`` seconds of work, with numpy's
        BLAS on all its threads; causal TFLOP/s of the rows done;
      * llama_prefill_1thread: the same measurement on the Llama-shaped
        prefill (one sequence of the B=8 batch) with BLAS held to one thread;
      * decode_step: one oracle decode step (append of the new token and one
        query over the cache) of the Grok-shaped 64-layer decode at T=8192 and
        of the 64-sequence serving decode, timed on a few layers or sequences
        and scaled to the whole step by the keys read."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits
    from oracle.cache_model import CacheModel
    threads, blas = _blas_info()
    K = inp.K.float().numpy()
    V = inp.V.float().numpy()
    Q = inp.Q.float().numpy()
    m = CacheModel(1, HKV, D, 16, N // 16, 1, N // 16, dtype="bf16", rope_theta=THETA, max_position=N)
    m.append(0, [0], K, V, np.ones((1, N), np.uint8), np.arange(N)[None])
    rate, rows_done, t_used = _oracle_prefill_rate(m, Q[0], N, HQ, budget_s)
    out = {"value": rate, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"{rows_done} query rows x {HQ} heads of the n=8192 prefill (blocks of 64 rows "
                     f"spread over the sequence, heaviest first), float64 numpy, {t_used:.1f} s",
           "blas": blas, "blas_threads": threads, **_host()}
    # Llama-shaped prefill on one BLAS thread
    sh = W.LLAMA
    li = W.llama()
    lm = CacheModel(1, sh.Hkv, sh.d, 16, sh.n // 16, 1, sh.n // 16, dtype="bf16", rope_theta=sh.theta,
                    max_position=sh.n)
    lm.append(0, [0], li.K[:1].float().numpy(), li.V[:1].float().numpy(), np.ones((1, sh.n), np.uint8),
              np.arange(sh.n)[None])
    with threadpool_limits(1):
        lrate, lrows, lt = _oracle_prefill_rate(lm, li.Q[0].float().numpy(), sh.n, sh.Hq, budget_s / 3)
    out["llama_prefill_1thread"] = {"value": lrate, "unit": "TFLOP/s", "threads": 1,
                                    "sample": f"{lrows} query rows x {sh.Hq} heads of one n=2048 sequence, "
                                              f"{lt:.1f} s"}
    # decode steps: Grok-shaped (64 layers of 8192 keys), timed on 2 layers
    def step_seconds(model, seq, T, q, k, v, reps=3):
        t = time.perf_counter()
        for _ in range(reps):
            model.truncate(seq, T - 1)
            model.append(0, [seq], k, v, np.ones((1, 1), np.uint8), np.array([[T - 1]]))
            model.decode(0, [seq], q, [T])
        return (time.perf_counter() - t) / reps
    g_layers, g_t = 2, 0.0
    for l in range(g_layers):
        kf = W.normal((1, HKV, N - 1, D), 70000 + l).float().numpy()
        vf = W.normal((1, HKV, N - 1, D), 80000 + l).float().numpy()
        gm = CacheModel(1, HKV, D, 16, N // 16, 1, N // 16, dtype="bf16", rope_theta=THETA, max_position=N + 16)
        gm.append(0, [0], kf, vf, np.ones((1, N - 1), np.uint8), np.arange(N - 1)[None])
        st = W.decode_step_inputs(W.GROK, 1004, l)
        g_t += step_seconds(gm, 0, N, st.q.float().numpy(), st.k.float().numpy(), st.v.float().numpy())
    grok_step = g_t / g_layers * LAYERS
    # serving decode: four sequences near the median length, scaled by keys read
    lens = W.serving_lengths()
    sv = W.SERVING
    order = sorted(range(len(lens)), key=lambda b: abs(lens[b] - sorted(lens)[len(lens) // 2]))[:4]
    s_t, s_keys = 0.0, 0
    st = W.decode_step_inputs(sv, 1005, 0)
    for b in order:
        L = lens[b]
        sm = CacheModel(1, sv.Hkv, sv.d, 16, L // 16 + 2, 1, L // 16 + 2, dtype="bf16", rope_theta=sv.theta,
                        max_position=32770)
        kb = torch.randn((1, sv.Hkv, L, sv.d), generator=torch.Generator().manual_seed(b)).numpy()
        sm.append(0, [0], kb, kb, np.ones((1, L), np.uint8), np.arange(L)[None])
        s_t += step_seconds(sm, 0, L + 1, st.q[b:b + 1].float().numpy(), st.k[b:b + 1].float().numpy(),
                            st.v[b:b + 1].float().numpy())
        s_keys += L + 1
    serving_step = s_t * sum(x + 1 for x in lens) / s_keys
    out["decode_step"] = {
        "grok_64_layers_s": grok_step,
        "grok_gbs": 2.0 * LAYERS * HKV * N * D * 2 / grok_step / 1e9,
        "serving_64_sequences_s": serving_step,
        "serving_gbs": sum((x + 1) * 2 * sv.Hkv * sv.d * 2 for x in lens) / serving_step / 1e9,
        "sample": f"oracle decode step (append + decode) timed on {g_layers} of the 64 Grok-shaped layers and "
                  f"on 4 serving sequences near the median length ({sum(lens[b] for b in order)} cached "
                  f"tokens), scaled by keys read; GB/s counts the bf16 K/V bytes the GPU reads"}
    return out


def _median_ms(fn, before=None, iters=20, warm=3, reps=5):
    """Per-call time of fn() when calls run back to back, as median and minimum
    over ``reps`` batches of ``iters`` calls.  before() runs before every call;
    it is host-only work (a truncate), so the GPU stays busy and the host
    preparation of one call overlaps the kernels of the previous one, as in a
    serving loop."""
    import torch
    for _ in range(warm):
        if before:
            before()
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(iters):
            if before:
                before()
            fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) / iters)
    ts.sort()
    return ts[len(ts) // 2], ts[0]


OTHER = ["llama_prefill", "llama_decode", "serving_decode", "verify_chunks", "shared_prompt_decode",
         "holey_mask_prefill", "window_prefill", "window_decode", "edit_reprefill", "small_latency"]


def other_configs(lib, W, only=None):
    """The other measured configurations; ``only`` names one of OTHER to run it
    alone (a profiling aid)."""
    import numpy as np
    import torch
    res = {}
    want = lambda name: only is None or only == name
    serving_cache = only is None or only in ("serving_decode", "verify_chunks", "window_decode",
                                             "shared_prompt_decode")
    if want("llama_prefill"):
        _llama(lib, W, res)
    if want("llama_decode"):
        _llama_decode(lib, W, res)
    if serving_cache:
        _serving(lib, W, res, want)
    if want("holey_mask_prefill"):
        _holey(lib, W, res)
    if want("window_prefill"):
        _window_prefill(lib, W, res)
    if want("window_decode"):
        _window_decode(lib, W, res)
    if want("edit_reprefill"):
        _edit(lib, W, res)
    if want("small_latency"):
        _small(lib, W, res)
    return res


def _llama(lib, W, res):
    import torch
    inp = W.llama()
    Q, K, V = inp.Q.cuda(), inp.K.cuda(), inp.V.cuda()
    O = torch.empty_like(Q)
    sh = W.LLAMA
    pre = lib.PagedCache(1, sh.Hkv, sh.d, sh.B * (sh.n // 16) + 16, sh.B, sh.n // 16 + 2, dtype=torch.bfloat16,
                         rope_theta=sh.theta, max_position=sh.n + 32)
    ids = list(range(sh.B))
    med, mn = _median_ms(lambda: lib.gqa_prefill(pre.handle, 0, ids, Q, K, V, inp.mask, inp.positions, O),
                         before=lambda: [lib.kv_cache_truncate(pre.handle, b, 0) for b in ids])
    flops = sum(2.0 * sh.Hq * sh.d * n * n for n in inp.lengths)
    res["llama_prefill"] = {"workload": "causal prefill B=8 n=2048 Hq=32 Hkv=8 d=128 (gqa_prefill)",
                            "tflops": round(flops / (med * 1e-3) / 1e12, 1),
                            "frac": round(flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                            "ms_median": round(med, 4), "ms_min": round(mn, 4)}
    pre.close()


def _llama_decode(lib, W, res):
    """The 64 decode steps that follow the Llama-shaped prefill: each step
    appends one token to each of the 8 sequences and decodes (gqa_decode_step,
    one layer), reading 2 * 8 * 128 * 2 bytes per cached token.  The ~67 MB a
    step reads fits in the 256 MB Infinity Cache, so the steps are timed twice:
    back to back (labelled cache-resident), and with a 512 MiB device read
    between steps, outside the timed span, which evicts the cache (a read
    leaves no dirty lines whose write-back would compete with the step)."""
    import torch
    inp = W.llama()
    sh = W.LLAMA
    cache = lib.PagedCache(1, sh.Hkv, sh.d, sh.B * (sh.n // 16 + 8), sh.B, sh.n // 16 + 8, dtype=torch.bfloat16,
                           rope_theta=sh.theta, max_position=sh.n + 160,
                           free_list_order=W.page_order(sh.B * (sh.n // 16 + 8), 3003))
    ids = list(range(sh.B))
    O = torch.empty_like(inp.Q.cuda())
    lib.gqa_prefill(cache.handle, 0, ids, inp.Q.cuda(), inp.K.cuda(), inp.V.cuda(), inp.mask, inp.positions, O)
    steps = [W.decode_step_inputs(sh, 1003, t) for t in range(64)]
    dev = [(s.q.cuda(), s.k.cuda(), s.v.cuda()) for s in steps]
    o = torch.empty_like(dev[0][0])
    ws = torch.zeros(lib.gqa_workspace_size(cache.handle, sh.B, sh.Hq), dtype=torch.uint8, device="cuda")
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    reset = lambda: [lib.kv_cache_truncate(cache.handle, b, sh.n) for b in ids]
    nbytes = sum(sh.B * (sh.n + t + 1) * 2 * sh.Hkv * sh.d * 2 for t in range(64))
    # eager pass first (uploads the rotation table), then the captures: one
    # graph of the 64 steps and one graph per step.  A replay runs the kernels
    # of its capture (positions 2048.. as captured), whatever the host state.
    reset()
    for q, k, v in dev:
        lib.gqa_decode_step(cache.handle, 0, ids, q, k, v, o, ws)
    torch.cuda.synchronize()
    reset()
    whole = torch.cuda.CUDAGraph()
    with torch.cuda.graph(whole):
        for q, k, v in dev:
            lib.gqa_decode_step(cache.handle, 0, ids, q, k, v, o, ws)
    reset()
    per_step = []
    for q, k, v in dev:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            lib.gqa_decode_step(cache.handle, 0, ids, q, k, v, o, ws)
        per_step.append(g)
    torch.cuda.synchronize()
    out = {}
    # cache-resident: the 64-step graph back to back (the ~67 MB a step reads
    # stays in the 256 MB Infinity Cache from one replay to the next)
    whole.replay()
    spans = []
    for _ in range(5):
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        whole.replay()
        z.record()
        torch.cuda.synchronize()
        spans.append(a.elapsed_time(z) * 1e3 / 64)
    spans.sort()
    us = spans[len(spans) // 2]
    out["cache_resident"] = {"us_per_step": round(us, 2), "gbs": round(nbytes / 64 / (us * 1e-6) / 1e9, 1),
                             "frac": round(nbytes / 64 / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                             "label": "LLC-resident: the steps' K/V fit in the 256 MB Infinity Cache"}
    # flushed: a 512 MiB device read before every step, outside the timed span
    # (it keeps the queue busy, so the events see GPU time only)
    ev = []
    sink = torch.zeros(64, dtype=torch.float32, device="cuda")
    for t, g in enumerate(per_step):
        torch.sum(flush, dim=0, keepdim=True, out=sink[t:t + 1])
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        z.record()
        ev.append((a, z))
    torch.cuda.synchronize()
    us_f = [a.elapsed_time(z) * 1e3 for a, z in ev]
    mean_f = sum(us_f) / len(us_f)
    out["cache_flushed"] = {"us_per_step": round(mean_f, 2), "gbs": round(nbytes / 64 / (mean_f * 1e-6) / 1e9, 1),
                            "frac": round(nbytes / 64 / (mean_f * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                            "label": "512 MiB read between steps (outside the timed span) evicts the cache"}
    lib.gqa_workspace_status(cache.handle, ws)
    res["llama_decode"] = {"workload": "64 gqa_decode_step calls after the Llama-shaped prefill, B=8, T=2049..2112, "
                                       "Hq=32 Hkv=8 d=128, one layer (~67 MB of K/V per step)", **out}
    cache.close()


def _small(lib, W, res):
    """Latency of the two small configurations: the float32 toy (B=1, n=4,
    Hq=2, Hkv=1, d=4: prefill, then a decode step) and the ragged bf16 batch
    (B=4, n=128, Hq=8, Hkv=2, d=64: prefill, then a decode step of the 4)."""
    import torch
    pre, steps = W.tiny()
    tc = lib.PagedCache(1, 1, 4, 8, 1, 4, dtype=torch.float32, rope_theta=0.0)
    Q, K, V = pre.Q.cuda(), pre.K.cuda(), pre.V.cuda()
    O = torch.empty_like(Q)
    q, k, v = steps[0].q.cuda(), steps[0].k.cuda(), steps[0].v.cuda()
    o = torch.empty_like(q)
    med_p, _ = _median_ms(lambda: lib.gqa_prefill(tc.handle, 0, [0], Q, K, V, pre.mask, pre.positions, O),
                          before=lambda: lib.kv_cache_truncate(tc.handle, 0, 0))
    med_d, _ = _median_ms(lambda: lib.gqa_decode_step(tc.handle, 0, [0], q, k, v, o),
                          before=lambda: lib.kv_cache_truncate(tc.handle, 0, 4))
    tc.close()
    inp = W.ragged()
    sh = inp.shape
    rc = lib.PagedCache(1, sh.Hkv, sh.d, 64, sh.B, 16, dtype=torch.bfloat16, rope_theta=sh.theta)
    Q, K, V = inp.Q.cuda(), inp.K.cuda(), inp.V.cuda()
    O = torch.empty_like(Q)
    ids = list(range(sh.B))
    st = W.decode_step_inputs(sh, 1002, 0)
    q, k, v = st.q.cuda(), st.k.cuda(), st.v.cuda()
    o = torch.empty_like(q)
    ws = torch.zeros(lib.gqa_workspace_size(rc.handle, sh.B, sh.Hq), dtype=torch.uint8, device="cuda")
    rmed_p, _ = _median_ms(lambda: lib.gqa_prefill(rc.handle, 0, ids, Q, K, V, inp.mask, inp.positions, O),
                           before=lambda: [lib.kv_cache_truncate(rc.handle, b, 0) for b in ids])
    lens = [int(x) for x in inp.lengths]
    rmed_d, _ = _median_ms(lambda: lib.gqa_decode_step(rc.handle, 0, ids, q, k, v, o, ws),
                           before=lambda: [lib.kv_cache_truncate(rc.handle, b, lens[b]) for b in ids])
    rc.close()
    res["small_latency"] = {
        "workload": "float32 toy B=1 n=4 Hq=2 Hkv=1 d=4; ragged bf16 B=4 n=128 (lengths U{1..128}) Hq=8 Hkv=2 d=64; "
                    "per-call time of 20 back-to-back calls (median of 5 batches)",
        "tiny_prefill_us": round(med_p * 1e3, 1), "tiny_decode_step_us": round(med_d * 1e3, 1),
        "ragged_prefill_us": round(rmed_p * 1e3, 1), "ragged_decode_step_us": round(rmed_d * 1e3, 1)}


def _serving(lib, W, res, want):
    import torch
    # serving decode
    lens = W.serving_lengths()
    Bs = len(lens)
    sh = W.SERVING
    pages = sum(-(-(x + 16) // 16) for x in lens) + 8
    cache = lib.PagedCache(1, sh.Hkv, sh.d, pages, Bs, 32768 // 16 + 2, dtype=torch.bfloat16, rope_theta=sh.theta,
                           max_position=32770, free_list_order=W.page_order(pages, 1005))
    for b, L in enumerate(lens):
        kf = W.normal_device((1, sh.Hkv, L, sh.d), 91000 + b)
        vf = W.normal_device((1, sh.Hkv, L, sh.d), 92000 + b)
        lib.kv_cache_append(cache.handle, 0, [b], kf, vf, torch.ones((1, L), dtype=torch.uint8),
                            torch.arange(L, dtype=torch.int32)[None])
    st = W.decode_step_inputs(sh, 1005, 0)
    q, k, v = st.q.cuda(), st.k.cuda(), st.v.cuda()
    o = torch.empty_like(q)
    ws = torch.zeros(max(lib.gqa_workspace_size(cache.handle, Bs, sh.Hq),
                         lib.gqa_attention_workspace_size(cache.handle, Bs, sh.Hq, 8)), dtype=torch.uint8,
                     device="cuda")
    ids = list(range(Bs))
    if want("serving_decode"):
        med, mn = _median_ms(lambda: lib.gqa_decode_step(cache.handle, 0, ids, q, k, v, o, ws),
                             before=lambda: [lib.kv_cache_truncate(cache.handle, b, lens[b]) for b in ids])
        lib.gqa_workspace_status(cache.handle, ws)
        nbytes = sum((L + 1) * 2 * sh.Hkv * sh.d * 2 for L in lens)
        gbs = nbytes / (med * 1e-3) / 1e9
        res["serving_decode"] = {"workload": "gqa_decode_step of 64 sequences, lengths log-uniform [512, 32768], "
                                             "Hq=32 Hkv=8 d=128, one layer",
                                 "kv_bytes": nbytes, "gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
                                 "us_median": round(med * 1e3, 1), "us_min": round(mn * 1e3, 1)}
    # speculative verify: a chunk of n draft tokens per sequence on the same caches,
    # split-T kernel (with workspace) beside the tiled prefill kernel (without)
    for n in ((4, 8) if want("verify_chunks") else ()):
        chunk = W.prefill_inputs(W.AttnShape(B=Bs, n=n, Hq=sh.Hq, Hkv=sh.Hkv, d=sh.d, dtype=sh.dtype,
                                             theta=sh.theta), 1007 + n, start=lens)
        Qc, Kc, Vc = chunk.Q.cuda(), chunk.K.cuda(), chunk.V.cuda()
        Oc = torch.empty_like(Qc)
        trunc = lambda: [lib.kv_cache_truncate(cache.handle, b, lens[b]) for b in ids]
        med, mn = _median_ms(lambda: lib.gqa_prefill(cache.handle, 0, ids, Qc, Kc, Vc, chunk.mask, chunk.positions,
                                                     Oc, ws), before=trunc)
        tmed, _ = _median_ms(lambda: lib.gqa_prefill(cache.handle, 0, ids, Qc, Kc, Vc, chunk.mask, chunk.positions,
                                                      Oc), before=trunc, iters=5, reps=3)
        nbytes = sum((L + n) * 2 * sh.Hkv * sh.d * 2 for L in lens)
        gbs = nbytes / (med * 1e-3) / 1e9
        res[f"verify_chunk_n{n}"] = {
            "workload": f"gqa_prefill of a {n}-token chunk on each of the 64 serving caches (append + attention), "
                        "Hq=32 Hkv=8 d=128, one layer, split-T kernel",
            "kv_bytes": nbytes, "gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
            "us_median": round(med * 1e3, 1), "us_min": round(mn * 1e3, 1),
            "tiled_kernel_us_median": round(tmed * 1e3, 1)}
    lib.gqa_workspace_status(cache.handle, ws)
    trunc = None
    cache.close()
    if not want("shared_prompt_decode"):
        return
    # shared system prompt: 64 requests forked from one 8192-token prompt, each
    # with 512 tokens of its own, decoding together; the prompt's pages are
    # stored once and read by every request
    P0, OWN = 8192, 512
    pages = P0 // 16 + Bs * (OWN // 16 + 1) + 8
    sc = lib.PagedCache(1, sh.Hkv, sh.d, pages, Bs + 1, (P0 + OWN) // 16 + 2, dtype=torch.bfloat16,
                        rope_theta=sh.theta, max_position=P0 + OWN + 16)
    kf, vf = W.normal_device((1, sh.Hkv, P0, sh.d), 93000), W.normal_device((1, sh.Hkv, P0, sh.d), 93001)
    lib.kv_cache_append(sc.handle, 0, [Bs], kf, vf, torch.ones((1, P0), dtype=torch.uint8),
                        torch.arange(P0, dtype=torch.int32)[None])
    for b in range(Bs):
        lib.kv_cache_fork(sc.handle, Bs, b, P0)
    ko, vo = W.normal_device((Bs, sh.Hkv, OWN, sh.d), 93002), W.normal_device((Bs, sh.Hkv, OWN, sh.d), 93003)
    lib.kv_cache_append(sc.handle, 0, ids, ko, vo, torch.ones((Bs, OWN), dtype=torch.uint8),
                        (P0 + torch.arange(OWN, dtype=torch.int32))[None].repeat(Bs, 1))
    del kf, vf, ko, vo
    med, mn = _median_ms(lambda: lib.gqa_decode_step(sc.handle, 0, ids, q, k, v, o, ws),
                         before=lambda: [lib.kv_cache_truncate(sc.handle, b, P0 + OWN) for b in ids])
    logical = Bs * (P0 + OWN + 1) * 2 * sh.Hkv * sh.d * 2
    stored = (P0 + Bs * (OWN + 1)) * 2 * sh.Hkv * sh.d * 2
    res["shared_prompt_decode"] = {
        "workload": "gqa_decode_step of 64 requests forked from one 8192-token prompt (kv_cache_fork), "
                    "512 own tokens each, Hq=32 Hkv=8 d=128, one layer",
        "logical_kv_bytes": logical, "stored_kv_bytes": stored,
        "logical_gbs": round(logical / (med * 1e-3) / 1e9, 1),
        "stored_gbs": round(stored / (med * 1e-3) / 1e9, 1),
        "us_median": round(med * 1e3, 1), "us_min": round(mn * 1e3, 1),
        "note": "the prompt's 32 MiB of pages are read by all 64 requests; after the first the reads "
                "come from L2 and the 256 MB last-level cache, so the logical rate is not an HBM rate"}
    sc.close()


def _holey(lib, W, res):
    import numpy as np
    import torch
    # masks with holes: 8 rows of 2048 rectangular slots, 1536 valid tokens each in
    # 16 runs separated by padding, beside the same tokens right-padded
    sh = W.LLAMA
    nv, runs = 1536, 16
    rng = np.random.default_rng(1008)
    hole_rows = []
    per_run = nv // runs
    for b in range(sh.B):
        # the padding rows: a random leading gap, 15 inner gaps of at least one row, a tail
        extra = rng.multinomial(sh.n - nv - (runs - 1), [1.0 / (runs + 1)] * (runs + 1))
        rows, r = [], int(extra[0])
        for run in range(runs):
            rows.extend(range(r, r + per_run))
            r += per_run + (1 + int(extra[run + 1]) if run + 1 < runs else 0)
        hole_rows.append(rows)
    inp = W.prefill_inputs(W.AttnShape(B=sh.B, n=sh.n, Hq=sh.Hq, Hkv=sh.Hkv, d=sh.d, dtype=sh.dtype,
                                       theta=sh.theta), 1008, lengths=[nv] * sh.B)
    Qh, Kh, Vh = inp.Q.cuda(), inp.K.cuda(), inp.V.cuda()
    Oh = torch.empty_like(Qh)
    hm = torch.zeros((sh.B, sh.n), dtype=torch.uint8)
    hp = torch.full((sh.B, sh.n), -1, dtype=torch.int32)
    for b, rows in enumerate(hole_rows):
        hm[b, rows] = 1
        hp[b, rows] = torch.arange(nv, dtype=torch.int32)
    pre = lib.PagedCache(1, sh.Hkv, sh.d, sh.B * (sh.n // 16) + 16, sh.B, sh.n // 16 + 2, dtype=torch.bfloat16,
                         rope_theta=sh.theta, max_position=sh.n + 32)
    ids = list(range(sh.B))
    reset = lambda: [lib.kv_cache_truncate(pre.handle, b, 0) for b in ids]
    med, mn = _median_ms(lambda: lib.gqa_prefill(pre.handle, 0, ids, Qh, Kh, Vh, hm, hp, Oh), before=reset)
    rmed, _ = _median_ms(lambda: lib.gqa_prefill(pre.handle, 0, ids, Qh, Kh, Vh, inp.mask, inp.positions, Oh),
                         before=reset)
    flops = sh.B * 2.0 * sh.Hq * sh.d * nv * nv
    res["holey_mask_prefill"] = {
        "workload": "gqa_prefill B=8, 2048 rectangular rows, 1536 valid tokens per row in 16 runs separated "
                    "by padding, Hq=32 Hkv=8 d=128",
        "tflops": round(flops / (med * 1e-3) / 1e12, 1), "ms_median": round(med, 4), "ms_min": round(mn, 4),
        "right_padded_ms_median": round(rmed, 4)}
    pre.close()


WIN = 4096


def _window_prefill(lib, W, res):
    import torch
    # sliding window W = 4096: the Grok-shaped prefill (one call, the ring holds
    # the whole prompt)
    sh = W.GROK
    inp = W.grok()
    Qg, Kg, Vg = inp.Q.cuda(), inp.K.cuda(), inp.V.cuda()
    Og = torch.empty_like(Qg)
    wc = lib.PagedCache(1, sh.Hkv, sh.d, sh.n // 16 + 8, 1, sh.n // 16 + 2, dtype=torch.bfloat16,
                        rope_theta=sh.theta, max_position=sh.n + 32, window=WIN)
    med, mn = _median_ms(lambda: lib.gqa_prefill(wc.handle, 0, [0], Qg, Kg, Vg, inp.mask, inp.positions, Og),
                         before=lambda: lib.kv_cache_truncate(wc.handle, 0, 0), iters=10, reps=3)
    visible = sum(min(p + 1, WIN) for p in range(sh.n))
    flops = 4.0 * sh.Hq * sh.d * visible
    res["window_prefill"] = {
        "workload": "gqa_prefill B=1 n=8192 Hq=48 Hkv=8 d=128 with a 4096-position sliding window",
        "tflops": round(flops / (med * 1e-3) / 1e12, 1),
        "frac": round(flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "ms_median": round(med, 4), "ms_min": round(mn, 4)}
    wc.close()


def _window_decode(lib, W, res):
    import torch
    # one decode step of the 64 serving sequences over rings of 4096 + 2048
    # tokens, filled in 2048-token chunks
    sh = W.SERVING
    Bs = 64
    st = W.decode_step_inputs(sh, 1005, 0)
    q = st.q.cuda()
    o = torch.empty_like(q)
    R = WIN // 16 + 1 + 2048 // 16
    lens = W.serving_lengths()
    pages = sum(min(R, -(-(x + 1) // 16)) for x in lens) + 8
    wc = lib.PagedCache(1, sh.Hkv, sh.d, pages, Bs, R, dtype=torch.bfloat16, rope_theta=sh.theta,
                        max_position=32770, free_list_order=W.page_order(pages, 1009), window=WIN)
    for b, L in enumerate(lens):
        for c0 in range(0, L, 2048):
            n = min(2048, L - c0)
            kf = W.normal_device((1, sh.Hkv, n, sh.d), 94000 + b * 16 + c0 // 2048)
            vf = W.normal_device((1, sh.Hkv, n, sh.d), 95000 + b * 16 + c0 // 2048)
            lib.kv_cache_append(wc.handle, 0, [b], kf, vf, torch.ones((1, n), dtype=torch.uint8),
                                torch.arange(c0, c0 + n, dtype=torch.int32)[None])
    del kf, vf
    ids = list(range(Bs))
    wws = torch.zeros(lib.gqa_workspace_size(wc.handle, Bs, sh.Hq), dtype=torch.uint8, device="cuda")
    # gqa_decode (the attention read alone): a ring is not truncated back between calls
    med, mn = _median_ms(lambda: lib.gqa_decode(wc.handle, 0, ids, q, lens, o, wws))
    nbytes = sum(min(L, WIN) * 2 * sh.Hkv * sh.d * 2 for L in lens)
    gbs = nbytes / (med * 1e-3) / 1e9
    res["window_decode"] = {
        "workload": "gqa_decode of the 64 serving sequences with a 4096-position sliding window over "
                    "ring caches, Hq=32 Hkv=8 d=128, one layer",
        "kv_bytes": nbytes, "gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
        "us_median": round(med * 1e3, 1), "us_min": round(mn * 1e3, 1)}
    lib.gqa_workspace_status(wc.handle, wws)
    wc.close()


def _edit(lib, W, res):
    import torch
    # edit re-prefill
    sh = W.EDIT
    full = W.prefill_inputs(sh, 1006)
    ms = W.edit_points(sh.B, sh.n)
    lens = [sh.n - m for m in ms]
    suffix = W.prefill_inputs(W.AttnShape(B=sh.B, n=max(lens), Hq=sh.Hq, Hkv=sh.Hkv, d=sh.d, dtype=sh.dtype,
                                          theta=sh.theta), 2006, lengths=lens, start=ms)
    cache = lib.PagedCache(1, sh.Hkv, sh.d, sh.B * (sh.n // 16) + 16, sh.B, sh.n // 16 + 2, dtype=torch.bfloat16,
                           rope_theta=sh.theta, max_position=sh.n + 32)
    ids = list(range(sh.B))
    Of = torch.empty((sh.B, sh.Hq, sh.n, sh.d), dtype=torch.bfloat16, device="cuda")
    lib.gqa_prefill(cache.handle, 0, ids, full.Q.cuda(), full.K.cuda(), full.V.cuda(), full.mask, full.positions, Of)
    Qs, Ks, Vs = suffix.Q.cuda(), suffix.K.cuda(), suffix.V.cuda()
    Os = torch.empty_like(Qs)
    med, mn = _median_ms(lambda: lib.gqa_prefill(cache.handle, 0, ids, Qs, Ks, Vs, suffix.mask, suffix.positions, Os),
                         before=lambda: [lib.kv_cache_truncate(cache.handle, b, m) for b, m in zip(ids, ms)])
    flops = sum(2.0 * sh.Hq * sh.d * (sh.n * sh.n - m * m) for m in ms)
    res["edit_reprefill"] = {"workload": "16 x 4096 cached, truncate at seeded m_b, re-prefill the suffix "
                                         "(gqa_prefill), Hq=32 Hkv=8 d=128",
                             "tflops": round(flops / (med * 1e-3) / 1e12, 1),
                             "frac": round(flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                             "ms_median": round(med, 4), "ms_min": round(mn, 4)}
    cache.close()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--prefill-only", action="store_true", help="skip the decode part (profiling aid)")
    ap.add_argument("--no-other-configs", action="store_true", help="skip the Llama, serving and edit measurements")
    ap.add_argument("--only", choices=OTHER, help="run one of the other configurations alone (profiling aid)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only copy 256 MiB device-to-device 5 times (calibrates rocprofv3 byte counters)")
    ap.add_argument("--gemm-probe", action="store_true",
                    help="only time the library's 8192^3 bf16 GEMM (profiling aid)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this library has no "
              f"multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    import causal_gqa_attention_attn_amd as lib

    torch.cuda.set_device(0)
    dev = "cuda"
    if args.copy_probe:
        src = torch.full((256 << 20,), 1, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_per_copy": 256 << 20, "copies": 5}), flush=True)
        return
    if args.gemm_probe:
        print(json.dumps({"library_gemm_bf16_8192_tflops": round(_library_gemm(torch), 1)}), flush=True)
        return
    if args.only:
        print(json.dumps({args.only: other_configs(lib, W, only=args.only)}), flush=True)
        return
    print("bench: generating inputs", file=sys.stderr, flush=True)
    inp = W.grok()
    Q, K, V = inp.Q.to(dev), inp.K.to(dev), inp.V.to(dev)
    O = torch.empty_like(Q)
    mask = inp.mask.numpy()
    pos = inp.positions.numpy()
    pages = N // 16 + 16
    pre = lib.PagedCache(1, HKV, D, pages, 1, pages, dtype=torch.bfloat16, rope_theta=THETA, max_position=N + 16)

    dec = lib.PagedCache(LAYERS, HKV, D, N // 16 + 2, 1, N // 16 + 2, dtype=torch.bfloat16,
                         rope_theta=THETA, max_position=N + 16)
    ones = torch.ones((1, N - 1), dtype=torch.uint8)
    pfill = torch.arange(N - 1, dtype=torch.int32)[None]
    for l in range(LAYERS):
        kf = W.normal_device((1, HKV, N - 1, D), 70000 + l)
        vf = W.normal_device((1, HKV, N - 1, D), 80000 + l)
        lib.kv_cache_append(dec.handle, l, [0], kf, vf, ones, pfill)
    steps_in = [W.decode_step_inputs(W.GROK, 1004, l) for l in range(LAYERS)]
    qd = [s.q.to(dev) for s in steps_in]
    kd = [s.k.to(dev) for s in steps_in]
    vd = [s.v.to(dev) for s in steps_in]
    od = [torch.empty_like(x) for x in qd]
    ws = torch.zeros(lib.gqa_workspace_size(dec.handle, 1, HQ), dtype=torch.uint8, device=dev)
    one = torch.ones((1, 1), dtype=torch.uint8)
    p_new = torch.tensor([[N - 1]], dtype=torch.int32)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def decode_layers():
        for l in range(LAYERS):
            lib.gqa_decode_step(dec.handle, l, [0], qd[l], kd[l], vd[l], od[l], ws)

    # The 64-layer decode loop is launch-bound from Python (two library calls per
    # layer), so it is captured once in a HIP graph and replayed: every replay
    # runs the same kernels with the same arguments (append at position 8191,
    # decode at T=8192) as the eager loop.
    decode_layers()                                  # eager warmup (uploads tables)
    lib.kv_cache_truncate(dec.handle, 0, N - 1)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode_layers()
    lib.kv_cache_truncate(dec.handle, 0, N - 1)
    torch.cuda.synchronize()

    def step(ev):
        lib.kv_cache_truncate(pre.handle, 0, 0)
        ev[0].record(stream)
        lib.kv_cache_append(pre.handle, 0, [0], K, V, mask, pos)
        ev[1].record(stream)
        lib.gqa_attention(pre.handle, 0, [0], Q, mask, pos, O)
        ev[2].record(stream)
        if args.prefill_only:
            return
        ev[3].record(stream)
        graph.replay()
        ev[4].record(stream)

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    print("bench: warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(mk())
    events = [mk() for _ in range(args.steps)]
    torch.cuda.synchronize()
    print("bench: timed steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    mean = lambda xs: sum(xs) / len(xs)
    append_ms = mean([e[0].elapsed_time(e[1]) for e in events])
    attn_ms = mean([e[1].elapsed_time(e[2]) for e in events])
    prefill_ms = append_ms + attn_ms
    flops = 2.0 * B * HQ * N * N * D
    value = flops / (prefill_ms * 1e-3) / 1e12
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    src_prefill = os.path.join(ROOT, "causal_gqa_attention_attn_amd", "csrc", "prefill_bf16.hip")
    out = {
        "metric": "causal prefill attention TFLOP/s (% MFMA peak) + decode KV-read GB/s (% HBM)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V)",
        "config": {"workload": "Grok-1-shaped attention: causal prefill B=1 n=8192 Hq=48 Hkv=8 d=128 "
                               "(one layer, rotation theta 1e4, paged cache of 16-token pages) + "
                               "decode at T=8192 over a 64-layer bf16 cache (2 GiB)",
                   "global_batch": B, "seq_len": N, "parallelism": "none (1 GPU)",
                   "prefill_ms": round(prefill_ms, 4), "cache_write_ms": round(append_ms, 4),
                   "attention_ms": round(attn_ms, 4),
                   "causal_flops": flops, "causal_flops_exact": 2.0 * HQ * D * N * (N + 1)},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": _traffic("prefill_bf16_kernel<128, false>", src_prefill),
                     "kernel": "prefill_bf16_kernel<128, false>",
                     "timing": "HIP events on the launch stream around the attention launch, mean of the timed steps"},
    }
    prof_us = _profiled_us("prefill_bf16_kernel<128, false>", src_prefill)
    if prof_us:
        out["roofline"]["profile_avg_us"] = prof_us
        out["roofline"]["profile_frac"] = round(flops / (prof_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)
    gemm = _library_gemm(torch)
    out["roofline"]["library_gemm_tflops"] = round(gemm, 1)
    out["roofline"]["frac_of_library_gemm"] = round(attn_tflops / gemm, 4)
    out["roofline"]["library_gemm_note"] = ("torch.matmul (hipBLASLt) bf16 8192x8192x8192 on random N(0,1) operands, "
                                            "same GPU and run: the practical rate of a plain contraction here")
    if not args.prefill_only:
        span_ms = mean([e[3].elapsed_time(e[4]) for e in events])
        kv_bytes = 2.0 * LAYERS * HKV * N * D * 2
        per_layer_ms = span_ms / LAYERS
        achieved = kv_bytes / LAYERS / (per_layer_ms * 1e-3) / 1e9
        out["decode"] = {"value": round(kv_bytes / (span_ms * 1e-3) / 1e9, 1), "unit": "GB/s",
                         "kv_bytes_per_step": kv_bytes, "ms_64_layers": round(span_ms, 4),
                         "note": "64 x gqa_decode_step (append of the new token + decode at T=8192, one launch each), replayed as one HIP graph"}
        src_dec = os.path.join(ROOT, "causal_gqa_attention_attn_amd", "csrc", "decode_bf16.hip")
        out["roofline_decode"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                                  "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                                  "traffic": _traffic("decode_bf16_kernel<128, false, false, *>", src_dec),
                                  "kernel": "one layer of the replayed decode graph: decode_bf16_kernel<128, false, false, false> "
                                            "(append, split-T attention and split combine), 32 MiB of K/V",
                                  "layer_us": round(per_layer_ms * 1e3, 2),
                                  "timing": "HIP events around the 64-layer graph replay / 64 (launch gaps included)"}
        dec_us = _profiled_us("decode_bf16_kernel<128, false, false, *>", src_dec)
        if dec_us:
            out["roofline_decode"]["profile_avg_us"] = dec_us
            out["roofline_decode"]["profile_frac"] = round(kv_bytes / LAYERS / (dec_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
            out["decode"]["kernel_sum_ms"] = round(dec_us * LAYERS / 1e3, 4)
            out["decode"]["kernel_sum_gbs"] = round(kv_bytes / (dec_us * LAYERS * 1e-6) / 1e9, 1)
        lib.gqa_workspace_status(dec.handle, ws)
    if not args.no_other_configs and not args.prefill_only:
        print("bench: other configurations", file=sys.stderr, flush=True)
        out["other_configs"] = other_configs(lib, W)
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds, W)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
