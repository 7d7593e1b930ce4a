"""Drive the HIP library and the oracle side by side on the same inputs.

Inputs come from ``workloads`` (seeded); the library runs through the C ABI
(``causal_gqa_attention_attn_amd``), the oracle through ``oracle.cache_model``.
Comparisons: cache contents and block tables bit for bit; outputs to 1e-5
absolute (float32) or 2e-2 of the row's largest magnitude (bfloat16, float32
accumulation), per query row.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch
from threadpoolctl import threadpool_limits

from oracle.cache_model import CacheModel

F32_ATOL = 1e-5
BF16_ROW_RTOL = 2e-2


def k_view(cache):
    """K pool as [layer, page, kv head, slot, d] (the layout include/gqa.h documents)."""
    return cache.k_pool.view(cache.L, cache.num_pages, cache.Hkv, cache.P, cache.d)


def v_view(cache):
    """V pool as [layer, page, kv head, d, slot] (values stored d-major inside a page)."""
    return cache.v_pool.view(cache.L, cache.num_pages, cache.Hkv, cache.d, cache.P)


def device_table(cache, seq_id, count):
    """The first ``count`` entries of a sequence's row of the device block table."""
    return cache.page_table.view(-1, cache.max_pages_per_seq)[seq_id, :count].cpu().tolist()


def gather(cache, seq_id, layer):
    """Logical (K_used, V) of one sequence and layer, [Hkv, len, d] on the host,
    read through the library's block table: slot t is page table[t // 16],
    offset t % 16 (plain torch indexing)."""
    lib = cache_lib()
    n = lib.gqa_cache_length(cache.handle, seq_id, layer)
    pages = lib.gqa_cache_page_table(cache.handle, seq_id)
    if n == 0:
        z = torch.zeros(cache.Hkv, 0, cache.d, dtype=cache.dtype)
        return z, z.clone()
    idx = torch.tensor(pages, dtype=torch.long, device=cache.k_pool.device)
    k = k_view(cache)[layer].index_select(0, idx)            # [np, Hkv, P, d]
    v = v_view(cache)[layer].index_select(0, idx)            # [np, Hkv, d, P]
    k = k.permute(1, 0, 2, 3).reshape(cache.Hkv, -1, cache.d)[:, :n]
    v = v.permute(1, 0, 3, 2).reshape(cache.Hkv, -1, cache.d)[:, :n]
    return k.cpu(), v.cpu()


def gather_resident(cache, seq_id, layer):
    """(first, K_used, V) of the positions [first, len) a ring still holds
    (first = 0 without a window): logical page L is read from table entry
    L mod max_pages_per_seq."""
    lib = cache_lib()
    n = lib.gqa_cache_length(cache.handle, seq_id, layer)
    if not cache.window:
        return (0,) + gather(cache, seq_id, layer)
    if n == 0:
        z = torch.zeros(cache.Hkv, 0, cache.d, dtype=cache.dtype)
        return 0, z, z.clone()
    R = cache.max_pages_per_seq
    pages = lib.gqa_cache_page_table(cache.handle, seq_id)
    last = (n - 1) // cache.P
    first_page = max(0, last - R + 1)
    idx = torch.tensor([pages[L % R] for L in range(first_page, last + 1)], dtype=torch.long,
                       device=cache.k_pool.device)
    k = k_view(cache)[layer].index_select(0, idx)
    v = v_view(cache)[layer].index_select(0, idx)
    first = first_page * cache.P
    k = k.permute(1, 0, 2, 3).reshape(cache.Hkv, -1, cache.d)[:, :n - first]
    v = v.permute(1, 0, 3, 2).reshape(cache.Hkv, -1, cache.d)[:, :n - first]
    return first, k.cpu(), v.cpu()


def cache_lib():
    import causal_gqa_attention_attn_amd as lib
    return lib


def as_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float32).numpy()


def dtype_tag(dt):
    return "bf16" if dt == torch.bfloat16 else "f32"


class Pair:
    """One library cache and one oracle cache with the same configuration."""

    def __init__(self, num_layers, Hkv, d, num_pages, max_seqs, max_pages_per_seq, dtype,
                 theta, max_position=None, free_order=None, window=0):
        import causal_gqa_attention_attn_amd as lib
        self.lib = lib
        self.dtype = dtype
        mp = max_position if max_position else max_pages_per_seq * 16
        self.gpu = lib.PagedCache(num_layers, Hkv, d, num_pages, max_seqs, max_pages_per_seq,
                                  dtype=dtype, rope_theta=theta, max_position=mp,
                                  free_list_order=free_order, window=window)
        self.ref = CacheModel(num_layers, Hkv, d, 16, num_pages, max_seqs, max_pages_per_seq,
                              dtype=dtype_tag(dtype), rope_theta=theta, max_position=mp,
                              free_order=free_order, window=window)
        self.ws = None

    def workspace(self, B, Hq):
        n = self.lib.gqa_workspace_size(self.gpu.handle, B, Hq)
        if self.ws is None or self.ws.numel() < n:
            self.ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
        return self.ws

    # ------------------------------------------------------------ calls
    def chunk_workspace(self, B, Hq, n):
        """Workspace for split-T prefill/attention calls (chunks of at most n rows)."""
        nb = max(self.lib.gqa_attention_workspace_size(self.gpu.handle, B, Hq, n),
                 self.lib.gqa_workspace_size(self.gpu.handle, B, Hq))
        if self.ws is None or self.ws.numel() < nb:
            self.ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
        return self.ws

    def prefill(self, layer, seq_ids, Q, K, V, mask, pos, oracle=True, workspace=None):
        dev = [t.to("cuda") for t in (Q, K, V)]
        O = torch.full_like(dev[0], float("nan"))
        self.lib.gqa_prefill(self.gpu.handle, layer, seq_ids, dev[0], dev[1], dev[2], mask, pos, O, workspace)
        torch.cuda.synchronize()
        ref = None
        if oracle:
            ref = self.ref.prefill(layer, seq_ids, as_f32(Q), as_f32(K), as_f32(V),
                                   mask.numpy(), pos.numpy())
        else:
            self.ref.append(layer, seq_ids, as_f32(K), as_f32(V), mask.numpy(), pos.numpy())
        return O, ref

    def append(self, layer, seq_ids, K, V, mask, pos):
        self.lib.kv_cache_append(self.gpu.handle, layer, seq_ids, K.to("cuda"), V.to("cuda"), mask, pos)
        self.ref.append(layer, seq_ids, as_f32(K), as_f32(V), mask.numpy(), pos.numpy())

    def decode(self, layer, seq_ids, q, lengths, oracle=True):
        qd = q.to("cuda")
        o = torch.full_like(qd, float("nan"))
        self.lib.gqa_decode(self.gpu.handle, layer, seq_ids, qd, lengths, o,
                            self.workspace(len(seq_ids), q.shape[1]))
        torch.cuda.synchronize()
        ref = self.ref.decode(layer, seq_ids, as_f32(q), lengths) if oracle else None
        return o, ref

    def step(self, layer, seq_ids, st):
        """One decode step: append the new token's k, v, then attend with q."""
        B = len(seq_ids)
        lens = [self.ref.cache_length(s, layer) for s in seq_ids]
        mask = torch.ones((B, 1), dtype=torch.uint8)
        pos = torch.tensor([[n] for n in lens], dtype=torch.int32)
        self.append(layer, seq_ids, st.k, st.v, mask, pos)
        return self.decode(layer, seq_ids, st.q, [n + 1 for n in lens])

    def step_fused(self, layer, seq_ids, st):
        """One decode step through gqa_decode_step (append + decode in one call)."""
        lens = [self.ref.cache_length(s, layer) for s in seq_ids]
        qd = st.q.to("cuda")
        o = torch.full_like(qd, float("nan"))
        self.lib.gqa_decode_step(self.gpu.handle, layer, seq_ids, qd, st.k.to("cuda"), st.v.to("cuda"), o,
                                 self.workspace(len(seq_ids), st.q.shape[1]))
        torch.cuda.synchronize()
        B = len(seq_ids)
        self.ref.append(layer, seq_ids, as_f32(st.k), as_f32(st.v), np.ones((B, 1), np.uint8),
                        np.array([[n] for n in lens]))
        ref = self.ref.decode(layer, seq_ids, as_f32(st.q), [n + 1 for n in lens])
        return o, ref

    def truncate(self, seq, m):
        self.lib.kv_cache_truncate(self.gpu.handle, seq, m)
        self.ref.truncate(seq, m)

    def fork(self, src, dst, m):
        self.lib.kv_cache_fork(self.gpu.handle, src, dst, m)
        self.ref.fork(src, dst, m)

    # ------------------------------------------------------------ checks
    def check_cache(self, seqs, layers=None, invariants=True, device_tables=True):
        """Block tables, lengths and K/V bytes of the given sequences against the
        oracle; with ``invariants`` also both sides' cache invariants (every
        layer of a sequence at the same length) and the free-page count.  Host-only
        calls (fork, truncate) leave the device block table to the next launch,
        so right after them ``device_tables=False``."""
        torch.cuda.synchronize()
        if invariants:
            self.lib.gqa_cache_check(self.gpu.handle)
            assert self.ref.check() == []
        assert self.lib.gqa_cache_free_pages(self.gpu.handle) == len(self.ref.free), "free page count"
        for s in seqs:
            host_table = self.lib.gqa_cache_page_table(self.gpu.handle, s)
            assert host_table == self.ref.page_table(s), f"block table of sequence {s}"
            if device_tables:
                assert device_table(self.gpu, s, len(host_table)) == host_table, f"device table of sequence {s}"
            for l in (layers if layers is not None else range(self.ref.L)):
                assert self.lib.gqa_cache_length(self.gpu.handle, s, l) == self.ref.cache_length(s, l)
                first, k, v = gather_resident(self.gpu, s, l)
                assert first == self.ref.resident_from(s, l)
                rk, rv = self.ref.keys(s, l)[:, first:], self.ref.values(s, l)[:, first:]
                assert k.shape == rk.shape, (k.shape, rk.shape)
                kk = k.to(torch.float32).numpy()
                vv = v.to(torch.float32).numpy()
                assert np.array_equal(kk.view(np.uint32), rk.view(np.uint32)), f"K cache seq {s} layer {l}"
                assert np.array_equal(vv.view(np.uint32), rv.view(np.uint32)), f"V cache seq {s} layer {l}"


def oracle_workers():
    """Host threads for oracle work: the machine's cores, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


def oracle_rows(model, layer, jobs, chunk=128, workers=None):
    """Oracle attention for many query rows of already written sequences.

    jobs: list of (seq, q_rows [Hq, r, d] un-rotated float32, positions [r]).
    Each job's rows are cut into blocks of ``chunk`` rows and every block is
    one call of ``model.prefill_rows`` (rows are independent); the blocks run on
    a thread pool with one BLAS thread each.  Returns one [Hq, r, d] float64
    array per job, in order."""
    tasks = []
    for j, (seq, q, pos) in enumerate(jobs):
        pos = np.asarray(pos, dtype=np.int64)
        for r0 in range(0, len(pos), chunk):
            tasks.append((j, r0, seq, q[:, r0:r0 + chunk], pos[r0:r0 + chunk]))
    outs = [np.zeros(np.asarray(q).shape, dtype=np.float64) for (_, q, _) in jobs]

    def run(t):
        j, r0, seq, q, pos = t
        outs[j][:, r0:r0 + len(pos)] = model.prefill_rows(layer, seq, q, pos)

    with threadpool_limits(1), ThreadPoolExecutor(max_workers=workers or oracle_workers()) as ex:
        # heaviest blocks (latest positions) first
        list(ex.map(run, sorted(tasks, key=lambda t: -int(t[4][-1]) if len(t[4]) else 0)))
    return outs


def compare_rows(o_gpu: torch.Tensor, o_ref: np.ndarray, dtype, rows_mask=None):
    """Per query row: float32 |o-ref| <= 1e-5; bf16 max|o-ref| <= 2e-2 * max|ref|.

    Returns (max_abs_error, max_row_relative_error)."""
    o = as_f32(o_gpu).astype(np.float64)
    ref = np.asarray(o_ref, dtype=np.float64)
    assert o.shape == ref.shape
    if rows_mask is not None:
        o = o[rows_mask]
        ref = ref[rows_mask]
    assert not np.isnan(o).any(), "NaN in a compared output row"
    err = np.abs(o - ref)
    scale = np.max(np.abs(ref), axis=-1, keepdims=True)
    rel = np.max(err, axis=-1) / np.maximum(np.squeeze(scale, -1), 1e-30)
    if dtype == torch.float32:
        assert err.max(initial=0) <= F32_ATOL, f"max abs error {err.max()}"
    else:
        assert rel.max(initial=0) <= BF16_ROW_RTOL, f"max row-relative error {rel.max()}"
    return float(err.max(initial=0)), float(rel.max(initial=0))
