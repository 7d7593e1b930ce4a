"""State model of the per-layer paged KV cache and of the three attention calls.

Test infrastructure.  Sources:

* page "Prefill：整层状态演化与 KV 建立":
  - section 2.1: preconditions are checked before any layer runs, and a
    violation fails the call rather than producing an undefined answer;
  - section 2.2: the validity mask G must agree with the valid positions;
  - section 2.5: LayerCache holds the keys actually used by attention (after the
    position transform), the values, positions and valid lengths; the logical
    read order is positions 0..n_b-1 whatever the physical layout;
  - section 2.5, cache invariants: equal length in every layer, shapes match
    the configuration, padding never becomes visible history;
  - section 2.6: prefill writes only the valid tokens' k_used and v at their
    logical positions, then runs causal attention;
  - section 2.11: positions that restart at 0 after reuse are a failure.
* page "KV Cache 与 Prefill/Decode 推理路径":
  - PagedAttention lesson: logical token t lives in logical block floor(t/P)
    at offset t mod P; each request keeps its own block table; when the last
    block is full any free physical block is taken from the global pool;
    paging changes addresses, never results; the tail wastes at most P-1 slots;
  - prompt-edit lesson: after an edit at position m keep every layer's KV for
    [0, m), drop the rest, and run an incremental prefill on the suffix;
  - decode lessons: a single new token appends one K/V per layer and reads all
    T cached entries, with no future entry to mask;
  - sliding-window lesson: with a window of W positions (the current one
    included) a query at position t reads positions t-W+1..t; keys that no
    query will read again need not be kept, and a ring of fixed capacity holds
    the latest window;
  - prefix-sharing lesson: requests whose first m token ids agree have equal
    per-layer K/V on positions 0..m-1 and may reference the same cache blocks;
    the system counts the references, and a shared block returns to the free
    pool only once no request references it; a fork inside a block is a
    matter of page granularity and copy-on-write.
* page "模型执行：从 token 到 Prefill 与 Decode": the decode step appends, then
  attends over T = (cached) + 1 entries.

Readings fixed here (the pages leave them open):

* position ids of the valid tokens must be c_b, c_b+1, ..., c_b+n_b-1 where c_b
  is the current cache length (slot = position); anything else is rejected;
* the valid tokens of a row may sit anywhere in it (padding before, after or
  between them); in row order they take consecutive positions and slots;
* pages are shared by all layers of a sequence: the first layer that needs a
  logical page takes it; pages are taken from the front of the free list in
  batch order, then logical-page order; pages freed by truncation go to the
  back in ascending logical order, remapped source pages in the order given;
* invalid (padding) query rows produce exact zeros;
* window W > 0 makes the cache a ring: a sequence's block table has at most
  R = max_pages_per_seq entries and logical page L lives in entry L mod R, so
  once the ring is full each new logical page reuses, in place, the page of
  the logical page R before it.  A call that writes positions [c, c+n) must
  find every position its queries read, [max(0, c-W+1), c+n), in at most R
  consecutive logical pages (else OUT_OF_PAGES); R must be at least
  ceil(W/P) + 1 so that a decode step fits.  Truncation of a ring sequence
  is supported only to 0 (release) or to at least its length (no change), and
  a ring sequence cannot be forked (UNSUPPORTED): positions the ring has
  overwritten cannot come back;
* a fork (sequence dst takes sequence src's positions [0, m)) makes dst's
  first ceil(m/P) table entries the same physical pages as src's, each page
  counting one more reference; nothing is copied then.  A write into a page
  with more than one reference (only possible into the page that holds slot
  c_b when c_b is not a multiple of P) first copies that page, every layer,
  to a page taken from the front of the free list and points the writer's
  entry at the copy: in batch order, a row's copy is taken before its new
  pages.  A page reaches the free list when its last reference goes.
"""
from collections import deque

import numpy as np

from . import attention
from .bf16 import round_to_storage
from .rope import rotate


class OracleError(Exception):
    """A rejected call; ``code`` is one of ARG SHAPE DTYPE MASK POSITION CACHE
    OUT_OF_PAGES UNSUPPORTED."""

    def __init__(self, code: str, msg: str = ""):
        super().__init__(f"{code}: {msg}")
        self.code = code


def _ceil_div(a, b):
    return -(-a // b)


def valid_rows(mask_row) -> tuple:
    """(rows, count): the rectangular rows whose entry is 1, in order; MASK error
    for an entry other than 0 or 1 (section 2.2: G takes values in {0, 1})."""
    row = np.asarray(mask_row)
    if not np.isin(row, (0, 1)).all():
        raise OracleError("MASK", "mask entries must be 0 or 1")
    idx = np.nonzero(row)[0]
    return idx, int(idx.size)


class CacheModel:
    def __init__(self, num_layers, num_kv_heads, head_dim, page_size, num_pages,
                 max_seqs, max_pages_per_seq, dtype="bf16", rope_theta=0.0,
                 max_position=None, free_order=None, window=0):
        self.L = num_layers
        self.Hkv = num_kv_heads
        self.d = head_dim
        self.P = page_size
        self.num_pages = num_pages
        self.max_seqs = max_seqs
        self.max_pages_per_seq = max_pages_per_seq
        self.dtype = dtype
        self.theta = rope_theta
        self.window = int(window)
        if self.window < 0 or (self.window and max_pages_per_seq < _ceil_div(self.window, page_size) + 1):
            raise OracleError("UNSUPPORTED", "a ring must hold a window plus one page")
        self.max_position = max_position if max_position is not None else max_pages_per_seq * page_size
        order = list(range(num_pages)) if free_order is None else [int(p) for p in free_order]
        if sorted(order) != list(range(num_pages)):
            raise OracleError("ARG", "free-list order must be a permutation of the pool")
        self.free = deque(order)
        self.ref = [0] * num_pages          # table entries that reference each page
        self.copies = []                    # (src, dst) page copies made by copy-on-write, in order
        self.pages = {s: [] for s in range(max_seqs)}
        self.length = {(s, l): 0 for s in range(max_seqs) for l in range(num_layers)}
        empty = np.zeros((num_kv_heads, 0, head_dim), dtype=np.float32)
        self.K = {(s, l): empty for s in range(max_seqs) for l in range(num_layers)}
        self.V = {(s, l): empty for s in range(max_seqs) for l in range(num_layers)}

    # ------------------------------------------------------------ queries
    def cache_length(self, seq, layer):
        return self.length[(seq, layer)]

    def page_table(self, seq):
        return list(self.pages[seq])

    def keys(self, seq, layer):
        return self.K[(seq, layer)]

    def values(self, seq, layer):
        return self.V[(seq, layer)]

    def logical_elements(self) -> int:
        """Cached scalars, K and V together: sum of 2 * Hkv * len * d."""
        return sum(2 * self.Hkv * n * self.d for n in self.length.values())

    def check(self) -> list:
        """Violations of the cache invariants (empty when consistent)."""
        bad = []
        refs = [0] * self.num_pages
        for s in range(self.max_seqs):
            lens = [self.length[(s, l)] for l in range(self.L)]
            if len(set(lens)) > 1:
                bad.append(f"sequence {s}: layer lengths differ {lens}")
            if len(self.pages[s]) != self._table_entries(max(lens)):
                bad.append(f"sequence {s}: {len(self.pages[s])} pages for length {max(lens)}")
            if len(set(self.pages[s])) != len(self.pages[s]):
                bad.append(f"sequence {s}: a page appears twice in its table")
            for p in self.pages[s]:
                refs[p] += 1
        if refs != self.ref:
            bad.append("reference counts differ from the tables")
        free = list(self.free)
        if len(set(free)) != len(free) or any(refs[p] for p in free):
            bad.append("a free page is listed twice or still referenced")
        if sorted(free + [p for p in range(self.num_pages) if refs[p]]) != list(range(self.num_pages)):
            bad.append("pages are lost")
        return bad

    # ------------------------------------------------------------ checks
    def _check_layer(self, layer):
        if not (0 <= layer < self.L):
            raise OracleError("ARG", "layer out of range")

    def _check_seqs(self, seq_ids):
        ids = [int(s) for s in seq_ids]
        if any(not (0 <= s < self.max_seqs) for s in ids):
            raise OracleError("ARG", "sequence id out of range")
        if len(set(ids)) != len(ids):
            raise OracleError("ARG", "a sequence appears twice in one call")
        return ids

    def _plan_append(self, layer, ids, K, V, mask, positions, dtype):
        """Every check of an append; returns per-row (start, count) and page needs."""
        B = len(ids)
        K = np.asarray(K)
        V = np.asarray(V)
        if dtype != self.dtype:
            raise OracleError("DTYPE", "input dtype differs from the cache dtype")
        if K.ndim != 4 or K.shape[0] != B or K.shape[1] != self.Hkv or K.shape[3] != self.d:
            raise OracleError("SHAPE", "K must be [B, Hkv, n, d]")
        if V.shape != K.shape:
            raise OracleError("SHAPE", "V must match K")
        n = K.shape[2]
        mask = np.asarray(mask)
        positions = np.asarray(positions)
        if mask.shape != (B, n) or positions.shape != (B, n):
            raise OracleError("SHAPE", "mask and positions must be [B, n]")
        runs = [valid_rows(mask[b]) for b in range(B)]
        for b, (s, nb) in enumerate(runs):
            c = self.length[(ids[b], layer)]
            want = np.arange(c, c + nb)
            if not np.array_equal(positions[b][s].astype(np.int64), want):
                raise OracleError("POSITION", "positions must continue the cache: c_b, c_b+1, ...")
            if c + nb > self.max_position:
                raise OracleError("POSITION", "position beyond the configured range")
            if self.window:
                first = max(0, c - self.window + 1)
                if nb and (c + nb - 1) // self.P - first // self.P + 1 > self.max_pages_per_seq:
                    raise OracleError("OUT_OF_PAGES", "the window and the new tokens exceed the ring")
            elif _ceil_div(c + nb, self.P) > self.max_pages_per_seq:
                raise OracleError("OUT_OF_PAGES", "sequence exceeds its block-table capacity")
        need = []
        ref = list(self.ref)        # references as the rows before this one leave them
        for b, (s, nb) in enumerate(runs):
            c = self.length[(ids[b], layer)]
            # writing from slot c touches an existing page only when c is inside
            # one; that page is copied first if another table references it
            cow = (not self.window and nb > 0 and c % self.P != 0
                   and self._copy_on_write(ref, self.pages[ids[b]][c // self.P]))
            if cow:
                ref[self.pages[ids[b]][c // self.P]] -= 1
            need.append((cow, max(0, self._table_entries(c + nb) - len(self.pages[ids[b]]))))
        if sum(int(cow) + k for cow, k in need) > len(self.free):
            raise OracleError("OUT_OF_PAGES", "not enough free pages")
        return runs, need

    def _table_entries(self, length) -> int:
        """Block-table entries a sequence of this length holds: one per logical
        page, at most R in a ring (page L reuses entry L mod R)."""
        entries = _ceil_div(length, self.P)
        return min(entries, self.max_pages_per_seq) if self.window else entries

    def resident_from(self, seq, layer) -> int:
        """First position a ring still holds (0 without a window)."""
        n = self.length[(seq, layer)]
        if not self.window or n == 0:
            return 0
        return max(0, ((n - 1) // self.P - self.max_pages_per_seq + 1) * self.P)

    @staticmethod
    def _copy_on_write(ref, page) -> bool:
        """A page must be copied before a write when another table references it."""
        return ref[page] > 1

    def _commit_append(self, layer, ids, K, V, runs, need):
        for b, (cow, k) in enumerate(need):
            table = self.pages[ids[b]]
            if cow:
                lp = self.length[(ids[b], layer)] // self.P
                new = self.free.popleft()
                self.copies.append((table[lp], new))
                self.ref[table[lp]] -= 1
                self.ref[new] = 1
                table[lp] = new
            for _ in range(k):
                page = self.free.popleft()
                self.ref[page] = 1
                table.append(page)
        for b, (s, nb) in enumerate(runs):
            if nb == 0:
                continue
            key = (ids[b], layer)
            c = self.length[key]
            pos = np.arange(c, c + nb)
            k_used = round_to_storage(rotate(np.asarray(K[b][:, s, :], np.float32), pos, self.theta),
                                      self.dtype)
            v = np.asarray(V[b][:, s, :], dtype=np.float32).copy()
            self.K[key] = np.concatenate([self.K[key], k_used], axis=1)
            self.V[key] = np.concatenate([self.V[key], v], axis=1)
            self.length[key] = c + nb

    # ------------------------------------------------------------ calls
    def append(self, layer, seq_ids, K, V, mask, positions, dtype=None):
        """Write the valid tokens' rotated keys and values at their positions."""
        self._check_layer(layer)
        ids = self._check_seqs(seq_ids)
        runs, need = self._plan_append(layer, ids, K, V, mask, positions,
                                       self.dtype if dtype is None else dtype)
        self._commit_append(layer, ids, K, V, runs, need)

    def prefill(self, layer, seq_ids, Q, K, V, mask, positions, dtype=None):
        """Append, then attention for every valid query row; returns O float64."""
        self._check_layer(layer)
        ids = self._check_seqs(seq_ids)
        Q = np.asarray(Q)
        B = len(ids)
        if Q.ndim != 4 or Q.shape[0] != B or Q.shape[3] != self.d or Q.shape[2] != np.asarray(K).shape[2]:
            raise OracleError("SHAPE", "Q must be [B, Hq, n, d]")
        Hq = Q.shape[1]
        if Hq % self.Hkv:
            raise OracleError("SHAPE", "Hkv must divide Hq")
        runs, need = self._plan_append(layer, ids, K, V, mask, positions,
                                       self.dtype if dtype is None else dtype)
        starts = [self.length[(s, layer)] for s in ids]
        self._commit_append(layer, ids, K, V, runs, need)
        O = np.zeros(Q.shape, dtype=np.float64)
        for b, (s, nb) in enumerate(runs):
            if nb == 0:
                continue
            pos = np.arange(starts[b], starts[b] + nb)
            q_used = round_to_storage(rotate(np.asarray(Q[b][:, s, :], np.float32), pos, self.theta),
                                      self.dtype)
            key = (ids[b], layer)
            O[b][:, s, :] = attention.attend_positions(q_used, pos, self.K[key], self.V[key], window=self.window)
        return O

    def prefill_rows(self, layer, seq, q_rows, positions):
        """Attention for selected query rows of an already written sequence.

        q_rows: [Hq, r, d] un-rotated queries at the given absolute positions.
        Used to check sampled outputs of large runs without recomputing all rows.
        """
        pos = np.asarray(positions, dtype=np.int64)
        if self.window and pos.size and max(0, pos.min() - self.window + 1) < self.resident_from(seq, layer):
            raise OracleError("POSITION", "the window of a query reaches positions the ring no longer holds")
        q_used = round_to_storage(rotate(np.asarray(q_rows, np.float32), pos, self.theta), self.dtype)
        key = (seq, layer)
        return attention.attend_positions(q_used, pos, self.K[key], self.V[key], window=self.window)

    def decode(self, layer, seq_ids, q, valid_lengths):
        """One query per sequence at position T-1 over all T cached slots."""
        self._check_layer(layer)
        ids = self._check_seqs(seq_ids)
        q = np.asarray(q)
        B = len(ids)
        if q.ndim != 4 or q.shape[0] != B or q.shape[2] != 1 or q.shape[3] != self.d:
            raise OracleError("SHAPE", "q must be [B, Hq, 1, d]")
        if q.shape[1] % self.Hkv:
            raise OracleError("SHAPE", "Hkv must divide Hq")
        lens = [int(x) for x in valid_lengths]
        if len(lens) != B:
            raise OracleError("SHAPE", "one valid length per sequence")
        for b, s in enumerate(ids):
            if lens[b] != self.length[(s, layer)]:
                raise OracleError("CACHE", "valid length differs from the cache length")
            if lens[b] < 1:
                raise OracleError("CACHE", "decode needs at least one cached token")
        o = np.zeros(q.shape, dtype=np.float64)
        for b, s in enumerate(ids):
            T = lens[b]
            o[b] = self.prefill_rows(layer, s, q[b], [T - 1])
        return o

    def truncate(self, seq, m):
        """Keep positions [0, m) in every layer; free pages no layer still uses."""
        if not (0 <= seq < self.max_seqs):
            raise OracleError("ARG", "sequence id out of range")
        if m < 0:
            raise OracleError("ARG", "negative truncation point")
        if self.window and 0 < m < max(self.length[(seq, l)] for l in range(self.L)):
            raise OracleError("UNSUPPORTED", "a ring sequence can only be released or left as it is")
        for l in range(self.L):
            key = (seq, l)
            n = min(self.length[key], m)
            self.length[key] = n
            self.K[key] = self.K[key][:, :n]
            self.V[key] = self.V[key][:, :n]
        keep = _ceil_div(max(self.length[(seq, l)] for l in range(self.L)), self.P)
        dropped = self.pages[seq][keep:]
        self.pages[seq] = self.pages[seq][:keep]
        for p in dropped:
            self.ref[p] -= 1
            if self.ref[p] == 0:
                self.free.append(p)

    def fork(self, src, dst, m):
        """Sequence dst (empty) takes src's positions [0, m) in every layer by
        referencing src's first ceil(m/P) pages; no page is copied."""
        if not (0 <= src < self.max_seqs and 0 <= dst < self.max_seqs) or src == dst:
            raise OracleError("ARG", "bad sequence ids")
        if m < 0:
            raise OracleError("ARG", "negative fork length")
        if self.window:
            raise OracleError("UNSUPPORTED", "ring sequences are not forked")
        if self.pages[dst] or any(self.length[(dst, l)] for l in range(self.L)):
            raise OracleError("CACHE", "the destination sequence is not empty")
        if m > min(self.length[(src, l)] for l in range(self.L)):
            raise OracleError("POSITION", "fork length beyond the source's length")
        self.pages[dst] = list(self.pages[src][:_ceil_div(m, self.P)])
        for p in self.pages[dst]:
            self.ref[p] += 1
        for l in range(self.L):
            key_s, key_d = (src, l), (dst, l)
            self.K[key_d] = self.K[key_s][:, :m].copy()
            self.V[key_d] = self.V[key_s][:, :m].copy()
            self.length[key_d] = m

    def remap(self, src, dst):
        """Move owned pages src[i] to free pages dst[i]; logical content is unchanged."""
        src = [int(x) for x in src]
        dst = [int(x) for x in dst]
        if len(src) != len(dst):
            raise OracleError("ARG", "src and dst differ in length")
        if len(set(src)) != len(src) or len(set(dst)) != len(dst):
            raise OracleError("ARG", "repeated page")
        free = set(self.free)
        for a, b in zip(src, dst):
            if not (0 <= a < self.num_pages and 0 <= b < self.num_pages):
                raise OracleError("ARG", "page id out of range")
            if self.ref[a] == 0:
                raise OracleError("CACHE", "source page is not in use")
            if b not in free:
                raise OracleError("CACHE", "destination page is not free")
        moved = dict(zip(src, dst))
        for pl in self.pages.values():
            for i, p in enumerate(pl):
                if p in moved:
                    pl[i] = moved[p]
        for a, b in zip(src, dst):
            self.ref[b] = self.ref[a]
            self.ref[a] = 0
            self.free.remove(b)
        self.free.extend(src)
