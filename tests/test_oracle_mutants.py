"""Plant plausible mistakes in the oracle (on the CPU) and see a pin catch each.

Every mutant replaces one oracle function by a subtly wrong copy: a dropped
scale, a wrong comparison, a swapped head map, a future key inside the
denominator, a flipped rotation sign, adjacent-pair rotation, truncating
bf16 conversion.  The pins of ``test_oracle_pins`` must fail on each.
"""
import numpy as np
import pytest

from oracle import attention, bf16, cache_model, rope
from oracle.cache_model import CacheModel, _ceil_div
import test_oracle_pins as pins

ALL_PINS = [pins.check_worked_example, pins.check_single_key_and_uniform,
            pins.check_against_textbook_sdpa, pins.check_brute_force,
            pins.check_mask_counts, pins.check_bf16_rounding, pins.check_rotation,
            pins.check_cache_counts, pins.check_prefix_sharing, pins.check_padding_placement_invariance,
            pins.check_fork_then_suffix_equals_full_prefill, pins.check_sliding_window,
            pins.check_ring_cache]


def _some_pin_fails():
    for pin in ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, cache_model.OracleError):
            return True
    return False


def _attend_no_scale(q_used, k_used, v, M):
    q_used, k_used, v = (np.asarray(a, np.float64) for a in (q_used, k_used, v))
    Hq, Hkv = q_used.shape[0], k_used.shape[0]
    out = np.zeros(q_used.shape)
    for h in range(Hq):
        g = attention.head_map(h, Hq, Hkv)
        out[h] = attention.softmax_finite(q_used[h] @ k_used[g].T + M) @ v[g]
    return out


def _attend_future_in_denominator(q_used, k_used, v, M):
    q_used, k_used, v = (np.asarray(a, np.float64) for a in (q_used, k_used, v))
    Hq, Hkv = q_used.shape[0], k_used.shape[0]
    out = np.zeros(q_used.shape)
    d = q_used.shape[-1]
    for h in range(Hq):
        g = attention.head_map(h, Hq, Hkv)
        S = q_used[h] @ k_used[g].T / np.sqrt(d)
        A = attention.softmax_finite(S) * np.isfinite(M)   # mask applied after normalising
        out[h] = A @ v[g]
    return out


def _attend_key_transposed(q_used, k_used, v, M):
    q_used, k_used, v = (np.asarray(a, np.float64) for a in (q_used, k_used, v))
    Hq, Hkv = q_used.shape[0], k_used.shape[0]
    out = np.zeros(q_used.shape)
    d = q_used.shape[-1]
    for h in range(Hq):
        g = attention.head_map(h, Hq, Hkv)
        S = q_used[h] @ k_used[g].T / np.sqrt(d) + M
        out[h] = attention.softmax_finite(S) @ v[g][::-1]     # values read in reverse order
    return out


def _rotate_sign(x, positions, theta):
    x = np.asarray(x, np.float32)
    if theta == 0:
        return x.copy()
    d = x.shape[-1]
    c, s = rope.cos_sin(theta, d, positions)
    h = d // 2
    a, b = x[..., :h], x[..., h:]
    out = np.empty_like(x)
    out[..., :h] = a * c + b * s
    out[..., h:] = -a * s + b * c
    return out


def _rotate_adjacent(x, positions, theta):
    x = np.asarray(x, np.float32)
    if theta == 0:
        return x.copy()
    d = x.shape[-1]
    c, s = rope.cos_sin(theta, d, positions)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def _bf16_truncate(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).copy()


def _truncate_ignoring_references(self, seq, m):
    """Frees every dropped page, even one another sequence still references."""
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
        self.ref[p] = 0
        self.free.append(p)


def _valid_span(mask_row):
    """Treats everything from the first to the last valid token as valid (holes included)."""
    idx = np.nonzero(np.asarray(mask_row))[0]
    if idx.size == 0:
        return idx, 0
    rows = np.arange(idx[0], idx[-1] + 1)
    return rows, int(rows.size)


def _window_one_too_wide(q_pos, T, W):
    q_pos = np.asarray(q_pos, dtype=np.int64)
    j = np.arange(T, dtype=np.int64)[None, :]
    visible = (j <= q_pos[:, None]) & ((j >= q_pos[:, None] - W) if W > 0 else True)
    return np.where(visible, 0.0, float("-inf"))


_fork = CacheModel.fork


def _fork_whole_pages_only(self, src, dst, m):
    """References floor(m/P) pages: the partly filled block of a mid-block fork is lost."""
    _fork(self, src, dst, m)
    for p in self.pages[dst][m // self.P:]:
        self.ref[p] -= 1
    self.pages[dst] = self.pages[dst][:m // self.P]


MUTANTS = {
    "head_map_modulo": (attention, "head_map", lambda h, Hq, Hkv: h % Hkv),
    "mask_strict": (attention, "slot_mask",
                    lambda q_pos, T: np.where(np.arange(T)[None, :] < np.asarray(q_pos)[:, None],
                                              0.0, float("-inf"))),
    "mask_rect_strict": (attention, "rect_mask",
                         lambda G: np.where(np.tril(np.ones((np.shape(G)[1],) * 2), -1)[None] > 0,
                                            0.0, float("-inf")) * np.ones((np.shape(G)[0], 1, 1))),
    "no_scale": (attention, "attend", _attend_no_scale),
    "future_in_denominator": (attention, "attend", _attend_future_in_denominator),
    "values_reversed": (attention, "attend", _attend_key_transposed),
    "rotation_sign": (rope, "rotate", _rotate_sign),
    "rotation_adjacent_pairs": (rope, "rotate", _rotate_adjacent),
    "bf16_truncation": (bf16, "round_f32_to_bf16", _bf16_truncate),
    "no_copy_on_write": (CacheModel, "_copy_on_write", staticmethod(lambda ref, page: False)),
    "shared_page_freed_on_truncate": (CacheModel, "truncate", _truncate_ignoring_references),
    "fork_whole_pages_only": (CacheModel, "fork", _fork_whole_pages_only),
    "holes_treated_as_valid": (cache_model, "valid_rows", _valid_span),
    "window_one_too_wide": (attention, "window_mask", _window_one_too_wide),
    "ring_never_reuses": (CacheModel, "_table_entries", lambda self, length: _ceil_div(length, self.P)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    assert _some_pin_fails() is False
    module, attr, fn = MUTANTS[name]
    monkeypatch.setattr(module, attr, fn)
    if module is bf16:
        monkeypatch.setattr(pins, "round_f32_to_bf16", fn)
    assert _some_pin_fails(), f"no pin catches mutant {name}"
