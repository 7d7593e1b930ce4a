"""Float64 CPU oracle for masked causal grouped-query attention with a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this package; only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code with the GPU path.

It is a plain restatement of the definitions on the source pages:

* ``attention``   the mask M, the scaled scores S, the row-stable softmax A over
                  finite scores and the output O (page "Prefill：整层状态演化与
                  KV 建立", sections 2.2 and 2.3), with the grouped-query head
                  map g(h) = floor(h*Hkv/Hq); numpy float64.
* ``brute``       the same definition in pure-Python loops with ``math.fsum``
                  (tiny shapes only), as an independent second reading.
* ``rope``        the position rotation applied to q and k before the dot
                  product (page "KV Cache 与 Prefill/Decode 推理路径", prefix
                  equality proof, RoPE paragraph), in the float32 rounding rule
                  fixed for this library.
* ``bf16``        round-to-nearest-even float32 -> bfloat16.
* ``cache_model`` the cache contract of section 2.5 (per-layer keys as used by
                  attention, values, lengths, layout), the paged block table of
                  the PagedAttention lesson, truncation at an edit point and
                  page remap, plus the precondition checks of section 2.1.

Parity pinned by ``tests/test_oracle_*.py`` (worked 2-D example, closed forms,
textbook scaled-dot-product attention, brute force, work counts, paging counts,
independent bf16 conversion, complex-number form of the rotation).  The choice
of rotation pairing (half-split) is a convention the pages leave open: parity
unpinned for that choice alone.
"""
from . import bf16, rope, attention, brute, cache_model  # noqa: F401
