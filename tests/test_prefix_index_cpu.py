"""Host prefix index (radix tree over token ids) against the brute-force oracle.

The oracle (oracle/prefix_match.py) compares a query with every recorded
request and keeps the longest common token-id prefix, smallest request id on
ties.  Its own pins are the prefix-sharing lesson's cases worked by hand.  The
library's radix tree must give the same answer after any sequence of inserts,
replacements and removals.  No GPU is used.
"""
import numpy as np

from oracle.prefix_match import PrefixTable, common_prefix


def test_oracle_pins_from_the_lesson():
    # two requests that start with the same system prompt and diverge at the
    # user's input share exactly the prompt
    prompt = [101, 7, 7, 42, 9]
    t = PrefixTable()
    t.insert(0, prompt + [5, 6])
    assert t.match(prompt + [8, 6, 5]) == (0, 5)
    # a_m != b_m: positions 0..m-1 are shared, nothing after
    assert common_prefix([1, 2, 3, 4], [1, 2, 9, 4]) == 2
    # reuse needs the exact ids: a request that differs at its first token shares nothing
    assert t.match([102] + prompt[1:]) == (-1, 0)
    # a query shorter than the cached request reuses all of itself
    assert t.match(prompt[:3]) == (0, 3)
    # ties go to the smallest id; a longer match wins over a smaller id
    t.insert(3, prompt + [5])
    t.insert(1, prompt)
    assert t.match(prompt + [5, 6, 7]) == (0, 7)
    assert t.match(prompt + [5]) == (0, 6)
    t.remove(0)
    assert t.match(prompt + [5, 6]) == (3, 6)
    assert t.match(prompt) == (1, 5)


def test_radix_index_matches_brute_force():
    import causal_gqa_attention_attn_amd as lib
    rng = np.random.default_rng(2024)
    ix = lib.PrefixIndex()
    ref = PrefixTable()
    stems = [list(rng.integers(0, 4, size=int(rng.integers(0, 12)))) for _ in range(6)]

    def draw():
        # a few shared stems with random continuations, over a 4-token alphabet
        s = stems[int(rng.integers(0, len(stems)))]
        tail = list(rng.integers(0, 4, size=int(rng.integers(0, 10))))
        return [int(x) for x in s[:int(rng.integers(0, len(s) + 1))] + tail]

    for step in range(3000):
        op = rng.random()
        if op < 0.35:
            seq, toks = int(rng.integers(0, 24)), draw()
            ix.insert(seq, toks)
            ref.insert(seq, toks)
        elif op < 0.5:
            seq = int(rng.integers(0, 24))
            ix.remove(seq)
            ref.remove(seq)
        else:
            q = draw()
            assert ix.match(q) == ref.match(q), (step, q)
    # empty query, empty recorded request
    ix.insert(30, [])
    ref.insert(30, [])
    assert ix.match([]) == ref.match([]) == (-1, 0)
    ix.close()
