"""Longest reusable prefix among recorded requests, by brute force.

Test infrastructure.  Source: page "KV Cache 与 Prefill/Decode 推理路径",
prefix-sharing lesson: a cached prefix may be reused only when the token-id
sequences agree exactly (not by meaning); two requests that first differ at
index m share positions 0..m-1, so the shareable length is the longest common
prefix of the token ids; a prefix tree over the requests answers which prefix
is reusable, the block table where it lives.

Reading fixed here: among the recorded requests with the longest common
prefix, the one with the smallest id is returned; a longest common prefix of
length 0 is no match (id -1).
"""


def common_prefix(a, b) -> int:
    """Number of leading token ids that a and b have in common."""
    m = 0
    for x, y in zip(a, b):
        if x != y:
            break
        m += 1
    return m


class PrefixTable:
    """Recorded requests: id -> token ids; every query compares against each."""

    def __init__(self):
        self.tokens = {}

    def insert(self, seq, tokens):
        self.tokens[int(seq)] = [int(t) for t in tokens]

    def remove(self, seq):
        self.tokens.pop(int(seq), None)

    def match(self, tokens):
        best_seq, best_m = -1, 0
        for seq in sorted(self.tokens):
            m = common_prefix(tokens, self.tokens[seq])
            if m > best_m:
                best_seq, best_m = seq, m
        return best_seq, best_m
