"""Pure-Python loops for the attention definition, test infrastructure.

A second, independent reading of page "Prefill：整层状态演化与 KV 建立",
sections 2.2-2.3, for tiny shapes: nested lists, ``math.exp`` and
``math.fsum`` (exactly rounded sums), no numpy.  Used to check the numpy
oracle, never the other way round.
"""
import math


def attend_brute(q_used, q_pos, k_used, v):
    """q_used[h][i][t], q_pos[i], k_used[g][j][t], v[g][j][t] -> O[h][i][t].

    Query i at position q_pos[i] reads cache slots j <= q_pos[i].
    """
    Hq = len(q_used)
    Hkv = len(k_used)
    assert Hq % Hkv == 0
    T = len(k_used[0])
    out = []
    for h in range(Hq):
        g = (h * Hkv) // Hq
        d = len(q_used[h][0]) if q_used[h] else 0
        rows = []
        for i, p in enumerate(q_pos):
            visible = [j for j in range(T) if j <= p]
            s = [math.fsum(q_used[h][i][t] * k_used[g][j][t] for t in range(d)) / math.sqrt(d)
                 for j in visible]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = math.fsum(e)
            rows.append([math.fsum(e[a] * v[g][j][t] for a, j in enumerate(visible)) / z
                         for t in range(d)])
        out.append(rows)
    return out
