"""Pure-Python brute force for tiny attention cases (test helper).

Written independently of `oracle/`: nested loops, `math.exp`, `math.fsum`,
its own head-group and token-offset arithmetic. Used only to pin the oracle.
"""
from __future__ import annotations

import math


def attend_brute(q, k, v, seq_lens, scale, h_kv):
    """q: nested lists [B][h_q][d]; k, v: [T][h_kv][d]; returns [B][h_q][d]."""
    B = len(q)
    h_q = len(q[0]) if B else 0
    d = len(q[0][0]) if B else 0
    out = []
    start = 0
    for b in range(B):
        S = int(seq_lens[b])
        rows = range(start, start + S)
        ob = []
        for h in range(h_q):
            g = (h * h_kv) // h_q          # contiguous groups of h_q / h_kv heads
            s = [scale * math.fsum(q[b][h][i] * k[t][g][i] for i in range(d)) for t in rows]
            if not s:
                ob.append([0.0] * d)
                continue
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            den = math.fsum(e)
            ob.append([math.fsum(e[j] * v[t][g][i] for j, t in enumerate(rows)) / den
                       for i in range(d)])
        out.append(ob)
        start += S
    return out


def attend_mp(q, k, v, seq_lens, scale, h_kv, dps=40):
    """Same as attend_brute in mpmath at `dps` decimal digits."""
    import mpmath as mp
    mp.mp.dps = dps
    B = len(q)
    h_q = len(q[0])
    d = len(q[0][0])
    out = []
    start = 0
    for b in range(B):
        S = int(seq_lens[b])
        ob = []
        for h in range(h_q):
            g = (h * h_kv) // h_q
            s = [mp.mpf(scale) * mp.fsum(mp.mpf(q[b][h][i]) * mp.mpf(k[t][g][i]) for i in range(d))
                 for t in range(start, start + S)]
            e = [mp.e ** x for x in s]
            den = mp.fsum(e)
            ob.append([float(mp.fsum(e[j] * mp.mpf(v[start + j][g][i]) for j in range(S)) / den)
                       for i in range(d)])
        out.append(ob)
        start += S
    return out
