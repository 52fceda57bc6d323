"""Oracle: pure-Python brute-force attention for tiny inputs -- test infrastructure.

The same definition as ``oracle.attention`` written as explicit loops over
Python floats with ``math.fsum`` (exactly rounded sums), so it shares no
NumPy/BLAS arithmetic with it.  Used only to pin ``oracle.attention`` on
tiny shapes.
"""
from __future__ import annotations

import math


def attention(q, k, v, scale, key_gaps=None, key_mask=None):
    """q ``[B][Nq][Hq][D]``, k/v ``[B][Nk][Hkv][D]`` nested lists (or arrays);
    ``key_mask`` ``[B][Nk]`` booleans (True = valid) or None.

    Returns ``(o, lse)`` as nested lists ``[B][Nq][Hq][D]`` and ``[B][Hq][Nq]``;
    a batch without a valid key gets o = 0, lse = -inf.
    """
    bsz, nq, hq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    nk, hkv = len(k[0]), len(k[0][0])
    rep = hq // hkv
    o = [[[[0.0] * d for _ in range(hq)] for _ in range(nq)] for _ in range(bsz)]
    lse = [[[0.0] * nq for _ in range(hq)] for _ in range(bsz)]
    for b in range(bsz):
        g0, g1 = (0, 0) if key_gaps is None else (int(key_gaps[b][0]), int(key_gaps[b][1]))
        keys = [j for j in range(nk) if not (g0 <= j < g1) and (key_mask is None or key_mask[b][j])]
        if not keys:
            for h in range(hq):
                lse[b][h] = [-math.inf] * nq
            continue
        for h in range(hq):
            hk = h // rep
            for i in range(nq):
                s = [scale * math.fsum(float(q[b][i][h][t]) * float(k[b][j][hk][t]) for t in range(d))
                     for j in keys]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                l = math.fsum(w)
                for t in range(d):
                    o[b][i][h][t] = math.fsum(w[n] * float(v[b][j][hk][t]) for n, j in enumerate(keys)) / l
                lse[b][h][i] = m + math.log(l)
    return o, lse
