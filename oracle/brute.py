"""Pure-Python brute-force attention for tiny inputs (test oracle).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

An independent second implementation of the definition in "RingAttention and
Context Parallelism" (llms.blog), section 1: A = softmax(q k^T / sqrt(d_k) + M) v,
with the causal rule of its section 5 (token i sees tokens j <= i) and the
log-sum-exp statistic of its section 7.  It uses no NumPy arithmetic: plain
loops, ``math.fsum`` for every sum (correctly rounded) and ``math.exp`` /
``math.log``.  Inputs are nested lists or anything indexable; outputs are
nested lists of floats.
"""

from __future__ import annotations

import math


def attend_row(q_row, keys, vals, scale):
    """One query row against a list of visible (key, value) vectors.

    Returns (a_vector, m, l, lse); with no visible key: (zeros, -inf, 0, -inf).
    """
    dv = len(vals[0]) if vals else 0
    if not keys:
        return [0.0] * dv, -math.inf, 0.0, -math.inf
    z = [scale * math.fsum(q_row[d] * key[d] for d in range(len(q_row))) for key in keys]
    m = max(z)
    w = [math.exp(zj - m) for zj in z]
    l = math.fsum(w)
    a = [math.fsum(w[j] * vals[j][e] for j in range(len(keys))) / l for e in range(dv)]
    return a, m, l, m + math.log(l)


def attend(q, k, v, scale, q_pos=None, k_pos=None, causal=False):
    """q [T][Hq][D], k/v [L][Hkv][D] (nested sequences).

    Query head h reads KV head h // (Hq // Hkv).  Returns nested lists
    A [T][Hq][D], m [T][Hq], l [T][Hq], lse [T][Hq].
    """
    T = len(q)
    Hq = len(q[0])
    L = len(k)
    Hkv = len(k[0]) if L else 1
    group = Hq // Hkv
    if q_pos is None:
        q_pos = list(range(T))
    if k_pos is None:
        k_pos = list(range(L))
    A, M, Ls, LSE = [], [], [], []
    for t in range(T):
        a_t, m_t, l_t, s_t = [], [], [], []
        for h in range(Hq):
            g = h // group
            keys, vals = [], []
            for j in range(L):
                if causal and k_pos[j] > q_pos[t]:
                    continue
                keys.append([float(x) for x in k[j][g]])
                vals.append([float(x) for x in v[j][g]])
            if not vals:
                dv = len(v[0][g]) if L else len(q[t][h])
                a, m, l, s = [0.0] * dv, -math.inf, 0.0, -math.inf
            else:
                a, m, l, s = attend_row([float(x) for x in q[t][h]], keys, vals, scale)
            a_t.append(a)
            m_t.append(m)
            l_t.append(l)
            s_t.append(s)
        A.append(a_t)
        M.append(m_t)
        Ls.append(l_t)
        LSE.append(s_t)
    return A, M, Ls, LSE
