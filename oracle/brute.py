"""Pure-Python brute force for tiny inputs -- TEST INFRASTRUCTURE.

Independent second derivation of the oracle's steps with plain loops, exact
summation (math.fsum) and an exhaustive pairwise-dominance top-k, used only to
pin oracle/dsa.py on inputs of a few dozen tokens.
"""
from __future__ import annotations

import math


def score(q, w, key):
    """sum over heads of w_h * max(0, q_h . key), exactly summed."""
    terms = []
    for h in range(len(q)):
        d = math.fsum(q[h][i] * key[i] for i in range(len(key)))
        terms.append(w[h] * (d if d > 0 else 0.0))
    return math.fsum(terms)


def topk_dominance(scores, k):
    """s is selected iff fewer than k entries beat it, where s' beats s when
    score[s'] > score[s], or the scores are equal and s' < s."""
    n = len(scores)
    sel = []
    for s in range(n):
        beaten_by = 0
        for s2 in range(n):
            if scores[s2] > scores[s] or (scores[s2] == scores[s] and s2 < s):
                beaten_by += 1
        if beaten_by < k:
            sel.append(s)
    return sel


def attention(q, lat, sm_scale, dv):
    """Softmax attention of one head over explicit rows; returns (o, lse)."""
    logits = [sm_scale * math.fsum(q[d] * row[d] for d in range(len(q))) for row in lat]
    mx = max(logits)
    e = [math.exp(x - mx) for x in logits]
    z = math.fsum(e)
    o = [math.fsum(e[s] * lat[s][d] for s in range(len(lat))) / z for d in range(dv)]
    return o, mx + math.log(z)
