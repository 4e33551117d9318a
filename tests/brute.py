"""Independent pure-Python scalar differential attention for tiny inputs.

Written from the pages' definitions with Python floats and ``math.exp`` only
(no numpy, no torch): two score rows per query, a max-subtracted softmax over
the allowed keys of each, the signed combination with lambda, and the weighted
sum of value rows.  The French lesson page builds the same thing from lists
("Étape 1" and "Étape 3"); the paperleet page says its grader uses an
independent scalar softmax.  Used only to cross-check the float64 oracle.
"""

import math


def _row_softmax(scores):
    top = max(scores)
    ex = [math.exp(x - top) for x in scores]
    tot = sum(ex)
    return [x / tot for x in ex]


def _dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def diff_attention_head(q1, k1, q2, k2, v, lam, causal):
    """q*, k*: lists of T rows of D floats; v: T rows of 2D floats."""
    t = len(q1)
    d = len(q1[0])
    out = []
    for i in range(t):
        allowed = range(i + 1) if causal else range(len(k1))
        w1 = _row_softmax([_dot(q1[i], k1[j]) / math.sqrt(d) for j in allowed])
        w2 = _row_softmax([_dot(q2[i], k2[j]) / math.sqrt(d) for j in allowed])
        row = [0.0] * len(v[0])
        for n, j in enumerate(allowed):
            w = w1[n] - lam * w2[n]
            for c in range(len(row)):
                row[c] += w * v[j][c]
        out.append(row)
    return out
