"""Exact brute-force evaluation used to pin the oracle (tiny inputs only).

Every binary16/bfloat16 value is a dyadic rational, so Fraction(float(v)) is exact and
sums of products of Fractions are exact.  These loops follow the epilog definitions
element by element, sharing nothing with the vectorised oracle.
"""
import math
from fractions import Fraction


def exact_matmul(a, b, b_layout):
    """Exact A.B as a list of lists of Fractions; a, b nested sequences of floats."""
    m = len(a)
    k = len(a[0])
    if b_layout == "KN":
        n = len(b[0])
        bat = lambda kk, j: b[kk][j]
    else:
        n = len(b)
        bat = lambda kk, j: b[j][kk]
    out = []
    for i in range(m):
        row = []
        for j in range(n):
            s = Fraction(0)
            for kk in range(k):
                s += Fraction(float(a[i][kk])) * Fraction(float(bat(kk, j)))
            row.append(s)
        out.append(row)
    return out


def exact_relu_aux_bias(a, b, bias, b_layout):
    """(P, Y, words) with P exact, Y = P if P > 0 else 0, and mask words assembled bit by bit."""
    z = exact_matmul(a, b, b_layout)
    m, n = len(z), len(z[0])
    p = [[z[i][j] + Fraction(float(bias[j])) for j in range(n)] for i in range(m)]
    y = [[v if v > 0 else Fraction(0) for v in row] for row in p]
    nw = (n + 31) // 32
    words = []
    for i in range(m):
        row = [0] * nw
        for j in range(n):
            if p[i][j] > 0:
                row[j // 32] |= 1 << (j % 32)
        words.append(row)
    return p, y, words


def exact_drelu_bgrad(dy, w_nk, words):
    """(dX, bgrad) exactly: dX[i][j] = G[i][j] if bit j of row i is set, else 0."""
    g = exact_matmul(dy, w_nk, "NK")
    m, n = len(g), len(g[0])
    dx = [[g[i][j] if (words[i][j // 32] >> (j % 32)) & 1 else Fraction(0) for j in range(n)]
          for i in range(m)]
    bgrad = [sum((dx[i][j] for i in range(m)), Fraction(0)) for j in range(n)]
    return dx, bgrad


def scalar_sigmoid(t):
    t = float(t)
    if t >= 0:
        return 1.0 / (1.0 + math.exp(-t))
    e = math.exp(t)
    return e / (1.0 + e)
