"""Pure-Python brute force for tiny inputs (N <= 64): no numpy, plain loops.

TEST INFRASTRUCTURE ONLY (see the oracle package header). These functions pin
the numpy oracle on tiny cases by recomputing each definition the long way:
masked softmax with explicit -inf entries, Lloyd's k-means with explicit
coordinate differences, and the ridge normal equations by Gauss-Jordan
elimination.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

Matrix = List[List[float]]


def _row_softmax_apply(logits: Sequence[float], v: Matrix) -> List[float]:
    m = max(logits)
    w = [math.exp(s - m) if s != -math.inf else 0.0 for s in logits]
    tot = sum(w)
    d = len(v[0])
    return [sum(w[j] * v[j][c] for j in range(len(v))) / tot for c in range(d)]


def attention(q: Matrix, k: Matrix, v: Matrix,
              allowed: Optional[List[List[bool]]] = None) -> Matrix:
    """softmax(Q K^T / sqrt(d) + mask) V, the mask being -inf where not allowed."""
    d = len(q[0])
    out = []
    for i, qi in enumerate(q):
        logits = []
        for j, kj in enumerate(k):
            if allowed is not None and not allowed[i][j]:
                logits.append(-math.inf)
            else:
                logits.append(sum(qi[c] * kj[c] for c in range(d)) / math.sqrt(d))
        out.append(_row_softmax_apply(logits, v))
    return out


def lloyd(points: Matrix, seeds: Sequence[int], iters: int) -> List[int]:
    """Lloyd's k-means from the given seed points; ties to the lowest index;
    empty groups keep their centroid; returns the last assignment."""
    cent = [list(points[s]) for s in seeds]
    labels = [0] * len(points)
    for _ in range(iters):
        for n, p in enumerate(points):
            best, best_d = 0, None
            for g, c in enumerate(cent):
                dist = sum((p[t] - c[t]) ** 2 for t in range(len(p)))
                if best_d is None or dist < best_d:
                    best, best_d = g, dist
            labels[n] = best
        for g in range(len(cent)):
            mem = [points[n] for n in range(len(points)) if labels[n] == g]
            if mem:
                cent[g] = [sum(m[t] for m in mem) / len(mem) for t in range(len(points[0]))]
    return labels


def solve(a: Matrix, b: Matrix) -> Matrix:
    """Gauss-Jordan with partial pivoting: A X = B."""
    n = len(a)
    m = [list(a[i]) + list(b[i]) for i in range(n)]
    w = len(m[0])
    for col in range(n):
        piv = max(range(col, n), key=lambda r: abs(m[r][col]))
        m[col], m[piv] = m[piv], m[col]
        pv = m[col][col]
        m[col] = [x / pv for x in m[col]]
        for r in range(n):
            if r != col and m[r][col] != 0.0:
                f = m[r][col]
                m[r] = [m[r][c] - f * m[col][c] for c in range(w)]
    return [row[n:] for row in m]


def ridge_affine(x: Matrix, y: Matrix, lam: float):
    """Minimise sum |y_p - b - x_p B|^2 + lam |B|_F^2 with b unpenalised, through
    the (d+1)-unknown normal equations of the augmented design [1, x]."""
    d = len(x[0])
    aug = [[1.0] + list(r) for r in x]
    a = [[sum(aug[p][i] * aug[p][j] for p in range(len(x))) for j in range(d + 1)]
         for i in range(d + 1)]
    for i in range(1, d + 1):
        a[i][i] += lam
    rhs = [[sum(aug[p][i] * y[p][c] for p in range(len(x))) for c in range(len(y[0]))]
           for i in range(d + 1)]
    sol = solve(a, rhs)
    return [sol[i] for i in range(1, d + 1)], sol[0]


def e4m3_values() -> List[float]:
    """Every finite non-negative FP8 E4M3 value, decoded code by code from the format's
    definition: code = E M (4 exponent bits, 3 mantissa bits); E = 0 is subnormal,
    M 2^-9; otherwise (1 + M / 8) 2^(E - 7); the code with E = 15, M = 7 is NaN."""
    out = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        out.append(m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return out


def e4m3_nearest(x: float) -> float:
    """x rounded to E4M3 by searching the decoded values: the nearest, and on a tie the one
    whose code has an even mantissa (its lowest bit clear); beyond 448 the largest."""
    vals = e4m3_values()
    a = abs(x)
    best = None
    for code, v in enumerate(vals):
        dist = abs(a - v)
        if best is None or dist < best[0] or (dist == best[0] and (code & 1) == 0):
            best = (dist, code, v)
    return math.copysign(best[2], x)
