"""Exact rational brute force for tiny inputs (a pin for the oracle, not part of it).

Decodes bf16 bit patterns with pure-Python integer arithmetic and evaluates
dot products, row maxima and duplicate counts with fractions.Fraction, so every
comparison is exact.
"""
from fractions import Fraction


def bf16_value(bits: int) -> Fraction:
    s = (bits >> 15) & 1
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0xFF:
        raise ValueError("non-finite")
    if e == 0:
        v = Fraction(f, 2 ** 133)
    else:
        m = f | 0x80
        x = e - 134
        v = Fraction(m * 2 ** x) if x >= 0 else Fraction(m, 2 ** (-x))
    return -v if s else v


def dot(a, b) -> Fraction:
    return sum((bf16_value(int(x)) * bf16_value(int(y)) for x, y in zip(a, b)), Fraction(0))


def row_max_count(q, k, causal):
    """Per query row: (exact max of q_i.k_j over visible j, how many j reach it)."""
    n = len(q)
    out = []
    for i in range(n):
        last = i if causal else n - 1
        vals = [dot(q[i], k[j]) for j in range(last + 1)]
        m = max(vals)
        out.append((m, sum(1 for v in vals if v == m)))
    return out


def merge(a, b):
    """(max, count) merge of two partial rows: the larger max keeps its count, equal maxima add."""
    (ma, ca), (mb, cb) = a, b
    if ma > mb:
        return a
    if mb > ma:
        return b
    return (ma, ca + cb)
