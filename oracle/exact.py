"""Exact rational evaluation of linear attention from its definition.

Test infrastructure only.  Used to write the worked examples under
``tests/golden/`` that pin the fp64 C oracle.  It evaluates the generalised
attention definition directly -- out_i = sum_j sim(q_i, k_j) v_j / sum_j
sim(q_i, k_j) with sim(q, k) = phi(q) . phi(k) -- as a double sum over token
pairs, in exact fractions ("Transformers are RNNs" blog digest, section
"Methods"; velog review sections 3.1 "Transformers" and 3.2 "Linearized
Attention"; itwiki "Linear attention", section "Formulas").  For the causal
form the inner sum runs over j <= i (velog review section 3.4 "Causal
Masking").

phi(x) = elu(x) + 1 is rational only for x >= 0 (x + 1 for x > 0 and
exp(0) = 1 at x = 0), so inputs q and k must be non-negative rationals here;
v and the upstream gradient may be any rationals.

Gradients are obtained by forward-mode differentiation with exact dual
numbers of the same double sum, one input element at a time -- no hand-derived
gradient formula is involved.  On x >= 0 the derivative of phi is 1 (at x = 0
both branches have slope 1).
"""
from __future__ import annotations

from fractions import Fraction
from typing import List, Sequence


class Dual:
    """a + b*eps with eps^2 = 0, over exact fractions."""

    __slots__ = ("a", "b")

    def __init__(self, a, b=0):
        self.a = Fraction(a)
        self.b = Fraction(b)

    @staticmethod
    def lift(x):
        return x if isinstance(x, Dual) else Dual(x, 0)

    def __add__(self, o):
        o = Dual.lift(o)
        return Dual(self.a + o.a, self.b + o.b)

    __radd__ = __add__

    def __sub__(self, o):
        o = Dual.lift(o)
        return Dual(self.a - o.a, self.b - o.b)

    def __rsub__(self, o):
        return Dual.lift(o) - self

    def __mul__(self, o):
        o = Dual.lift(o)
        return Dual(self.a * o.a, self.a * o.b + self.b * o.a)

    __rmul__ = __mul__

    def __truediv__(self, o):
        o = Dual.lift(o)
        return Dual(self.a / o.a, (self.b * o.a - self.a * o.b) / (o.a * o.a))


def phi(x):
    """elu(x) + 1 for rational x >= 0 (value x + 1, or 1 at x = 0; slope 1)."""
    xa = x.a if isinstance(x, Dual) else Fraction(x)
    if xa < 0:
        raise ValueError("exact evaluation needs non-negative q and k entries")
    if xa > 0:
        return x + 1
    # x == 0: exp(0) = 1 and the slope of exp at 0 is 1, so phi = 1 + x there.
    return Dual.lift(x) + 1 if isinstance(x, Dual) else Fraction(1)


def attention(q: Sequence[Sequence], k: Sequence[Sequence], v: Sequence[Sequence],
              causal: bool) -> List[List]:
    """One (batch, head) slice: q, k are N x dk, v is N x dv; returns N x dv."""
    N = len(q)
    out = []
    for i in range(N):
        fq = [phi(x) for x in q[i]]
        num = [Fraction(0)] * len(v[0])
        den = Fraction(0)
        last = i + 1 if causal else N
        for j in range(last):
            fk = [phi(x) for x in k[j]]
            s = sum((a * b for a, b in zip(fq, fk)), Fraction(0))
            den = den + s
            num = [n + s * vv for n, vv in zip(num, v[j])]
        out.append([n / den for n in num])
    return out


def denominators(q, k, causal: bool = True) -> List:
    """den_i = sum over the attended j of phi(q_i) . phi(k_j)."""
    N = len(q)
    res = []
    for i in range(N):
        fq = [phi(x) for x in q[i]]
        last = i + 1 if causal else N
        d = Fraction(0)
        for j in range(last):
            fk = [phi(x) for x in k[j]]
            d += sum((a * b for a, b in zip(fq, fk)), Fraction(0))
        res.append(d)
    return res


def _loss(q, k, v, g, causal):
    out = attention(q, k, v, causal)
    total = Dual(0)
    for oi, gi in zip(out, g):
        for a, b in zip(oi, gi):
            total = total + Dual.lift(a) * b
    return total


def gradients(q, k, v, g, causal: bool = True):
    """Exact dL/dq, dL/dk, dL/dv for L = sum_i g_i . out_i, by dual numbers."""
    q = [[Fraction(x) for x in r] for r in q]
    k = [[Fraction(x) for x in r] for r in k]
    v = [[Fraction(x) for x in r] for r in v]
    g = [[Fraction(x) for x in r] for r in g]

    def seeded(mat, i, e):
        return [[Dual(x, 1 if (a == i and b == e) else 0) for b, x in enumerate(r)]
                for a, r in enumerate(mat)]

    dq = [[_loss(seeded(q, i, e), k, v, g, causal).b for e in range(len(q[0]))] for i in range(len(q))]
    dk = [[_loss(q, seeded(k, i, e), v, g, causal).b for e in range(len(k[0]))] for i in range(len(k))]
    dv = [[_loss(q, k, seeded(v, i, e), g, causal).b for e in range(len(v[0]))] for i in range(len(v))]
    return dq, dk, dv
