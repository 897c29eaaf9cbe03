"""Pure-Python fp64 brute force for tiny rows -- TEST INFRASTRUCTURE ONLY.

A second, independent evaluation of the same definitions as ``vjsd_oracle.c``,
written the other way round: it works in the probability domain (normalised
exponentials summed with ``math.fsum``, divergences as ``p * log(p / q)``) where
the C oracle works with log-probabilities and ``logaddexp``, and it takes
gradients by central finite differences instead of closed forms.  Agreement of
the two on tiny inputs pins the C oracle's algebra.

Page keys: [JSD-PR] DeepSpeed PR #8958 "[VocabTP] Add vocabulary-parallel
generalized JSD with Triton kernels"; [OPS-PR] DeepSpeed PR #8791 "Add
vocabulary-parallel logprobs, entropy and KL ops".

Rows are Python lists of floats; ``-inf`` marks a masked token.
"""
from __future__ import annotations

import math

NINF = float("-inf")


def softmax(x):
    """Probabilities of a logit row, or None when every logit is -inf [OPS-PR, How]."""
    m = max(x)
    if m == NINF:
        return None
    e = [math.exp(v - m) if v != NINF else 0.0 for v in x]
    z = math.fsum(e)
    return [v / z for v in e]


def _kl(p, q, support_p, support_q):
    """KL(p || q) over p's support; +inf if p's support leaves q's [OPS-PR, Tests]."""
    if any(a and not b for a, b in zip(support_p, support_q)):
        return math.inf
    return math.fsum(pi * math.log(pi / qi) for pi, qi, a in zip(p, q, support_p)
                     if a and pi > 0.0)


def jsd(s, t, beta):
    """Generalized JSD [JSD-PR, Motivation/Changes] in the probability domain."""
    ps, pt = softmax(s), softmax(t)
    if ps is None or pt is None:
        return math.nan
    sup_s = [v != NINF for v in s]
    sup_t = [v != NINF for v in t]
    if beta == 0.0:
        return _kl(pt, ps, sup_t, sup_s)
    if beta == 1.0:
        return _kl(ps, pt, sup_s, sup_t)
    M = [beta * a + (1.0 - beta) * b for a, b in zip(pt, ps)]
    sup_m = [a or b for a, b in zip(sup_t, sup_s)]
    return beta * _kl(pt, M, sup_t, sup_m) + (1.0 - beta) * _kl(ps, M, sup_s, sup_m)


def entropy(x):
    p = softmax(x)
    if p is None:
        return math.nan
    return -math.fsum(pi * math.log(pi) for pi in p if pi > 0.0)


def logprob(x, i):
    p = softmax(x)
    if p is None:
        return math.nan
    return math.log(p[i]) if p[i] > 0.0 else NINF


def fd_grad(f, x, h=1e-5):
    """Central finite differences of f at every finite coordinate of x (0 at -inf)."""
    g = []
    for i, v in enumerate(x):
        if v == NINF:
            g.append(0.0)
            continue
        xp = list(x)
        xm = list(x)
        xp[i] = v + h
        xm[i] = v - h
        g.append((f(xp) - f(xm)) / (2.0 * h))
    return g
