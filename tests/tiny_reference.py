"""Brute-force pure-Python statements of the sampling law, for tiny vocabularies.

Used only to pin the NumPy oracle. Each quantity is re-derived by plain
enumeration rather than by the oracle's vectorised steps: ranks by counting
how many tokens beat a token, prefix masses with math.fsum over every prefix
length, and the min-p rule in probability form (p_t >= min_p * p_max) rather
than the oracle's log form.
"""
import math


def rank(xs, t):
    return sum(1 for s in range(len(xs)) if xs[s] > xs[t] or (xs[s] == xs[t] and s < t))


def filtered_law(xs, T, top_k, top_p, min_p):
    """Exact filtered, renormalised distribution {token: probability}."""
    V = len(xs)
    m = max(xs)
    w = [math.exp((x - m) / T) for x in xs]
    by_rank = [None] * V
    for t in range(V):
        by_rank[rank(xs, t)] = t
    S = by_rank[:top_k] if 0 < top_k < V else by_rank
    if top_p < 1.0:
        total = math.fsum(w[t] for t in S)
        for L in range(1, len(S) + 1):
            if math.fsum(w[t] for t in S[:L]) >= top_p * total:
                S = S[:L]
                break
    if min_p > 0.0:
        Zs = math.fsum(w)
        pmax = 1.0 / Zs
        S = [t for t in S if w[t] / Zs >= min_p * pmax]
    Z = math.fsum(w[t] for t in S)
    return {t: w[t] / Z for t in S}


def rejection_law(rows, drafts, params):
    """Law of (accepted length, next token) of the textbook rejection sampler.

    A point-mass draft d is accepted with probability min(1, p(d)/q(d)) = p(d);
    on rejection the replacement is drawn from the residual max(0, p - q)
    renormalised, which is p restricted to t != d. After K accepted drafts
    the bonus is drawn from the last row's p.
    """
    K = len(drafts)
    ps = [filtered_law(x, *params) for x in rows]
    law = {}
    prefix = 1.0
    for n in range(K + 1):
        p = ps[n]
        for t, pt in p.items():
            if n < K and t == drafts[n]:
                continue
            law[(n, t)] = law.get((n, t), 0.0) + prefix * pt
        if n < K:
            prefix *= p.get(drafts[n], 0.0)
    return law
