"""Verification with probabilistic drafts: CPU oracle (test infrastructure only).

Only tests/ call this module; the library does not implement it yet, and
nothing here comes from the library.

The pages support point-mass drafts only: their ragged verifier says that
with deterministic drafts, rejection sampling reduces to matching, and it
refuses probabilistic drafts before execution (xLLM docs, "Adaptive
speculative inference", DSpark section "Launch example"). This module
defines the general case that sentence reduces from: the rejection sampler
of speculative decoding, with the point-mass path as its special case.

Per request i with drafts d_0 .. d_{K-1}, target rows x_0 .. x_K and draft
rows y_0 .. y_{K-1}:

* p_j is the target's distribution at row j: the filtered, renormalised
  softmax of x_j / T_i that the sampled path draws from (top-k, top-p,
  min-p), or a point mass at the arg-max when T_i = 0;
* q_j is the draft's distribution: softmax(y_j / Td_i), or a point mass at
  the draft row's arg-max when Td_i = 0;
* draft j is accepted iff u_acc(i, j) * q_j(d_j) < p_j(d_j), which happens
  with probability min(1, p_j(d_j) / q_j(d_j));
* at the first rejected row j the request emits the residual draw: the
  inverse CDF, in the target's rank order (value desc, index asc), of
  max(0, p_j - q_j) at u(i, j), first cumulative weight strictly above
  u times the total;
* when all K drafts are accepted the request emits the bonus row's draw
  from p_K at u(i, K), exactly as the sampled path does.

Readings taken where nothing fixes them (listed in the design notes): q is
the unfiltered draft softmax at the request's draft temperature; u(i, j) is
the sampled path's uniform (word 0 of the Philox block at counter
(j, i, offset lo, offset hi)) and u_acc(i, j) = (word 1 >> 8) * 2^-24 of the
same block; a residual with no mass (possible only when p_j = q_j) emits the
row's draw from p_j.

Parity-pinned by tests/test_oracle_probabilistic.py: averaged over drafts
drawn from q, the first emitted token has law p (the defining property of
the rejection sampler), by enumeration of both uniforms on grids; the
point-mass draft gives the point-mass path's law; q = p accepts always; a
greedy target accepts exactly its arg-max; and a batch worked by hand.
"""

import numpy as np

from .philox import MASK32, philox4x32_10
from .verify import (_check_layout, _compact, _prefix_accept, filtered_support, greedy_token, rank_order,
                     row_f64, sample_from_u)


def target_probs(x, temperature, top_k, top_p, min_p):
    """p over all V tokens: the sampled path's filtered law, or the arg-max."""
    p = np.zeros(x.shape[0])
    if temperature == 0:
        p[greedy_token(x)] = 1.0
        return p
    S, w = filtered_support(x, temperature, top_k, top_p, min_p)
    p[S] = w[S] / np.sum(w[S])
    return p


def draft_probs(y, draft_temperature):
    """q over all V tokens: softmax(y / Td), or the arg-max when Td = 0."""
    q = np.zeros(y.shape[0])
    if draft_temperature == 0:
        q[greedy_token(y)] = 1.0
        return q
    z = (y - np.max(y)) / draft_temperature
    e = np.exp(z)
    return e / np.sum(e)


def accepts(p, q, d, u_acc):
    """Rejection test of draft d: u_acc * q(d) < p(d)."""
    return bool(u_acc * q[d] < p[d])


def residual_draw(x, p, q, u):
    """Inverse CDF of max(0, p - q) in the rank order of x at u (strict >)."""
    r = np.maximum(p - q, 0.0)
    order = rank_order(x)
    c = np.cumsum(r[order])
    if not c[-1] > 0:
        return None
    n = int(np.flatnonzero(c > u * c[-1])[0])
    return int(order[n])


def row_margins(x, y, temperature, top_k, top_p, min_p, draft_temperature, d, u, u_acc):
    """Distances of a draft row's two float decisions from their thresholds
    (used to re-draw synthetic rows whose outcome would hinge on rounding).

    Returns (accept_margin, residual_margin):
    * accept_margin: |p(d) - u_acc q(d)| relative to the larger of the two,
      inf when p(d) = 0 or q(d) = 0 (the test is then exact);
    * residual_margin: how far, in probability mass, u times the residual
      total lies from the nearest cumulative boundary of max(0, p - q) in
      rank order; inf when the residual has no mass (the row then emits its
      own draw, whose margin is the sampled path's).
    The filters' own cuts are the sampled path's margins."""
    p = target_probs(x, temperature, top_k, top_p, min_p)
    q = draft_probs(y, draft_temperature)
    accept_margin = np.inf
    if 0 <= d < x.shape[0] and p[d] > 0 and q[d] > 0:
        a, b = p[d], u_acc * q[d]
        accept_margin = abs(a - b) / max(a, b)
    residual = np.clip(p - q, 0.0, None)
    c = np.cumsum(residual[rank_order(x)])
    residual_margin = np.inf
    if c[-1] > 0:
        t = u * c[-1]
        n = int(np.flatnonzero(c > t)[0])
        residual_margin = c[n] - t
        if n > 0:
            residual_margin = min(residual_margin, t - c[n - 1])
    return float(accept_margin), float(residual_margin)


def row_uniforms(seed, request, row, offset):
    """(u, u_acc): words 0 and 1 of the Philox block of (request, row)."""
    seed, offset = int(seed), int(offset)
    w = philox4x32_10((int(row), int(request), offset & MASK32, (offset >> 32) & MASK32),
                      (seed & MASK32, (seed >> 32) & MASK32))
    return (w[0] >> 8) * (1.0 / 16777216.0), (w[1] >> 8) * (1.0 / 16777216.0)


def verify_probabilistic(logits, dtype, vocab, offsets, owner, drafts, draft_logits, temperature, top_k,
                         top_p, min_p, draft_temperature, seed, offset, uniforms=None):
    """Rejection-sampling verification of a packed batch.

    draft_logits holds the R - B draft rows, draft j of request i at
    off[i] - i + j (the drafts' layout). `uniforms`, if given, maps
    (request, row) -> (u, u_acc) (tests only). row_token holds, for a draft
    row, the residual draw it emits if it is the first rejection, and for a
    bonus row its draw from p.
    """
    R = logits.shape[0]
    off, B = _check_layout(offsets, owner, R)
    drafts = np.asarray(drafts, dtype=np.int64)
    if drafts.shape[0] != R - B or draft_logits.shape[0] != R - B:
        raise ValueError("need R - B draft tokens and draft rows")
    T = np.asarray(temperature, dtype=np.float32).astype(np.float64)
    TK = np.asarray(top_k, dtype=np.int64)
    TP = np.asarray(top_p, dtype=np.float32).astype(np.float64)
    MP = np.asarray(min_p, dtype=np.float32).astype(np.float64)
    TD = np.asarray(draft_temperature, dtype=np.float32).astype(np.float64)
    row_token = np.zeros(R, dtype=np.int32)
    accept_bits = np.zeros(R - B, dtype=bool)
    results = []
    for i in range(B):
        r0, r1 = int(off[i]), int(off[i + 1])
        K = r1 - r0 - 1
        d = drafts[r0 - i: r0 - i + K]
        acc = []
        for j in range(K + 1):
            x = row_f64(logits, dtype, r0 + j, vocab)
            u, u_acc = uniforms[(i, j)] if uniforms is not None else row_uniforms(seed, i, j, offset)
            if T[i] == 0:
                own = greedy_token(x)
            else:
                own = sample_from_u(x, T[i], int(TK[i]), TP[i], MP[i], u)
            if j == K:
                row_token[r0 + j] = own
                continue
            p = target_probs(x, T[i], int(TK[i]), TP[i], MP[i])
            y = row_f64(draft_logits, dtype, r0 - i + j, vocab)
            q = draft_probs(y, TD[i])
            ok = 0 <= d[j] < vocab and accepts(p, q, int(d[j]), u_acc)
            res = residual_draw(x, p, q, u)
            row_token[r0 + j] = own if res is None else res
            accept_bits[r0 - i + j] = ok
            acc.append(ok)
        results.append(_prefix_accept(row_token[r0:r1], acc, d))
    a, nxt, out_off, toks = _compact(B, results)
    return dict(accepted_len=a, next_token=nxt, out_offsets=out_off, out_tokens=toks,
                row_token=row_token, accept_bits=accept_bits)
