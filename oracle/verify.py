"""Plain CPU oracle for packed draft-token verification (float64 NumPy).

Test infrastructure only: tests, the smoke check and the benchmark's CPU
baseline may call it; the product path never does. It shares no code with
the HIP library; the only thing both sides consume is the synthetic input
generator in `synth/`, which holds none of the arithmetic below.

What is computed, and where the pages fix it:

* Greedy target (temperature 0) selects the target's arg-max token; a
  positive temperature samples the target, and mixed temperatures may share a
  batch (xLLM docs, "Adaptive speculative inference", DSpark section "Launch
  example").
* The random target path samples every verify row; per-request parameters are
  reached through a packed-row owner map; with a deterministic (point-mass)
  draft the rejection sampler reduces to prefix matching: the run of leading
  matches is accepted, the sample at the first mismatch replaces the draft,
  and when every draft matches, the last row's sample is the bonus token
  (same page and section).
* Strict top-1 acceptance accepts a draft token only if it equals the target
  greedy token; relaxed top-K acceptance accepts it if it lies in the target
  top-K, which changes generated text (vllm-hust-vspec 0.13.0 README,
  sections "Scope of support" and "EAGLE features").
* Draft confidence is exp(selected_logit - logsumexp(draft_logits)), the
  selected token's draft probability (xLLM docs, "Adaptive speculative
  inference", section "Adaptive target verification from MTP logits").

Readings taken where the pages are silent (each listed in the design notes):
row layout K_i draft-verify rows then the bonus row; arg-max ties go to the
lowest index; rank order is (value desc, index asc); filters apply in the
order top-k, top-p (renormalised over the top-k survivors, shortest prefix
whose mass reaches top_p), min-p (z >= ln(min_p) with z = (x - max) / T);
u from Philox4x32-10 keyed (seed; request, local row, offset); inverse CDF in
rank order with a strict ">"; row_lse is the log-sum-exp of the logits the
row uses (x, or x / T when sampled).

Parity-pinned by tests/test_oracle_*.py (closed forms, brute force on tiny
vocabularies, textbook special cases, rocRAND's Philox engine).
"""
import math

import numpy as np

from .philox import row_uniform

F32 = 0
BF16 = 1


class PreconditionError(ValueError):
    """Input that the device path can only flag, never check up front."""


def bf16_bits_to_f64(bits):
    """Exact widening of raw bfloat16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def row_f64(logits, dtype, r, vocab):
    """Row r of a packed [rows, ld] logits array, first `vocab` entries."""
    if dtype == BF16:
        return bf16_bits_to_f64(logits[r, :vocab])
    if dtype == F32:
        return np.asarray(logits[r, :vocab], dtype=np.float32).astype(np.float64)
    raise ValueError("unknown dtype")


def check_row(x):
    if np.isnan(x).any() or np.isposinf(x).any():
        raise PreconditionError("NaN or +inf logit")
    if np.isneginf(x).all():
        raise PreconditionError("row is entirely -inf")


# --------------------------------------------------------------------------
# Row reductions


def greedy_token(x):
    """Lowest index attaining the row maximum (IEEE compare: -0 == +0)."""
    m = np.max(x)
    return int(np.flatnonzero(x == m)[0])


def logsumexp(x, temperature=1.0):
    """log sum_t exp(x_t / T), evaluated as m/T + log sum exp((x - m)/T)."""
    m = np.max(x)
    z = (x - m) / temperature
    return float(m / temperature + math.log(np.sum(np.exp(z))))


def rank_of(x, t):
    """Position of token t in the order (value desc, index asc), 0-based."""
    v = x[t]
    return int(np.count_nonzero(x > v) + np.count_nonzero(x[:t] == v))


def rank_order(x):
    """All token ids sorted by (value desc, index asc)."""
    return np.lexsort((np.arange(x.shape[0]), -x))


def filtered_support(x, temperature, top_k, top_p, min_p):
    """Survivor set S (in rank order) and the weights w_t = exp((x_t - m)/T).

    Filters, in the order the page lists them: top-k keeps the first top_k
    tokens of the rank order (off when top_k <= 0 or >= V); top-p keeps the
    shortest prefix of those whose weight reaches top_p of their total, the
    crossing token included (off when top_p >= 1); min-p keeps tokens with
    (x - m)/T >= ln(min_p), i.e. probability at least min_p times the
    largest one (off when min_p <= 0). Every stage keeps a prefix of the rank
    order and keeps the arg-max.
    """
    V = x.shape[0]
    m = np.max(x)
    z = (x - m) / temperature
    w = np.exp(z)
    order = rank_order(x)
    S = order
    if 0 < top_k < V:
        S = S[:top_k]
    if top_p < 1.0:
        c = np.cumsum(w[S])
        W = c[-1]
        L = int(np.flatnonzero(c >= top_p * W)[0]) + 1
        S = S[:L]
    if min_p > 0.0:
        keep = z[S] >= math.log(min_p)
        S = S[keep]
    return S, w


def sample_from_u(x, temperature, top_k, top_p, min_p, u):
    """Inverse CDF of the filtered, renormalised distribution at u in [0,1).

    The chosen token is S[n] for the smallest n whose cumulative weight (in
    rank order) is strictly greater than u times the survivor total.
    """
    S, w = filtered_support(x, temperature, top_k, top_p, min_p)
    c = np.cumsum(w[S])
    n = int(np.flatnonzero(c > u * c[-1])[0])
    return int(S[n])


# --------------------------------------------------------------------------
# Packed batch verification


def _check_layout(offsets, owner, num_rows):
    off = np.asarray(offsets, dtype=np.int64)
    B = off.shape[0] - 1
    if B < 0 or off[0] != 0 or off[-1] != num_rows or np.any(np.diff(off) < 1):
        raise PreconditionError("row offsets must start at 0, end at R and grow by >= 1")
    if owner is not None:
        own = np.asarray(owner, dtype=np.int64)
        expect = np.repeat(np.arange(B), np.diff(off))
        if own.shape[0] != num_rows or np.any(own != expect):
            raise PreconditionError("row owners disagree with row offsets")
    return off, B


def _prefix_accept(tokens, accepts, drafts):
    """Accepted length, next token and emitted tokens of one request.

    a = number of leading accepted drafts; the token at row a is the
    replacement (a < K) or the bonus (a == K); the emitted tokens are the
    accepted drafts followed by that token.
    """
    a = 0
    while a < len(accepts) and accepts[a]:
        a += 1
    nxt = int(tokens[a])
    return a, nxt, [int(d) for d in drafts[:a]] + [nxt]


def _compact(B, results):
    accepted = np.zeros(B, dtype=np.int32)
    nxt = np.zeros(B, dtype=np.int32)
    out_off = np.zeros(B + 1, dtype=np.int32)
    toks = []
    for i, (a, n, emitted) in enumerate(results):
        accepted[i] = a
        nxt[i] = n
        out_off[i + 1] = out_off[i] + a + 1
        toks.extend(emitted)
    return accepted, nxt, out_off, np.asarray(toks, dtype=np.int32)


def verify_greedy(logits, dtype, vocab, offsets, owner, drafts, relaxed_topk=1):
    """Greedy target verification of a packed batch.

    logits: [R, ld] float32, or uint16 bfloat16 bits; request i owns rows
    offsets[i] .. offsets[i+1]-1 (its K_i verify rows, then its bonus row);
    its j-th draft token is drafts[offsets[i] - i + j]. relaxed_topk == 1 is
    strict top-1 acceptance; K > 1 accepts a draft whose rank is below K and
    emits the accepted draft token itself.
    """
    R = logits.shape[0]
    off, B = _check_layout(offsets, owner, R)
    drafts = np.asarray(drafts, dtype=np.int64)
    if drafts.shape[0] != R - B:
        raise ValueError("need R - B draft tokens")
    if not 1 <= relaxed_topk <= vocab:
        raise ValueError("relaxed_topk must lie in [1, V]")
    row_token = np.zeros(R, dtype=np.int32)
    row_lse = np.zeros(R, dtype=np.float64)
    results = []
    for i in range(B):
        r0, r1 = int(off[i]), int(off[i + 1])
        K = r1 - r0 - 1
        d = drafts[r0 - i : r0 - i + K]
        accepts = []
        for j in range(K + 1):
            x = row_f64(logits, dtype, r0 + j, vocab)
            check_row(x)
            row_token[r0 + j] = greedy_token(x)
            row_lse[r0 + j] = logsumexp(x)
            if j < K:
                t = int(d[j])
                if not 0 <= t < vocab:
                    accepts.append(False)
                elif relaxed_topk == 1:
                    accepts.append(t == row_token[r0 + j])
                else:
                    accepts.append(rank_of(x, t) < relaxed_topk)
        results.append(_prefix_accept(row_token[r0 : r1], accepts, d))
    acc, nxt, out_off, toks = _compact(B, results)
    return dict(accepted_len=acc, next_token=nxt, out_offsets=out_off,
                out_tokens=toks, row_token=row_token, row_lse=row_lse)


def relaxed_accepts(x, j, generated, draft, topk=1, margin=0.0, from_position=0, after_tokens=0,
                    protected=()):
    """Whether greedy verification accepts `draft` at draft position j of a
    request that has generated `generated` tokens, given its target row x.

    The pages name these switches without formulas (vllm-hust-vspec 0.13.0
    README: "Launch" sets a confidence-accept margin of 5.25 and says it
    relaxes greedy acceptance; "General parameters" lists the margin, its
    from-position and after-tokens gates and protected token ids; "EAGLE
    features" lists top-K relaxed acceptance, its after-tokens gate and the
    strict prefix). The reading taken here:
      * a draft equal to the target's greedy token is always accepted;
      * otherwise relaxation applies only at positions j >= from_position
        where generated + j >= after_tokens (the first tokens of an answer
        and of a window stay strict), and only when neither the draft nor
        the greedy token is protected;
      * where it applies, top-K accepts a draft whose rank is below topk
        (topk > 1), and the margin accepts a draft whose logit lies less than
        `margin` below the row maximum (margin > 0), i.e. whose target
        log-probability is within `margin` of the greedy token's.
    With topk = 1 and margin = 0 every draft is verified strictly.
    """
    V = x.shape[0]
    if not 0 <= draft < V:
        return False
    g = greedy_token(x)
    if draft == g:
        return True
    if j < from_position or generated + j < after_tokens:
        return False
    if draft in protected or g in protected:
        return False
    if topk > 1 and rank_of(x, draft) < topk:
        return True
    if margin > 0.0 and float(np.max(x)) - float(x[draft]) < margin:
        return True
    return False


def verify_greedy_relaxed(logits, dtype, vocab, offsets, owner, drafts, topk=1, margin=0.0, from_position=0,
                          after_tokens=0, generated=None, protected=()):
    """Greedy verification with the relaxed acceptance variants of
    relaxed_accepts. generated[i] is request i's count of generated tokens
    (None: 0 for all); margin is read as the float32 value the device takes.
    An accepted draft is emitted as itself; the replacement and bonus are
    the greedy tokens."""
    R = logits.shape[0]
    off, B = _check_layout(offsets, owner, R)
    drafts = np.asarray(drafts, dtype=np.int64)
    if drafts.shape[0] != R - B:
        raise ValueError("need R - B draft tokens")
    if not 1 <= topk <= vocab:
        raise ValueError("topk must lie in [1, V]")
    margin = float(np.float32(margin))
    gen = np.zeros(B, dtype=np.int64) if generated is None else np.asarray(generated, dtype=np.int64)
    prot = set(int(t) for t in protected)
    row_token = np.zeros(R, dtype=np.int32)
    row_lse = np.zeros(R, dtype=np.float64)
    results = []
    for i in range(B):
        r0, r1 = int(off[i]), int(off[i + 1])
        K = r1 - r0 - 1
        d = drafts[r0 - i: r0 - i + K]
        accepts = []
        for j in range(K + 1):
            x = row_f64(logits, dtype, r0 + j, vocab)
            check_row(x)
            row_token[r0 + j] = greedy_token(x)
            row_lse[r0 + j] = logsumexp(x)
            if j < K:
                accepts.append(relaxed_accepts(x, j, int(gen[i]), int(d[j]), topk, margin, from_position,
                                               after_tokens, prot))
        results.append(_prefix_accept(row_token[r0: r1], accepts, d))
    acc, nxt, out_off, toks = _compact(B, results)
    return dict(accepted_len=acc, next_token=nxt, out_offsets=out_off,
                out_tokens=toks, row_token=row_token, row_lse=row_lse)


def verify_sampled(logits, dtype, vocab, offsets, owner, drafts, temperature,
                   top_k, top_p, min_p, seed, offset, uniforms=None):
    """Sampled (or mixed) target verification of a packed batch.

    Per-request parameters are float32 temperature/top_p/min_p and int32
    top_k, read exactly as the device reads them. Requests with temperature 0
    use the greedy rule. Every row of a sampled request draws its own token
    with u = Philox(seed; request, local row, offset); `uniforms`, if given,
    maps (request, row) -> u and overrides the generator (tests only).
    """
    R = logits.shape[0]
    off, B = _check_layout(offsets, owner, R)
    drafts = np.asarray(drafts, dtype=np.int64)
    if drafts.shape[0] != R - B:
        raise ValueError("need R - B draft tokens")
    T = np.asarray(temperature, dtype=np.float32).astype(np.float64)
    TK = np.asarray(top_k, dtype=np.int64)
    TP = np.asarray(top_p, dtype=np.float32).astype(np.float64)
    MP = np.asarray(min_p, dtype=np.float32).astype(np.float64)
    row_token = np.zeros(R, dtype=np.int32)
    row_lse = np.zeros(R, dtype=np.float64)
    results = []
    for i in range(B):
        if not (T[i] >= 0 and 0 < TP[i] <= 1 and 0 <= MP[i] <= 1):
            raise PreconditionError("sampling parameters out of range")
        r0, r1 = int(off[i]), int(off[i + 1])
        K = r1 - r0 - 1
        d = drafts[r0 - i : r0 - i + K]
        accepts = []
        for j in range(K + 1):
            x = row_f64(logits, dtype, r0 + j, vocab)
            check_row(x)
            if T[i] == 0:
                tok = greedy_token(x)
                row_lse[r0 + j] = logsumexp(x)
            else:
                if uniforms is not None:
                    u = uniforms[(i, j)]
                else:
                    u = row_uniform(seed, i, j, offset)
                tok = sample_from_u(x, T[i], int(TK[i]), TP[i], MP[i], u)
                row_lse[r0 + j] = logsumexp(x, T[i])
            row_token[r0 + j] = tok
            if j < K:
                accepts.append(int(d[j]) == tok)
        results.append(_prefix_accept(row_token[r0 : r1], accepts, d))
    acc, nxt, out_off, toks = _compact(B, results)
    return dict(accepted_len=acc, next_token=nxt, out_offsets=out_off,
                out_tokens=toks, row_token=row_token, row_lse=row_lse)


def draft_confidence(draft_logits, dtype, vocab, selected=None):
    """c_q = exp(y[sel_q] - logsumexp(y)) for every draft row q.

    Raw draft logits, no temperature; `selected` None means the draft row's
    own arg-max (lowest index). Returns (confidence, lse) in float64.
    """
    D = draft_logits.shape[0]
    conf = np.zeros(D, dtype=np.float64)
    lse = np.zeros(D, dtype=np.float64)
    for q in range(D):
        y = row_f64(draft_logits, dtype, q, vocab)
        check_row(y)
        s = greedy_token(y) if selected is None else int(selected[q])
        lse[q] = logsumexp(y)
        conf[q] = math.exp(y[s] - lse[q]) if 0 <= s < vocab else 0.0
    return conf, lse


# --------------------------------------------------------------------------
# Decision margins (used to re-draw synthetic sampled rows whose outcome
# would hinge on rounding; see the input recipe)


def sampled_row_margins(x, temperature, top_k, top_p, min_p, u):
    """Distances of the row's three float decisions from their thresholds.

    Returns (topp_margin, u_margin, minp_margin): how far, in normalised
    cumulative mass, the top-p target and u*W' lie from the nearest
    cumulative boundary, and how far the nearest z = (x - m)/T of a top-p
    survivor lies from ln(min_p). inf where a decision does not apply.
    """
    V = x.shape[0]
    m = np.max(x)
    z = (x - m) / temperature
    w = np.exp(z)
    S = rank_order(x)
    if 0 < top_k < V:
        S = S[:top_k]
    topp_margin = math.inf
    if top_p < 1.0:
        c = np.cumsum(w[S])
        cn = c / c[-1]
        L = int(np.flatnonzero(c >= top_p * c[-1])[0])
        topp_margin = cn[L] - top_p
        if L > 0:
            topp_margin = min(topp_margin, top_p - cn[L - 1])
        S = S[: L + 1]
    minp_margin = math.inf
    if min_p > 0.0:
        lm = math.log(min_p)
        # tokens equal to the maximum have z = 0 exactly on any machine
        zs = z[S][x[S] < m]
        if zs.size:
            minp_margin = float(np.min(np.abs(zs - lm)))
        S = S[z[S] >= lm]
    c = np.cumsum(w[S])
    cn = c / c[-1]
    n = int(np.flatnonzero(c > u * c[-1])[0])
    u_margin = cn[n] - u
    if n > 0:
        u_margin = min(u_margin, u - cn[n - 1])
    return float(topp_margin), float(u_margin), float(minp_margin)
