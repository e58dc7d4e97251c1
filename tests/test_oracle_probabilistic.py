"""Pins of the probabilistic-draft verification oracle (CPU only).

The rejection sampler's defining property: whatever the draft law q, the
first emitted token, averaged over drafts drawn from q, has the target law
p. Both uniforms are enumerated on grids, so the law is computed exactly up
to the grid step. Further pins: a point-mass draft gives the point-mass
path's law, q = p always accepts, a greedy target accepts exactly its
arg-max, and a batch worked by hand."""
import numpy as np
import pytest

import oracle
from oracle.philox import philox4x32_10
from oracle.probabilistic import (accepts, draft_probs, residual_draw, row_uniforms, target_probs,
                                  verify_probabilistic)

GRID = 1 << 13
US = np.arange(GRID) / GRID          # exact multiples of the grid step, in [0, 1)


def _first_token_law(x, y, T, tk, tp, mp, Td):
    p = target_probs(x, T, tk, tp, mp)
    q = draft_probs(y, Td)
    V = x.shape[0]
    law = np.zeros(V)
    for d in range(V):
        if q[d] == 0:
            continue
        pacc = np.mean([accepts(p, q, d, u) for u in US])
        law[d] += q[d] * pacc
        if pacc < 1:
            res = np.zeros(V)
            for u in US:
                res[residual_draw(x, p, q, u)] += 1.0 / GRID
            law += q[d] * (1 - pacc) * res
    return law, p


CASES = [(1.0, 0, 1.0, 0.0, 1.0), (0.7, 0, 1.0, 0.0, 1.3), (1.0, 3, 1.0, 0.0, 0.8), (1.2, 0, 0.8, 0.0, 1.0),
         (1.0, 0, 1.0, 0.2, 0.5), (0.0, 0, 1.0, 0.0, 1.0), (1.0, 0, 1.0, 0.0, 0.0), (0.9, 4, 0.9, 0.05, 2.0)]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_first_token_has_the_target_law(case):
    T, tk, tp, mp, Td = CASES[case]
    rng = np.random.default_rng(40 + case)
    x = rng.normal(0, 1.5, 6)
    y = rng.normal(0, 1.5, 6)
    law, p = _first_token_law(x, y, T, tk, tp, mp, Td)
    assert np.allclose(law, p, atol=3.0 / GRID, rtol=0), (law, p)


def test_point_mass_draft_gives_the_point_mass_law():
    # Td = 0: q is a point mass at the draft row's arg-max d*. The sampled
    # path accepts d* iff its own draw equals d*, and otherwise emits that
    # draw: the same law as accepting with probability p(d*) and drawing the
    # residual p restricted to the other tokens
    rng = np.random.default_rng(7)
    for _ in range(5):
        x = rng.normal(0, 1.0, 5)
        y = rng.normal(0, 1.0, 5)
        p = target_probs(x, 0.9, 0, 0.95, 0.0)
        q = draft_probs(y, 0.0)
        ds = int(np.argmax(q))
        own = np.array([oracle.sample_from_u(x, 0.9, 0, 0.95, 0.0, u) for u in US])
        pacc = np.mean([accepts(p, q, ds, u) for u in US])
        assert abs(pacc - np.mean(own == ds)) <= 2.0 / GRID
        if pacc < 1:
            res = np.bincount([residual_draw(x, p, q, u) for u in US], minlength=5) / GRID
            cond = np.bincount(own[own != ds], minlength=5) / max(1, np.count_nonzero(own != ds))
            assert np.allclose(res, cond, atol=3.0 / GRID)


def test_equal_laws_always_accept():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 2.0, 8)
    p = target_probs(x, 1.1, 0, 1.0, 0.0)
    q = draft_probs(x, 1.1)
    for d in range(8):
        assert all(accepts(p, q, d, u) for u in US[::64])


def test_greedy_target_accepts_only_its_argmax():
    rng = np.random.default_rng(5)
    x = rng.normal(0, 2.0, 7)
    y = rng.normal(0, 2.0, 7)
    g = int(np.argmax(x))
    p = target_probs(x, 0.0, 0, 1.0, 0.0)
    q = draft_probs(y, 1.0)
    for d in range(7):
        got = [accepts(p, q, d, u) for u in US[::128]]
        assert all(got) if d == g else not any(got)
    assert all(residual_draw(x, p, q, u) == g for u in US[::128])


def test_uniforms_are_the_sampled_paths_and_the_next_word():
    for (s, i, j, o) in [(1, 0, 0, 0), (2005, 17, 3, 9), (2**40 + 5, 511, 7, 2**33)]:
        u, ua = row_uniforms(s, i, j, o)
        assert u == oracle.row_uniform(s, i, j, o)
        w = philox4x32_10((j, i, o & 0xFFFFFFFF, o >> 32), (s & 0xFFFFFFFF, s >> 32))
        assert ua == (w[1] >> 8) / 16777216.0


def test_batch_worked_by_hand():
    # p = (1/2, 1/4, 1/8, 1/8) on every target row (x = log p, T = 1, no
    # filters), q uniform on every draft row. Draft 0 and draft 1 have
    # p/q >= 1 and are always accepted; draft 2 has p/q = 1/2. The residual
    # max(0, p - q) is (1/4, 0, 0, 0): every rejection emits token 0.
    p = np.array([0.5, 0.25, 0.125, 0.125])
    x = np.log(p).astype(np.float32)
    logits = np.tile(x, (6, 1))
    dlog = np.zeros((4, 4), dtype=np.float32)
    off = np.array([0, 3, 6])
    owner = np.array([0, 0, 0, 1, 1, 1])
    drafts = np.array([0, 2, 1, 0])
    U = {(0, 0): (0.1, 0.9), (0, 1): (0.3, 0.7), (0, 2): (0.2, 0.0),
         (1, 0): (0.4, 0.99), (1, 1): (0.5, 0.99), (1, 2): (0.6, 0.0)}
    out = verify_probabilistic(logits, oracle.F32, 4, off, owner, drafts, dlog, [1.0, 1.0], [0, 0], [1.0, 1.0],
                               [0.0, 0.0], [1.0, 1.0], 0, 0, uniforms=U)
    # request 0: draft 0 accepted, draft 2 rejected (0.7 >= 1/2): residual 0
    # request 1: drafts 1 and 0 accepted: bonus draw at u = 0.6 -> token 1
    assert list(out["accepted_len"]) == [1, 2]
    assert list(out["next_token"]) == [0, 1]
    assert list(out["out_offsets"]) == [0, 2, 5]
    assert list(out["out_tokens"]) == [0, 0, 1, 0, 1]
    assert list(out["accept_bits"]) == [True, False, True, True]
    # with u_acc below 1/2 the same draft 2 is accepted
    U[(0, 1)] = (0.3, 0.4)
    out = verify_probabilistic(logits, oracle.F32, 4, off, owner, drafts, dlog, [1.0, 1.0], [0, 0], [1.0, 1.0],
                               [0.0, 0.0], [1.0, 1.0], 0, 0, uniforms=U)
    assert list(out["accepted_len"]) == [2, 2]


def test_probabilistic_margins_bound_the_decisions():
    """Moving u_acc by half the acceptance margin (relative) keeps the
    acceptance; moving it just past flips it. Moving u by half the residual
    margin (in residual mass) keeps the residual draw; just past changes it."""
    from oracle.probabilistic import accepts, residual_draw, row_margins
    rng = np.random.default_rng(4800)
    flips = draws = 0
    for trial in range(80):
        V = int(rng.integers(6, 120))
        x = rng.standard_normal(V) * 2.0
        y = x + 0.8 * rng.standard_normal(V)
        T, k, tp, mp = float(rng.choice([0.7, 1.0])), int(rng.choice([0, 10])), float(rng.choice([1.0, 0.9])), 0.0
        Td = float(rng.choice([0.7, 1.0]))
        p = target_probs(x, T, k, tp, mp)
        q = draft_probs(y, Td)
        d = int(rng.choice(V, p=q))
        u, ua = float(rng.uniform(0.01, 0.99)), float(rng.uniform(0.01, 0.99))
        am, rm = row_margins(x, y, T, k, tp, mp, Td, d, u, ua)
        if np.isfinite(am):
            ok = accepts(p, q, d, ua)
            # ua * q(d) moves by the margin's share of the larger side
            step = am * max(p[d], ua * q[d]) / q[d]
            assert accepts(p, q, d, ua + 0.5 * step) == ok and accepts(p, q, d, ua - 0.5 * step) == ok
            toward = ua + step * (1 + 1e-9) if ok else ua - step * (1 + 1e-9)
            assert accepts(p, q, d, toward) != ok, trial
            flips += 1
        if np.isfinite(rm):
            tot = float(np.sum(np.maximum(p - q, 0.0)))
            t0 = residual_draw(x, p, q, u)
            du = rm / tot
            assert residual_draw(x, p, q, u + 0.5 * du) == t0 and residual_draw(x, p, q, u - 0.5 * du) == t0
            moved = [residual_draw(x, p, q, v) for v in (u + du * (1 + 1e-9), u - du * (1 + 1e-9)) if 0 <= v < 1]
            if not any(m != t0 for m in moved):
                # the nearest boundary is 0 or the whole residual mass, which
                # no u in [0, 1) passes
                assert min(abs(u + du - 1.0), abs(u - du)) < 1e-9, trial
                continue
            draws += 1
    assert flips > 40 and draws > 40
