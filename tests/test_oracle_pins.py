"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: NumPy/SciPy
textbook routines, closed forms built into the synthetic inputs, brute-force
enumeration on tiny vocabularies, the textbook rejection-sampling law, and
rocRAND's independent Philox4x32-10 engine.
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest
import scipy.special

import oracle
import synth
from tests import tiny_reference as tiny

HERE = os.path.dirname(os.path.abspath(__file__))
GRID = 1 << 24


# ---------------------------------------------------------------- Philox

@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND reference")
    exe = str(tmp_path_factory.mktemp("rr") / "rocrand_philox_ref")
    subprocess.run([hipcc, "-O1", os.path.join(HERE, "rocrand_philox_ref.cpp"), "-o", exe],
                   check=True, capture_output=True)
    return exe


def test_philox_matches_rocrand_engine(rocrand_ref):
    rng = np.random.default_rng(7)
    cases = [(0, 0, 0, 0, 0, 0), (0xFFFFFFFF, 0, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF)]
    for _ in range(300):
        c = [int(v) for v in rng.integers(0, 2**32, size=4, dtype=np.uint64)]
        c[1] = c[1] % (1 << 29)        # block index * 4 must fit in 64 bits
        k = [int(v) for v in rng.integers(0, 2**32, size=2, dtype=np.uint64)]
        cases.append(tuple(c + k))
    cases[1] = (0xFFFFFFFF, 5, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF)
    inp = "".join("%d %d %d %d %d %d\n" % cs for cs in cases)
    out = subprocess.run([rocrand_ref], input=inp, capture_output=True, text=True, check=True).stdout
    got = [tuple(int(v) for v in line.split()) for line in out.strip().splitlines()]
    assert len(got) == len(cases)
    for cs, ref in zip(cases, got):
        assert oracle.philox4x32_10(cs[:4], cs[4:]) == ref, cs


def test_row_uniform_is_on_the_24bit_grid():
    for (s, i, j, o) in [(0, 0, 0, 0), (2005, 3, 6, 0), (2**40 + 3, 511, 7, 2**33 + 1)]:
        u = oracle.row_uniform(s, i, j, o)
        assert 0.0 <= u < 1.0 and float(u * GRID).is_integer()
    # distinct rows and requests give distinct draws
    us = {oracle.row_uniform(2003, i, j, 0) for i in range(16) for j in range(8)}
    assert len(us) == 128


def test_row_uniform_is_rocrand_word0_on_the_grid(rocrand_ref):
    # reading c10: key = (seed lo, seed hi), counter = (row, request, offset
    # lo, offset hi), u = (word 0 >> 8) * 2^-24, word 0 from rocRAND's engine
    cases = [(0, 0, 0, 0), (2005, 3, 6, 0), (2**40 + 3, 511, 7, 2**33 + 1), (2**64 - 1, 7, 1, 2**64 - 1)]
    rng = np.random.default_rng(9)
    for _ in range(60):
        cases.append((int(rng.integers(0, 2**63)), int(rng.integers(0, 4096)), int(rng.integers(0, 8)),
                      int(rng.integers(0, 2**40))))
    m = 0xFFFFFFFF
    inp = "".join("%d %d %d %d %d %d\n" % (j, i, o & m, o >> 32, s_ & m, s_ >> 32) for (s_, i, j, o) in cases)
    out = subprocess.run([rocrand_ref], input=inp, capture_output=True, text=True, check=True).stdout
    words = [int(line.split()[0]) for line in out.strip().splitlines()]
    assert len(words) == len(cases)
    for (s_, i, j, o), w0 in zip(cases, words):
        assert oracle.row_uniform(s_, i, j, o) == (w0 >> 8) / GRID


def test_row_uniform_spans_the_unit_interval():
    us = np.array([oracle.row_uniform(2003, i, j, 0) for i in range(512) for j in range(8)])
    assert abs(us.mean() - 0.5) < 0.02
    assert us.min() < 0.01 and us.max() > 0.99
    assert abs(np.mean(us < 0.25) - 0.25) < 0.03


# ---------------------------------------------------------------- reductions

def _tied_rows(rng, n, V):
    for _ in range(n):
        yield rng.integers(-4, 5, size=V).astype(np.float64)


def test_greedy_token_is_numpy_first_argmax():
    rng = np.random.default_rng(1)
    for x in _tied_rows(rng, 300, 37):
        assert oracle.greedy_token(x) == int(np.argmax(x))
    x = np.array([-1.0, -0.0, 0.0, -3.0])
    assert oracle.greedy_token(x) == 1       # -0 == +0, lowest index wins
    x = np.array([-np.inf, -np.inf, -5.0, -np.inf])
    assert oracle.greedy_token(x) == 2


def test_logsumexp_matches_scipy_and_normalises():
    rng = np.random.default_rng(2)
    for T in (1.0, 0.5, 0.7, 2.0):
        for _ in range(20):
            x = rng.standard_normal(5000) * 3
            lse = oracle.logsumexp(x, T)
            assert lse == pytest.approx(scipy.special.logsumexp(x / T), rel=1e-13, abs=1e-13)
            assert math.fsum(np.exp(x / T - lse)) == pytest.approx(1.0, abs=1e-12)
    x = np.array([0.0, -np.inf, -np.inf])
    assert oracle.logsumexp(x) == 0.0


def test_rank_matches_brute_force():
    rng = np.random.default_rng(3)
    for x in _tied_rows(rng, 100, 23):
        for t in range(23):
            assert oracle.rank_of(x, t) == tiny.rank(list(x), t)
        order = oracle.rank_order(x)
        assert [tiny.rank(list(x), int(t)) for t in order] == list(range(23))


# ------------------------------------------------ tiny greedy batch: closed form

def test_tiny_closed_form_from_planted_mismatches():
    w = synth.make("tiny")
    res = oracle.verify_greedy(w.logits, w.dtype, w.V, w.offsets, w.owner, w.drafts)
    assert w.planted.tolist().count(4) == 1
    expect_toks = []
    for i in range(w.B):
        m = int(w.planted[i])
        assert res["accepted_len"][i] == m
        r = int(w.offsets[i]) + m
        top = int(np.argmax(w.logits[r, : w.V]))
        assert res["next_token"][i] == top
        expect_toks += [int(np.argmax(w.logits[int(w.offsets[i]) + j, : w.V])) for j in range(m)] + [top]
    assert res["out_offsets"].tolist() == [0] + np.cumsum(w.planted + 1).tolist()
    assert res["out_tokens"].tolist() == expect_toks


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_first_mismatch_replacement_and_bonus(seed):
    """top_k = 1 makes every sample the arg-max, so acceptance is closed form."""
    w = synth.make("tiny", seed=seed)
    B = w.B
    ones = np.ones(B, dtype=np.float32)
    res = oracle.verify_sampled(w.logits, w.dtype, w.V, w.offsets, w.owner, w.drafts,
                                ones, np.ones(B, np.int32), ones, np.zeros(B, np.float32), 5, 0)
    for i in range(B):
        m = int(w.planted[i])
        assert res["accepted_len"][i] == m
        assert res["next_token"][i] == int(np.argmax(w.logits[int(w.offsets[i]) + m, : w.V]))


# ---------------------------------------------------------------- relaxed

def _tiny_batch(rng, B, K, V, ties=True):
    R = B * (K + 1)
    if ties:
        logits = rng.integers(-3, 4, size=(R, V)).astype(np.float32)
    else:
        logits = rng.standard_normal((R, V)).astype(np.float32)
    offsets = np.arange(0, R + 1, K + 1, dtype=np.int32)
    owner = np.repeat(np.arange(B, dtype=np.int32), K + 1)
    drafts = rng.integers(0, V, size=R - B).astype(np.int32)
    return logits, offsets, owner, drafts


def test_relaxed_acceptance_brute_force():
    rng = np.random.default_rng(4)
    for Kr in (1, 2, 3, 5):
        logits, off, own, d = _tiny_batch(rng, 6, 3, 9)
        res = oracle.verify_greedy(logits, oracle.F32, 9, off, own, d, relaxed_topk=Kr)
        for i in range(6):
            a = 0
            while a < 3:
                xs = [float(v) for v in logits[4 * i + a]]
                if tiny.rank(xs, int(d[3 * i + a])) >= Kr:
                    break
                a += 1
            assert res["accepted_len"][i] == a


def test_relaxed_k1_is_strict_and_kv_accepts_all():
    rng = np.random.default_rng(5)
    logits, off, own, d = _tiny_batch(rng, 8, 4, 6)
    strict = oracle.verify_greedy(logits, oracle.F32, 6, off, own, d)
    k1 = oracle.verify_greedy(logits, oracle.F32, 6, off, own, d, relaxed_topk=1)
    for key in ("accepted_len", "next_token", "out_offsets", "out_tokens"):
        assert np.array_equal(strict[key], k1[key])
    kv = oracle.verify_greedy(logits, oracle.F32, 6, off, own, d, relaxed_topk=6)
    assert kv["accepted_len"].tolist() == [4] * 8
    # accepted drafts themselves are emitted
    assert kv["out_tokens"].reshape(8, 5)[:, :4].ravel().tolist() == d.tolist()


def test_out_of_range_draft_is_a_mismatch():
    rng = np.random.default_rng(6)
    logits, off, own, d = _tiny_batch(rng, 2, 2, 5)
    d[:] = [5, 0, -1, 0]
    res = oracle.verify_greedy(logits, oracle.F32, 5, off, own, d, relaxed_topk=5)
    assert res["accepted_len"].tolist() == [0, 0]


# ---------------------------------------------------------------- T = 0

def test_temperature_zero_equals_greedy():
    w = synth.make("mixed", B=6, V=4096)
    B = w.B
    z = np.zeros(B, dtype=np.float32)
    s = oracle.verify_sampled(w.logits, w.dtype, w.V, w.offsets, w.owner, w.drafts,
                              z, w.top_k, w.top_p, w.min_p, w.seed, 0)
    g = oracle.verify_greedy(w.logits, w.dtype, w.V, w.offsets, w.owner, w.drafts)
    for key in ("accepted_len", "next_token", "out_offsets", "out_tokens", "row_token"):
        assert np.array_equal(s[key], g[key])
    assert np.allclose(s["row_lse"], g["row_lse"], rtol=0, atol=0)


def test_sampled_row_lse_is_logsumexp_of_x_over_t():
    # reading c12: a sampled row reports the log-sum-exp of x / T
    w = synth.make("ragged", B=5, V=2048)
    T = np.full(w.B, 0.5, dtype=np.float32)
    res = oracle.verify_sampled(w.logits, w.dtype, w.V, w.offsets, w.owner, w.drafts,
                                T, w.top_k, w.top_p, w.min_p, w.seed, 0)
    for r in range(w.R):
        x = oracle.row_f64(w.logits, w.dtype, r, w.V)
        assert res["row_lse"][r] == pytest.approx(scipy.special.logsumexp(x / 0.5), rel=1e-12)


def test_draw_is_the_first_cumulative_weight_strictly_above_u():
    # the inverse CDF worked by hand: equal logits 0, 0, 0, 0 (weights 1 each,
    # rank order 0, 1, 2, 3, total 4); u * 4 = 1 lies exactly on the first
    # cumulative boundary, so the draw is the second token; just below it, the
    # first; u * 4 = 3 gives the last token
    x = np.zeros(4)
    assert oracle.sample_from_u(x, 1.0, 0, 1.0, 0.0, 0.25) == 1
    assert oracle.sample_from_u(x, 1.0, 0, 1.0, 0.0, 0.25 - 2.0**-24) == 0
    assert oracle.sample_from_u(x, 1.0, 0, 1.0, 0.0, 0.75) == 3
    assert oracle.sample_from_u(x, 1.0, 0, 1.0, 0.0, 0.0) == 0


# ---------------------------------------------------------------- sampling law

def _token_intervals(x, params):
    """Exact {token: count of grid points u = n / 2^24 that select it}."""
    def tok(n):
        return oracle.sample_from_u(x, *params, n / GRID)
    pos = {int(t): k for k, t in enumerate(oracle.rank_order(x))}
    out = {}
    n = 0
    while n < GRID:
        t = tok(n)
        lo, hi = n, GRID - 1
        while lo < hi:               # last grid point still selecting t
            mid = (lo + hi + 1) // 2
            if pos[tok(mid)] <= pos[t]:
                lo = mid
            else:
                hi = mid - 1
        out[t] = lo - n + 1
        n = lo + 1
    return out


PARAMS = [
    (1.0, 0, 1.0, 0.0), (0.5, 0, 1.0, 0.0), (1.0, 3, 1.0, 0.0), (1.0, 0, 0.6, 0.0),
    (0.7, 0, 1.0, 0.3), (1.3, 4, 0.8, 0.1), (0.9, 2, 0.5, 0.05), (1.0, 0, 0.95, 0.0),
]


@pytest.mark.parametrize("params", PARAMS)
def test_sampling_law_matches_brute_force(params):
    rng = np.random.default_rng(hash(params) % 2**32)
    for _ in range(4):
        x = (rng.integers(-6, 7, size=7) * 0.5).astype(np.float64)
        counts = _token_intervals(x, params)
        law = tiny.filtered_law(list(x), *params)
        assert set(counts) <= set(law)
        for t, p in law.items():
            assert abs(counts.get(t, 0) / GRID - p) <= 2.0 / GRID, (t, p)


def test_unfiltered_law_is_softmax_and_topk_is_truncated_softmax():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(6) * 2
    for T in (1.0, 0.6):
        sm = scipy.special.softmax(x / T)
        counts = _token_intervals(x, (T, 0, 1.0, 0.0))
        for t in range(6):
            assert abs(counts.get(t, 0) / GRID - sm[t]) <= 2.0 / GRID
        top3 = np.argsort(-x)[:3]
        c3 = _token_intervals(x, (T, 3, 1.0, 0.0))
        for t in range(6):
            want = sm[t] / sm[top3].sum() if t in top3 else 0.0
            assert abs(c3.get(t, 0) / GRID - want) <= 2.0 / GRID


def test_filter_special_cases():
    rng = np.random.default_rng(9)
    for _ in range(50):
        x = rng.integers(-5, 6, size=11).astype(np.float64)
        g = int(np.argmax(x))
        u = rng.random()
        assert oracle.sample_from_u(x, 1.0, 1, 1.0, 0.0, u) == g          # top_k = 1
        assert oracle.sample_from_u(x, 1.0, 0, 1e-9, 0.0, u) == g         # top_p -> 0+
        assert x[oracle.sample_from_u(x, 1e-4, 0, 1.0, 0.0, u)] == x.max()  # T -> 0+: a max tie
        tok = oracle.sample_from_u(x, 1.0, 0, 1.0, 1.0, u)                # min_p = 1
        assert x[tok] == x.max()
        ties = np.flatnonzero(x == x.max())
        counts = _token_intervals(x, (1.0, 0, 1.0, 1.0))
        assert set(counts) == set(int(t) for t in ties)
        for t in ties:
            assert abs(counts[int(t)] / GRID - 1.0 / len(ties)) <= 2.0 / GRID
        S, _ = oracle.filtered_support(x, 0.8, 4, 0.7, 0.1)
        order = oracle.rank_order(x)
        assert np.array_equal(S, order[: len(S)]) and S[0] == g          # prefix, keeps arg-max


def _law_of_verify(rows, drafts, params):
    """Exact law of the oracle's (accepted length, next token) over u-grids."""
    K = len(drafts)
    V = rows[0].shape[0]
    logits = np.stack(rows).astype(np.float32)
    xs = [logits[j].astype(np.float64) for j in range(K + 1)]
    cells = []
    for x in xs:
        iv = _token_intervals(x, params)
        pos = {int(t): k for k, t in enumerate(oracle.rank_order(x))}
        # representative u for each token's interval, in grid order
        start, reps = 0, []
        for t in sorted(iv, key=lambda t: pos[t]):
            reps.append((start / GRID, iv[t] / GRID))
            start += iv[t]
        cells.append(reps)
    T, k, p, mp = params
    law = {}
    off = np.array([0, K + 1], dtype=np.int32)
    own = np.zeros(K + 1, dtype=np.int32)
    import itertools
    for combo in itertools.product(*cells):
        us = {(0, j): combo[j][0] for j in range(K + 1)}
        prob = math.prod(c[1] for c in combo)
        res = oracle.verify_sampled(logits, oracle.F32, V, off, own, np.asarray(drafts),
                                    [T], [k], [p], [mp], 0, 0, uniforms=us)
        key = (int(res["accepted_len"][0]), int(res["next_token"][0]))
        law[key] = law.get(key, 0.0) + prob
    return law


@pytest.mark.parametrize("params", [(1.0, 0, 1.0, 0.0), (0.8, 3, 0.9, 0.1), (1.2, 0, 0.7, 0.0)])
def test_point_mass_rejection_equals_prefix_matching(params):
    """The oracle's (a, next) law equals the textbook rejection sampler's."""
    rng = np.random.default_rng(10)
    V, K = 4, 2
    for _ in range(3):
        rows = [(rng.integers(-3, 4, size=V) * 0.7).astype(np.float32) for _ in range(K + 1)]
        drafts = [int(rng.integers(0, V)) for _ in range(K)]
        got = _law_of_verify(rows, drafts, params)
        want = tiny.rejection_law([list(r.astype(np.float64)) for r in rows], drafts, params)
        for key in set(got) | set(want):
            assert abs(got.get(key, 0.0) - want.get(key, 0.0)) <= 4 * (K + 1) / GRID, key


# ---------------------------------------------------------------- confidence

def test_draft_confidence_properties():
    rng = np.random.default_rng(12)
    y = (rng.standard_normal((3, 50)) * 3).astype(np.float32)
    conf, lse = oracle.draft_confidence(y, oracle.F32, 50)
    sm = scipy.special.softmax(y.astype(np.float64), axis=1)
    assert np.allclose(conf, sm.max(axis=1), rtol=1e-13)
    assert np.allclose(lse, scipy.special.logsumexp(y.astype(np.float64), axis=1), rtol=1e-13)
    for q in range(3):
        allc = [oracle.draft_confidence(y[q:q + 1], oracle.F32, 50, [t])[0][0] for t in range(50)]
        assert math.fsum(allc) == pytest.approx(1.0, abs=1e-12)
        assert all(0.0 < c <= 1.0 for c in allc)
    c, _ = oracle.draft_confidence(y[:1], oracle.F32, 50, [50])
    assert c[0] == 0.0


def test_bf16_widening_is_exact():
    f = np.array([1.0, -2.5, 3.140625, -0.0, 65280.0], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(f)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), f.astype(np.float64))
    # round to nearest even at the halfway point
    half = np.array([1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8], dtype=np.float32)
    assert oracle.bf16_bits_to_f64(synth.f32_to_bf16_bits(half)).tolist() == [1.0, 1.0 + 2.0**-6]


# ---------------------------------------------------------------- preconditions

def test_layout_preconditions_raise():
    logits = np.zeros((4, 3), dtype=np.float32)
    d = np.zeros(2, dtype=np.int32)
    with pytest.raises(oracle.PreconditionError):
        oracle.verify_greedy(logits, oracle.F32, 3, [0, 2, 3], None, d)      # ends short of R
    with pytest.raises(oracle.PreconditionError):
        oracle.verify_greedy(logits, oracle.F32, 3, [0, 2, 2, 4], None, np.zeros(1))
    with pytest.raises(oracle.PreconditionError):
        oracle.verify_greedy(logits, oracle.F32, 3, [0, 2, 4], [0, 1, 1, 1], d)
    bad = logits.copy()
    bad[1, 1] = np.nan
    with pytest.raises(oracle.PreconditionError):
        oracle.verify_greedy(bad, oracle.F32, 3, [0, 2, 4], None, d)


def test_margins_are_consistent_with_decisions():
    rng = np.random.default_rng(14)
    x = rng.standard_normal(3000) * 2.5
    for params in [(0.5, 50, 0.9, 0.05), (0.7, 0, 0.95, 0.0)]:
        u = 0.3
        tp, um, mp = oracle.sampled_row_margins(x, *params, u)
        assert tp >= 0 and um >= 0 and mp >= 0
        # moving u by less than its margin keeps the token
        t0 = oracle.sample_from_u(x, *params, u)
        assert oracle.sample_from_u(x, *params, u + 0.5 * um) == t0
        assert oracle.sample_from_u(x, *params, u - 0.5 * um) == t0


def _survivors(x, T, k, p, mp):
    return oracle.filtered_support(x, T, k, p, mp)[0].tolist()


def test_topp_margin_is_the_distance_to_the_nearest_cut():
    """Moving top_p by half its margin keeps the survivor set; moving it just
    past the margin, toward the boundary the margin measures, changes it."""
    rng = np.random.default_rng(140)
    checked = 0
    for trial in range(60):
        V = int(rng.integers(8, 200))
        x = rng.standard_normal(V) * float(rng.choice([1.0, 2.5, 4.0]))
        T = float(rng.choice([0.5, 0.7, 1.0, 1.6]))
        k = int(rng.choice([0, 5, 20]))
        p = float(rng.uniform(0.05, 0.98))
        tp, _, _ = oracle.sampled_row_margins(x, T, k, p, 0.0, 0.5)
        assert 0 <= tp < 1
        S = _survivors(x, T, k, p, 0.0)
        assert _survivors(x, T, k, p + 0.5 * tp, 0.0) == S
        assert _survivors(x, T, k, p - 0.5 * tp, 0.0) == S
        moved = [_survivors(x, T, k, q, 0.0) for q in (p + tp + 1e-9, p - tp - 1e-9) if 0 < q < 1]
        if not any(m != S for m in moved):
            # the cut is at the last top-k token: the nearest boundary is the
            # whole mass, which top_p cannot pass (top_p >= 1 is "off")
            assert p + tp == pytest.approx(1.0, abs=1e-12), (trial, p, tp)
            continue
        checked += 1
    assert checked > 40


def test_minp_margin_is_the_distance_to_the_nearest_z():
    """Moving ln(min_p) by half its margin keeps the survivor set; moving it
    just past the margin, toward the z the margin measures, changes it."""
    rng = np.random.default_rng(141)
    for trial in range(60):
        V = int(rng.integers(8, 200))
        x = rng.standard_normal(V) * 2.5
        T = float(rng.choice([0.5, 1.0, 1.5]))
        k = int(rng.choice([0, 30]))
        p = float(rng.choice([1.0, 0.95]))
        mp = float(rng.uniform(0.01, 0.6))
        _, _, mm = oracle.sampled_row_margins(x, T, k, p, mp, 0.5)
        S = _survivors(x, T, k, p, mp)
        if not np.isfinite(mm):
            # only the maximum's ties are top-p survivors: min-p cannot cut
            assert len(set(x[S].tolist())) == 1
            continue
        lm = math.log(mp)
        for s_ in (0.5, -0.5):
            if lm + s_ * mm <= 0.0:       # min_p above 1 is out of range
                assert _survivors(x, T, k, p, math.exp(lm + s_ * mm)) == S
        moved = [_survivors(x, T, k, p, math.exp(lm + s * (mm + 1e-9))) for s in (1, -1)
                 if math.exp(lm + s * (mm + 1e-9)) <= 1.0]
        assert any(m != S for m in moved), (trial, mp, mm)


def test_margins_for_top_k_then_top_p_then_min_p():
    """All three margins on one row where every filter cuts: each is the
    distance the pins above define, taken after the filters before it."""
    x = np.array([3.0, 2.0, 2.0, 1.0, 0.5, 0.0, -1.0, -3.0])
    T, k, p, mp = 1.0, 6, 0.8, 0.3
    tp, um, mm = oracle.sampled_row_margins(x, T, k, p, mp, 0.25)
    w = np.exp(x - 3.0)
    c = np.cumsum(w[:6]) / np.sum(w[:6])         # ranks 0..5 after top-k
    L = int(np.flatnonzero(c >= p)[0])
    assert tp == pytest.approx(min(c[L] - p, p - c[L - 1]), rel=1e-12)
    zs = (x[:L + 1] - 3.0)[1:]                    # top-p survivors below the max
    assert mm == pytest.approx(float(np.min(np.abs(zs - math.log(mp)))), rel=1e-12)
    S = [t for t in range(L + 1) if x[t] - 3.0 >= math.log(mp)]
    cs = np.cumsum(w[S]) / np.sum(w[S])
    n = int(np.flatnonzero(cs > 0.25)[0])
    assert um == pytest.approx(min(cs[n] - 0.25, 0.25 - cs[n - 1]) if n else cs[n] - 0.25, rel=1e-12)


# ---------------------------------------------------------------------------
# Relaxed acceptance variants (margin, position and token gates, protected
# ids): what the reading fixes, stated independently of the oracle's code.


def _tiny_accept_set(xs, margin, protected=()):
    """Drafts accepted at an ungated position, by plain enumeration: the
    lowest index of the maximum, and every other token whose value lies
    strictly less than `margin` below the maximum, unless it or the greedy
    token is protected."""
    m = max(xs)
    g = min(t for t in range(len(xs)) if xs[t] == m)
    out = {g}
    if g in protected:
        return out
    for t in range(len(xs)):
        if t not in protected and margin > 0 and (m - xs[t]) < margin:
            out.add(t)
    return out


def test_relaxed_defaults_are_strict():
    for key, kw in (("tiny", {}), ("relaxed", dict(B=6, V=700))):
        wl = synth.make(key, **kw)
        a = oracle.verify_greedy(wl.logits, wl.dtype, wl.V, wl.offsets, wl.owner, wl.drafts)
        b = oracle.verify_greedy_relaxed(wl.logits, wl.dtype, wl.V, wl.offsets, wl.owner, wl.drafts)
        for k in a:
            assert np.array_equal(a[k], b[k]), k


def test_relaxed_topk_alone_is_top_k_acceptance():
    wl = synth.make("relaxed", B=8, V=900)
    for K in (2, 4, 9):
        a = oracle.verify_greedy(wl.logits, wl.dtype, wl.V, wl.offsets, wl.owner, wl.drafts, relaxed_topk=K)
        b = oracle.verify_greedy_relaxed(wl.logits, wl.dtype, wl.V, wl.offsets, wl.owner, wl.drafts, topk=K)
        for k in a:
            assert np.array_equal(a[k], b[k]), (K, k)


def test_margin_worked_row():
    # maximum 3.0 at tokens 1 and 3 (the lowest index, 1, is greedy); token 2
    # lies 0.5 below it, token 0 2.0 below
    x = np.array([1.0, 3.0, 2.5, 3.0])
    acc = lambda m: {d for d in range(4) if oracle.relaxed_accepts(x, 0, 0, d, margin=m)}
    assert acc(0.0) == {1}
    assert acc(0.5) == {1, 3}               # 0.5 below is not strictly within 0.5
    assert acc(0.500001) == {1, 2, 3}
    assert acc(2.0) == {1, 2, 3}
    assert acc(2.000001) == {0, 1, 2, 3}
    assert {d for d in range(4) if oracle.relaxed_accepts(x, 0, 0, d, margin=5.25, protected={3})} == {0, 1, 2}
    assert {d for d in range(4) if oracle.relaxed_accepts(x, 0, 0, d, margin=5.25, protected={1})} == {1}
    assert not oracle.relaxed_accepts(x, 0, 0, 4, margin=100.0)   # out of range


def test_margin_brute_force_tiny_vocab():
    rng = np.random.default_rng(150)
    for trial in range(300):
        V = int(rng.integers(1, 12))
        xs = [float(v) for v in rng.integers(-6, 7, size=V) * 0.5]
        margin = float(rng.choice([0.0, 0.25, 0.5, 1.0, 1.75, 5.25]))
        prot = set(int(t) for t in rng.choice(V, size=int(rng.integers(0, 3)), replace=True)) if V else set()
        x = np.array(xs)
        got = {d for d in range(V) if oracle.relaxed_accepts(x, 3, 10, d, margin=margin, protected=prot)}
        assert got == _tiny_accept_set(xs, margin, prot), (xs, margin, prot)


def test_margin_huge_accepts_every_draft_like_top_v():
    wl = synth.make("relaxed", B=5, V=333)
    a = oracle.verify_greedy(wl.logits, wl.dtype, wl.V, wl.offsets, wl.owner, wl.drafts, relaxed_topk=wl.V)
    b = oracle.verify_greedy_relaxed(wl.logits, wl.dtype, wl.V, wl.offsets, wl.owner, wl.drafts, margin=1e30)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    assert np.array_equal(b["accepted_len"], np.diff(wl.offsets) - 1)


def test_relaxed_gates_and_protection_on_a_request():
    """One request of four drafts: drafts 0 and 1 are the greedy tokens,
    drafts 2 and 3 are other tokens within the margin. Where relaxation is
    allowed only from position p (or from output token N), the accepted
    length is the first gated-off position of a non-greedy draft."""
    V = 10
    rows = np.zeros((5, V), dtype=np.float32)
    for j in range(5):
        rows[j] = np.arange(V, dtype=np.float32) * 0.1
        rows[j, j] = 5.0                     # greedy token of row j is j
        rows[j, 9] = 4.5                     # 0.5 below the maximum
    drafts = np.array([0, 1, 9, 9], dtype=np.int32)
    off, own = np.array([0, 5]), np.zeros(5, dtype=np.int32)
    run = lambda **kw: oracle.verify_greedy_relaxed(rows, oracle.F32, V, off, own, drafts, **kw)
    assert run()["accepted_len"][0] == 2                         # strict
    assert run(margin=1.0)["accepted_len"][0] == 4
    assert run(margin=1.0)["next_token"][0] == 4                 # bonus = greedy token of the last row
    assert list(run(margin=1.0)["out_tokens"]) == [0, 1, 9, 9, 4]
    assert run(margin=1.0, from_position=2)["accepted_len"][0] == 4
    assert run(margin=1.0, from_position=3)["accepted_len"][0] == 2
    assert run(margin=1.0, after_tokens=5, generated=[3])["accepted_len"][0] == 4   # 3 + 2 >= 5
    assert run(margin=1.0, after_tokens=5, generated=[2])["accepted_len"][0] == 2   # 2 + 2 < 5
    assert run(margin=1.0, protected=[9])["accepted_len"][0] == 2
    assert run(margin=1.0, protected=[2])["accepted_len"][0] == 2   # greedy token of row 2 protected
    assert run(margin=1.0, protected=[3])["accepted_len"][0] == 3   # ... of row 3
    assert run(margin=0.4)["accepted_len"][0] == 2
    assert run(topk=2)["accepted_len"][0] == 4                   # token 9 ranks second
    assert run(topk=2, after_tokens=4, generated=[1])["accepted_len"][0] == 2   # 1 + 2 < 4
    assert run(topk=2, after_tokens=4, generated=[2])["accepted_len"][0] == 4   # 2 + 2 >= 4
