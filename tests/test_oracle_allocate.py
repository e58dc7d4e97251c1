"""Pins of the adaptive verify-allocation oracle (CPU only).

The allocation is checked against brute force over every allocation of tiny
batches, closed forms for equal and unit scores, its nesting in the budget,
and its packed layout against the verification oracle itself.
"""
import itertools

import numpy as np
import pytest

import oracle
from oracle.allocate import allocate_verify, clamp_scores, prefix_scores


def _expected_accepts(P, k):
    """Expected accepted drafts of an allocation: sum of the chosen products."""
    return sum(float(P[i, j]) for i in range(P.shape[0]) for j in range(int(k[i])))


@pytest.mark.parametrize("seed", range(12))
def test_allocation_is_optimal_by_brute_force(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 4))
    K = int(rng.integers(1, 4))
    conf = rng.uniform(0.0, 1.0, size=B * K).astype(np.float32)
    if seed % 3 == 0:
        conf[rng.integers(0, B * K)] = 1.0   # equal products across positions
    drafts = rng.integers(0, 100, size=B * K)
    P = prefix_scores(conf, B, K)
    for G in range(B, B * (K + 1) + 1):
        res = allocate_verify(conf, drafts, B, K, G)
        k = res["verify_len"]
        assert int(k.sum()) == G - B and (k >= 0).all() and (k <= K).all()
        best = max(_expected_accepts(P, ks)
                   for ks in itertools.product(range(K + 1), repeat=B) if sum(ks) == G - B)
        assert _expected_accepts(P, k) == pytest.approx(best, rel=0, abs=1e-12)


def test_products_are_float32_left_to_right():
    rng = np.random.default_rng(3)
    c = rng.uniform(0.05, 1.0, size=(5, 7)).astype(np.float32)
    P = prefix_scores(c.ravel(), 5, 7)
    assert P.dtype == np.float32
    assert np.array_equal(P, np.cumprod(c, axis=1, dtype=np.float32))


def test_equal_scores_fill_position_by_position():
    B, K = 5, 4
    conf = np.full(B * K, 0.7, dtype=np.float32)
    for G in range(B, B * (K + 1) + 1):
        M = G - B
        k = allocate_verify(conf, np.zeros(B * K), B, K, G)["verify_len"]
        want = [M // B + (1 if i < M % B else 0) for i in range(B)]
        assert list(k) == want, (G, list(k))


def test_unit_scores_fill_requests_in_order():
    B, K = 4, 3
    conf = np.ones(B * K, dtype=np.float32)
    for G in range(B, B * (K + 1) + 1):
        M = G - B
        k = allocate_verify(conf, np.zeros(B * K), B, K, G)["verify_len"]
        assert list(k) == [min(K, max(0, M - i * K)) for i in range(B)], G


def test_budget_extremes_and_bounds():
    rng = np.random.default_rng(5)
    B, K = 6, 5
    conf = rng.uniform(size=B * K)
    assert (allocate_verify(conf, np.zeros(B * K), B, K, B)["verify_len"] == 0).all()
    assert (allocate_verify(conf, np.zeros(B * K), B, K, B * (K + 1))["verify_len"] == K).all()
    for G in (B - 1, B * (K + 1) + 1):
        with pytest.raises(ValueError):
            allocate_verify(conf, np.zeros(B * K), B, K, G)


def test_allocations_nest_as_the_budget_grows():
    rng = np.random.default_rng(11)
    B, K = 7, 5
    conf = rng.uniform(0.2, 1.0, size=B * K).astype(np.float32)
    prev = allocate_verify(conf, np.zeros(B * K), B, K, B)["verify_len"]
    for G in range(B + 1, B * (K + 1) + 1):
        k = allocate_verify(conf, np.zeros(B * K), B, K, G)["verify_len"]
        d = k - prev
        assert (d >= 0).all() and int(d.sum()) == 1
        prev = k


def test_zero_score_gets_rows_only_after_every_positive_one():
    B, K = 3, 2
    conf = np.array([0.0, 0.9, 0.5, 0.5, 0.8, 0.8], dtype=np.float32)
    # positive products: (1,0)=.5 (1,1)=.25 (2,0)=.8 (2,1)=.64; zeros: (0,0), (0,1)
    k = [list(allocate_verify(conf, np.zeros(6), B, K, B + M)["verify_len"]) for M in range(7)]
    assert k == [[0, 0, 0], [0, 0, 1], [0, 0, 2], [0, 1, 2], [0, 2, 2], [1, 2, 2], [2, 2, 2]]


def test_scores_are_clamped_before_the_products():
    raw = np.array([1.5, 0.5, np.nan, 0.9, -0.2, 0.7], dtype=np.float32)
    assert list(clamp_scores(raw)) == [1.0, 0.5, 0.0, np.float32(0.9), 0.0, np.float32(0.7)]
    for G in range(3, 10):
        a = allocate_verify(raw, np.arange(6), 3, 2, G)
        b = allocate_verify(clamp_scores(raw), np.arange(6), 3, 2, G)
        assert np.array_equal(a["verify_len"], b["verify_len"])


@pytest.mark.parametrize("seed", range(4))
def test_packed_layout_verifies_like_each_truncated_request(seed):
    # the packed batch, fed to the verification oracle, gives every request
    # the result of verifying its first k_i drafts on its own
    rng = np.random.default_rng(100 + seed)
    B, K, V = 5, 4, 64
    x = rng.normal(0.0, 2.0, size=(B * (K + 1), V)).astype(np.float32)
    am = x.argmax(axis=1)
    drafts = np.array([am[i * (K + 1) + j] if rng.uniform() < 0.7 else (am[i * (K + 1) + j] + 1) % V
                       for i in range(B) for j in range(K)], dtype=np.int32)
    conf = rng.uniform(0.3, 1.0, size=B * K).astype(np.float32)
    G = int(rng.integers(B, B * (K + 1) + 1))
    res = allocate_verify(conf, drafts, B, K, G)
    got = oracle.verify_greedy(x[res["row_source"]], oracle.F32, V, res["row_offsets"],
                               res["row_owner"], res["packed_drafts"])
    for i in range(B):
        k = int(res["verify_len"][i])
        rows = x[i * (K + 1): i * (K + 1) + k + 1]
        one = oracle.verify_greedy(rows, oracle.F32, V, np.array([0, k + 1]), np.zeros(k + 1, dtype=np.int32),
                                   drafts[i * K: i * K + k])
        assert got["accepted_len"][i] == one["accepted_len"][0]
        assert got["next_token"][i] == one["next_token"][0]
