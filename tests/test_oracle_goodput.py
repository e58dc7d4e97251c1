"""Pins of the goodput step-selection oracle (CPU only).

Closed forms for constant and geometric acceptance with affine costs, the
strict switching margin, the window's expiry and estimate persistence, and
brute force over small histories."""

import numpy as np
import pytest

from oracle.goodput import GoodputController, batch_counts, score, select


def test_batch_counts_by_hand():
    # requests verified 3, 3, 1, 0 drafts and accepted 2, 3, 1, 0 of them
    reached, accepted = batch_counts([2, 3, 1, 0], [3, 3, 1, 0], 4)
    assert list(reached) == [3, 2, 2, 0]
    assert list(accepted) == [3, 2, 1, 0]
    with pytest.raises(ValueError):
        batch_counts([2], [1], 3)


@pytest.mark.parametrize("alpha", [0.0, 0.3, 0.6, 0.9, 1.0])
@pytest.mark.parametrize("c0,c1", [(10.0, 1.0), (2.0, 1.0), (1.0, 3.0)])
def test_geometric_acceptance_with_affine_cost(alpha, c0, c1):
    # prefix acceptance alpha^(j+1), cost c0 + c1 * s: the score is
    # B (1 + alpha (1 - alpha^s) / (1 - alpha)) / (c0 + c1 s), the geometric
    # series summed in closed form rather than term by term
    S = 8
    pa = np.array([alpha ** (j + 1) for j in range(S)])
    cost = np.array([c0 + c1 * s for s in range(1, S + 1)])

    def closed(s):
        g = s if alpha == 1.0 else (alpha * (1 - alpha ** s) / (1 - alpha) if alpha != 0.0 else 0.0)
        return 16 * (1 + g) / (c0 + c1 * s)

    want = max(range(1, S + 1), key=lambda s: (closed(s), -s))
    for s in range(1, S + 1):
        assert score(pa, cost, s, 16) == pytest.approx(closed(s), rel=1e-12)
    assert select(pa, cost, 16, want, 0.0) == want
    # from any other step with no margin, the best is taken unless tied
    for cur in range(1, S + 1):
        got = select(pa, cost, 16, cur, 0.0)
        assert got == cur if closed(cur) >= closed(want) else got == want


def test_zero_acceptance_picks_the_cheapest_step():
    cost = np.array([3.0, 2.0, 2.5, 4.0])
    assert select(np.zeros(4), cost, 8, 4, 0.0) == 2


def test_full_acceptance_with_flat_cost_picks_the_longest():
    assert select(np.ones(6), np.full(6, 5.0), 8, 1, 0.05) == 6


def test_switch_needs_strictly_more_than_the_margin():
    # from s = 1 (score B * (1 + p0) / c1) to s = 2 (score B * (1 + p0 + p1) / c2)
    cost = np.array([1.0, 1.0])
    assert select(np.array([0.0, 0.06]), cost, 4, 1, 0.05) == 2     # 6 % gain: switch
    assert select(np.array([0.0, 0.05]), cost, 4, 1, 0.05) == 1     # exactly 5 %: stay
    assert select(np.array([0.0, 0.04]), cost, 4, 1, 0.05) == 1     # 4 %: stay
    assert select(np.array([1.0, 0.05]), cost, 4, 1, 0.05) == 1     # 2.5 %: stay
    assert select(np.array([0.0, 0.04]), cost, 4, 1, 0.0) == 2      # no margin: any gain


def test_ties_go_to_the_smaller_step():
    assert select(np.array([0.0, 0.0, 0.0]), np.array([2.0, 2.0, 2.0]), 4, 3, 0.0) == 3
    assert select(np.array([0.0, 0.0, 0.0]), np.array([2.0, 2.0, 2.0]), 4, 3, -0.5) == 1


def test_window_expires_old_batches_and_keeps_unreached_estimates():
    g = GoodputController(4, window_size=3, update_interval=1, switch_min_gain=0.0)
    for _ in range(3):
        g.observe([4, 4], [4, 4])                 # everything accepted
    assert list(g.estimate) == [1.0, 1.0, 1.0, 1.0]
    for _ in range(3):
        g.observe([0, 1], [2, 2])                 # only positions 0, 1 verified
    # the window now holds only the last three batches: positions 2, 3 keep 1.0
    assert list(g.estimate) == [0.5, 0.0, 1.0, 1.0]


def test_rescoring_every_update_interval():
    g = GoodputController(3, window_size=20, update_interval=5, switch_min_gain=0.0)
    cost = np.array([1.0, 10.0, 10.0])            # one step is far cheaper
    for b in range(12):
        g.observe([0], [3])
        s = g.step(cost, 1)
        assert s == (3 if b < 4 else 1), b       # the first re-scoring follows the 5th batch


def _brute_force(history, costs, B, S, W, I, m):
    """Re-derive every step decision from the raw history."""
    cur, since, est, out = S, 0, [0.0] * S, []
    for t, (a, k) in enumerate(history):
        lo = max(0, t + 1 - W)
        for j in range(S):
            reach = sum(1 for u in range(lo, t + 1) for x in history[u][1] if x > j)
            acc = sum(1 for u in range(lo, t + 1) for x in history[u][0] if x > j)
            if reach:
                est[j] = acc / reach
        since += 1
        if since >= I:
            sc = [B * (1 + sum(est[:s])) / costs[s - 1] for s in range(1, S + 1)]
            best = max(range(1, S + 1), key=lambda s: (sc[s - 1], -s))
            if best != cur and sc[best - 1] > (1 + m) * sc[cur - 1]:
                cur = best
            since = 0
        out.append(cur)
    return out


@pytest.mark.parametrize("seed", range(6))
def test_controller_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    S, W, I, m, B = 4, int(rng.integers(2, 6)), int(rng.integers(1, 4)), 0.05, 6
    costs = np.sort(rng.uniform(1.0, 4.0, S))
    history = []
    for _ in range(25):
        k = rng.integers(0, S + 1, B)
        a = np.array([rng.integers(0, x + 1) for x in k])
        history.append((a, k))
    g = GoodputController(S, W, I, m)
    got = []
    for a, k in history:
        g.observe(a, k)
        got.append(g.step(costs, B))
    assert got == _brute_force(history, costs, B, S, W, I, m)
