"""Goodput step selection: CPU oracle (test infrastructure only).

Only tests/ call this module; the library never does, and nothing here
comes from it.

What the pages fix (xLLM docs, "Adaptive speculative inference", section
"Adaptive draft step (MTP)", with its table of policy options):

* before a decode batch is submitted, one step count is chosen for the whole
  batch, the one that maximises B * (1 + sum(prefix_acceptance[:s])) /
  cost_ms(s), from the per-position prefix acceptance of completed
  verification results and the full-round cost of each candidate step count;
* num_speculative_tokens is the largest step count;
* policy.window_size (default 20): completed batches counted in the
  per-position prefix acceptance;
* policy.update_interval (default 5): the candidates are re-scored every this
  many completed batches;
* policy.switch_min_gain (default 0.05): the step count changes only when the
  predicted relative throughput gain is strictly above it.

Readings taken where the page gives no rule (each listed in the design
notes):

* the candidates are 1 .. S, S = num_speculative_tokens, and the controller
  starts at S;
* prefix_acceptance[j] is the share, among the window's requests that
  verified at least j + 1 drafts, of those whose accepted length is at least
  j + 1; a position that no request in the window verified keeps its last
  estimate (0 before any), since a step count below j + 1 produces no data
  for it;
* the estimate is refreshed after every observed batch, the candidates are
  re-scored when update_interval batches have been observed since the last
  re-scoring, and equal scores go to the smaller step count.

Parity-pinned by tests/test_oracle_goodput.py: closed forms for constant
and geometric acceptance with affine costs, the strict switching margin, the
window's expiry, and brute force over small histories.
"""
import numpy as np


def batch_counts(accepted_len, verify_len, S):
    """Per-position counts of one batch: (reached[j], accepted[j]), j < S."""
    a = np.asarray(accepted_len, dtype=np.int64)
    k = np.asarray(verify_len, dtype=np.int64)
    if a.shape != k.shape or (k < 0).any() or (a < 0).any() or (a > k).any():
        raise ValueError("need 0 <= accepted_len <= verify_len")
    reached = np.array([int((k > j).sum()) for j in range(S)], dtype=np.int64)
    accepted = np.array([int((a > j).sum()) for j in range(S)], dtype=np.int64)
    return reached, accepted


def score(prefix_acc, cost_ms, s, B):
    """B * (1 + sum of the first s prefix acceptances) / cost of s steps."""
    total = 1.0
    for j in range(s):
        total += float(prefix_acc[j])
    return B * total / float(cost_ms[s - 1])


def select(prefix_acc, cost_ms, B, current, min_gain):
    """Best step count, kept at `current` unless the gain is above min_gain."""
    S = len(cost_ms)
    best, best_score = 1, score(prefix_acc, cost_ms, 1, B)
    for s in range(2, S + 1):
        v = score(prefix_acc, cost_ms, s, B)
        if v > best_score:
            best, best_score = s, v
    if best != current and best_score > (1.0 + min_gain) * score(prefix_acc, cost_ms, current, B):
        return best
    return current


class GoodputController:
    """Window of completed batches, estimates and the current step count."""

    def __init__(self, max_steps, window_size=20, update_interval=5, switch_min_gain=0.05):
        self.S = int(max_steps)
        self.window = int(window_size)
        self.interval = int(update_interval)
        self.min_gain = float(switch_min_gain)
        self.batches = []              # (reached, accepted) per completed batch
        self.estimate = np.zeros(self.S)
        self.current = self.S
        self.since = 0

    def observe(self, accepted_len, verify_len):
        self.batches.append(batch_counts(accepted_len, verify_len, self.S))
        self.batches = self.batches[-self.window:]
        reached = sum(b[0] for b in self.batches)
        accepted = sum(b[1] for b in self.batches)
        for j in range(self.S):
            if reached[j] > 0:
                self.estimate[j] = float(accepted[j]) / float(reached[j])
        self.since += 1

    def step(self, cost_ms, B):
        if self.since >= self.interval:
            self.current = select(self.estimate, cost_ms, B, self.current, self.min_gain)
            self.since = 0
        return self.current
