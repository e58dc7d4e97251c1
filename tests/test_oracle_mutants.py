"""Mutation check of the oracle's pins (CPU only).

Each mutant plants one plausible mistake in a copy of `oracle/` (a dropped
term, a wrong tie rule or boundary, an off-by-one index, a swapped filter
order, a wrong Philox constant). The pin suite of the mutated module
(`test_oracle_pins.py`, `test_oracle_allocate.py` for the verify
allocation, `test_oracle_goodput.py` for goodput step selection,
`test_oracle_probabilistic.py` for probabilistic drafts) then runs against the mutant in a subprocess and must fail: a
mistake that no pin catches would also slip past parity, since parity
compares the HIP path with this oracle.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")
PINS_BY_FILE = {"allocate.py": os.path.join(ROOT, "tests", "test_oracle_allocate.py"),
                "goodput.py": os.path.join(ROOT, "tests", "test_oracle_goodput.py"),
                "probabilistic.py": os.path.join(ROOT, "tests", "test_oracle_probabilistic.py")}

# (name, file, original text, mutated text); the original must occur once.
MUTANTS = [
    ("argmax_last_tie", "verify.py",
     "return int(np.flatnonzero(x == m)[0])",
     "return int(np.flatnonzero(x == m)[-1])"),
    ("lse_drops_max", "verify.py",
     "return float(m / temperature + math.log(np.sum(np.exp(z))))",
     "return float(math.log(np.sum(np.exp(z))))"),
    ("rank_ties_after", "verify.py",
     "np.count_nonzero(x[:t] == v)",
     "np.count_nonzero(x[t + 1:] == v)"),
    ("rank_order_index_desc", "verify.py",
     "np.lexsort((np.arange(x.shape[0]), -x))",
     "np.lexsort((-np.arange(x.shape[0]), -x))"),
    ("topk_keeps_one_more", "verify.py",
     "        S = S[:top_k]\n    if top_p < 1.0:\n        c = np.cumsum(w[S])\n        W = c[-1]",
     "        S = S[:top_k + 1]\n    if top_p < 1.0:\n        c = np.cumsum(w[S])\n        W = c[-1]"),
    ("topp_drops_crossing_token", "verify.py",
     "L = int(np.flatnonzero(c >= top_p * W)[0]) + 1",
     "L = max(1, int(np.flatnonzero(c >= top_p * W)[0]))"),
    ("minp_strict", "verify.py",
     "keep = z[S] >= math.log(min_p)",
     "keep = z[S] > math.log(min_p)"),
    ("temperature_multiplies", "verify.py",
     "    z = (x - m) / temperature\n    w = np.exp(z)\n    order = rank_order(x)",
     "    z = (x - m) * temperature\n    w = np.exp(z)\n    order = rank_order(x)"),
    ("filters_topp_before_topk", "verify.py",
     "    if 0 < top_k < V:\n        S = S[:top_k]\n    if top_p < 1.0:\n        c = np.cumsum(w[S])\n"
     "        W = c[-1]\n        L = int(np.flatnonzero(c >= top_p * W)[0]) + 1\n        S = S[:L]\n",
     "    if top_p < 1.0:\n        c = np.cumsum(w[S])\n        W = c[-1]\n"
     "        L = int(np.flatnonzero(c >= top_p * W)[0]) + 1\n        S = S[:L]\n"
     "    if 0 < top_k < V:\n        S = S[:top_k]\n"),
    ("draw_boundary_inclusive", "verify.py",
     "n = int(np.flatnonzero(c > u * c[-1])[0])\n    return int(S[n])",
     "n = int(np.flatnonzero(c >= u * c[-1])[0])\n    return int(S[n])"),
    ("accepts_not_prefix", "verify.py",
     "    a = 0\n    while a < len(accepts) and accepts[a]:\n        a += 1\n",
     "    a = int(sum(bool(v) for v in accepts))\n"),
    ("next_token_from_last_row", "verify.py",
     "nxt = int(tokens[a])",
     "nxt = int(tokens[-1])"),
    ("offsets_miss_next_token", "verify.py",
     "out_off[i + 1] = out_off[i] + a + 1",
     "out_off[i + 1] = out_off[i] + a"),
    ("relaxed_rank_inclusive", "verify.py",
     "accepts.append(rank_of(x, t) < relaxed_topk)",
     "accepts.append(rank_of(x, t) <= relaxed_topk)"),
    ("greedy_drafts_shifted", "verify.py",
     "        d = drafts[r0 - i : r0 - i + K]\n        accepts = []\n        for j in range(K + 1):\n"
     "            x = row_f64(logits, dtype, r0 + j, vocab)\n            check_row(x)\n            row_token[r0 + j] = greedy_token(x)",
     "        d = drafts[r0 - i + 1 : r0 - i + K + 1]\n        accepts = []\n        for j in range(K + 1):\n"
     "            x = row_f64(logits, dtype, r0 + j, vocab)\n            check_row(x)\n            row_token[r0 + j] = greedy_token(x)"),
    ("sampled_lse_ignores_temperature", "verify.py",
     "row_lse[r0 + j] = logsumexp(x, T[i])",
     "row_lse[r0 + j] = logsumexp(x)"),
    ("confidence_against_max", "verify.py",
     "conf[q] = math.exp(y[s] - lse[q])",
     "conf[q] = math.exp(y[s] - np.max(y))"),
    ("philox_multiplier", "philox.py",
     "PHILOX_M0 = 0xD2511F53",
     "PHILOX_M0 = 0xD2511F55"),
    ("philox_weyl_key", "philox.py",
     "PHILOX_W1 = 0xBB67AE85",
     "PHILOX_W1 = 0xBB67AE87"),
    ("uniform_drops_a_bit", "philox.py",
     "return (w[0] >> 8) * (1.0 / 16777216.0)",
     "return (w[0] >> 9) * (1.0 / 16777216.0)"),
    ("allocation_scores_not_products", "allocate.py",
     "run = np.float32(run * c[i, j])",
     "run = np.float32(c[i, j])"),
    ("allocation_ties_request_desc", "allocate.py",
     "np.lexsort((jj.ravel(), ii.ravel(), -P.ravel().astype(np.float64)))",
     "np.lexsort((jj.ravel(), -ii.ravel(), -P.ravel().astype(np.float64)))"),
    ("allocation_budget_without_bonus_rows", "allocate.py",
     "    M = G - B\n",
     "    M = G - B + 1\n"),
    ("allocation_drafts_shifted", "allocate.py",
     "packed[off[i] - i + j] = d[i, j]",
     "packed[off[i] - i + j] = d[i, min(j + 1, K - 1)]"),
    ("allocation_source_stride", "allocate.py",
     "source[off[i] + j] = i * (K + 1) + j",
     "source[off[i] + j] = i * K + j"),
    ("goodput_margin_inclusive", "goodput.py",
     "best_score > (1.0 + min_gain) * score(",
     "best_score >= (1.0 + min_gain) * score("),
    ("goodput_ties_to_larger_step", "goodput.py",
     "        if v > best_score:\n",
     "        if v >= best_score:\n"),
    ("goodput_score_without_one", "goodput.py",
     "    total = 1.0\n",
     "    total = 0.0\n"),
    ("goodput_unreached_positions_reset", "goodput.py",
     "            if reached[j] > 0:\n                self.estimate[j] = float(accepted[j]) / float(reached[j])",
     "            self.estimate[j] = float(accepted[j]) / float(max(reached[j], 1))"),
    ("goodput_window_one_longer", "goodput.py",
     "self.batches = self.batches[-self.window:]",
     "self.batches = self.batches[-self.window - 1:]"),
    ("goodput_rescore_early", "goodput.py",
     "if self.since >= self.interval:",
     "if self.since >= self.interval - 1:"),
    ("prob_ratio_inverted", "probabilistic.py",
     "return bool(u_acc * q[d] < p[d])",
     "return bool(u_acc * p[d] < q[d])"),
    ("prob_accept_inclusive", "probabilistic.py",
     "return bool(u_acc * q[d] < p[d])",
     "return bool(u_acc * q[d] <= p[d])"),
    ("prob_residual_q_minus_p", "probabilistic.py",
     "r = np.maximum(p - q, 0.0)",
     "r = np.maximum(q - p, 0.0)"),
    ("prob_residual_not_clipped", "probabilistic.py",
     "r = np.maximum(p - q, 0.0)",
     "r = np.abs(p - q)"),
    ("prob_draft_without_temperature", "probabilistic.py",
     "z = (y - np.max(y)) / draft_temperature",
     "z = (y - np.max(y))"),
    ("prob_acceptance_word", "probabilistic.py",
     "(w[1] >> 8) * (1.0 / 16777216.0)",
     "(w[2] >> 8) * (1.0 / 16777216.0)"),
    ("goodput_counts_inclusive", "goodput.py",
     "accepted = np.array([int((a > j).sum())",
     "accepted = np.array([int((a >= j).sum())"),
    ("relaxed_margin_inclusive", "verify.py",
     "float(np.max(x)) - float(x[draft]) < margin",
     "float(np.max(x)) - float(x[draft]) <= margin"),
    ("relaxed_margin_against_min", "verify.py",
     "float(np.max(x)) - float(x[draft]) < margin",
     "float(x[draft]) - float(np.min(x)) < margin"),
    ("relaxed_from_position_off_by_one", "verify.py",
     "if j < from_position or generated + j < after_tokens:",
     "if j <= from_position or generated + j < after_tokens:"),
    ("relaxed_after_tokens_off_by_one", "verify.py",
     "if j < from_position or generated + j < after_tokens:",
     "if j < from_position or generated + j + 1 < after_tokens:"),
    ("relaxed_protects_draft_only", "verify.py",
     "if draft in protected or g in protected:",
     "if draft in protected:"),
    ("relaxed_gate_ignores_generated", "verify.py",
     "if j < from_position or generated + j < after_tokens:",
     "if j < from_position or j < after_tokens:"),
    ("margin_topp_farther_boundary", "verify.py",
     "topp_margin = min(topp_margin, top_p - cn[L - 1])",
     "topp_margin = max(topp_margin, top_p - cn[L - 1])"),
    ("margin_minp_all_tokens", "verify.py",
     "zs = z[S][x[S] < m]",
     "zs = z[x < m]"),
    ("margin_accept_smaller_side", "probabilistic.py",
     "accept_margin = abs(a - b) / max(a, b)",
     "accept_margin = abs(a - b) / min(a, b)"),
    ("margin_residual_normalised", "probabilistic.py",
     "        residual_margin = c[n] - t\n",
     "        residual_margin = (c[n] - t) / c[-1]\n"),
]


def _run_pins_on(name, fname, old, new):
    """Exit status of the pin suite against a mutant oracle, and its output tail."""
    tmp = tempfile.mkdtemp(prefix="oracle_mutant_")
    try:
        shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(tmp, "oracle"),
                        ignore=shutil.ignore_patterns("__pycache__"))
        path = os.path.join(tmp, "oracle", fname)
        src = open(path).read()
        assert src.count(old) == 1, "mutant %s: anchor text must occur exactly once" % name
        open(path, "w").write(src.replace(old, new))
        env = dict(os.environ)
        # the mutant package comes first; the repository (synth, tests) after it
        env["PYTHONPATH"] = os.pathsep.join([tmp, ROOT])
        env["PYTHONDONTWRITEBYTECODE"] = "1"
        cmd = [sys.executable, "-m", "pytest", PINS_BY_FILE.get(fname, PINS), "-x", "-q", "-p", "no:cacheprovider",
               "--import-mode=append", "--rootdir", ROOT]
        if fname != "philox.py":
            cmd += ["-k", "not rocrand"]
        r = subprocess.run(cmd, cwd=tmp, env=env, capture_output=True, text=True, timeout=600)
        # the suite must really have run against the mutant
        return r.returncode, (r.stdout + r.stderr)[-1500:]
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_every_mutant_fails_a_pin():
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        futs = {ex.submit(_run_pins_on, *m): m[0] for m in MUTANTS}
        results = {futs[f]: f.result() for f in concurrent.futures.as_completed(futs)}
    survived = [n for n, (rc, _) in results.items() if rc == 0]
    broken = {n: out for n, (rc, out) in results.items() if rc not in (0, 1)}
    assert not broken, "mutants that did not run as tests: %s" % broken
    assert not survived, "mutants no pin catches: %s" % survived


def test_unmutated_copy_passes_the_pins():
    # the same harness with a no-op substitution must pass, so a failure above
    # comes from the planted mistake and not from the harness
    rc, out = _run_pins_on("identity", "verify.py", "F32 = 0", "F32 = 0")
    assert rc == 0, out
