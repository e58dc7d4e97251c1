"""GPU parity of sampled (and mixed greedy/sampled) verification.

Rows are drawn with a tie margin (tests/workloads.py) so that no decision
hinges on rounding; tokens, accepted lengths and compacted outputs must be
bit-exact, log-sum-exp within 1e-5 relative."""
import numpy as np
import pytest

import oracle
import synth
from tests.workloads import (assert_lse_close, assert_same, cuda_or_skip, custom_sampled, host,
                             oracle_custom, oracle_of, to_dev, upload, with_margins)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vsv():
    cuda_or_skip()
    import draft_token_verification_packed_amd as m
    m.lib()
    return m


def run_sampled(vsv, wl, d=None):
    import torch
    d = upload(wl) if d is None else d
    out = vsv.verify_sampled(d["logits"], d["offsets"], d["owner"], d["drafts"], d["temperature"],
                             d["top_k"], d["top_p"], d["min_p"], wl.seed, wl.offset, vocab=wl.V)
    torch.cuda.synchronize()
    return out


def run_custom(vsv, b):
    import torch
    t = to_dev(b["store"])[:, b["shift"]:]
    out = vsv.verify_sampled(t, to_dev(b["offsets"]), to_dev(b["owner"]), to_dev(b["drafts"]), to_dev(b["T"]),
                             to_dev(b["TK"]), to_dev(b["TP"]), to_dev(b["MP"]), b["seed"], b["offset"],
                             vocab=b["V"])
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("B", [16, 128])
def test_ragged_sampled(vsv, B):
    wl = with_margins(synth.make("ragged", B=B))
    out = run_sampled(vsv, wl)
    assert_same(out, oracle_of(wl))


@pytest.mark.parametrize("B", [8, 48])
def test_large_mixed_batch(vsv, B):
    wl = with_margins(synth.make("mixed", B=B))
    out = run_sampled(vsv, wl)
    ref = oracle_of(wl)
    assert_same(out, ref)
    # the exact whole-row path is for rare rows only at this shape
    sampled_rows = int(sum(int(wl.offsets[i + 1] - wl.offsets[i]) for i in range(wl.B) if wl.temperature[i] > 0))
    assert int(host(out["slow_rows"])[0]) <= max(1, sampled_rows // 20)


def test_temperature_zero_is_greedy(vsv):
    import torch
    wl = synth.make("mixed", B=16)
    d = upload(wl)
    z = torch.zeros_like(d["temperature"])
    s = vsv.verify_sampled(d["logits"], d["offsets"], d["owner"], d["drafts"], z, d["top_k"], d["top_p"],
                           d["min_p"], wl.seed)
    g = vsv.verify_greedy(d["logits"], d["offsets"], d["owner"], d["drafts"])
    torch.cuda.synchronize()
    for k in ("accepted_len", "next_token", "out_offsets", "row_token"):
        assert np.array_equal(host(s[k]), host(g[k])), k
    # the greedy entry point sums a row in pieces, so the two log-sum-exps may
    # differ in their last float bits; both are held to the oracle
    assert_lse_close(host(s["row_lse"]), host(g["row_lse"]), rtol=1e-6)
    ref = oracle.verify_greedy(wl.logits, wl.dtype, wl.V, wl.offsets, wl.owner, wl.drafts)
    assert_same(s, ref)
    assert_same(g, ref)


GRID = [
    (1.0, 0, 1.0, 0.0), (0.5, 50, 0.9, 0.05), (1.0, 50, 0.9, 0.05), (0.7, 0, 0.95, 0.0), (1.3, 7, 1.0, 0.0),
    (0.8, 0, 0.6, 0.0), (1.0, 0, 1.0, 0.2), (0.6, 3, 0.5, 0.3), (2.0, 0, 0.9, 0.0), (1.0, 1, 1.0, 0.0),
    (1.0, 0, 1e-6, 0.0), (1.0, 0, 1.0, 1.0), (0.05, 0, 1.0, 0.0), (0.0, 5, 0.5, 0.1), (1.5, 200, 0.99, 0.01),
    (0.9, 0, 1.0, 0.01),
]


@pytest.mark.parametrize("V,dtype", [(152064, oracle.BF16), (152064, oracle.F32), (4099, oracle.BF16),
                                     (33, oracle.F32), (1, oracle.BF16)])
def test_filter_grid(vsv, V, dtype):
    rng = np.random.default_rng(V + dtype)
    b = custom_sampled(rng, len(GRID), 3, V, dtype, lambda i: GRID[i], seed=77 + V, offset=5)
    out = run_custom(vsv, b)
    assert_same(out, oracle_custom(b))


@pytest.mark.parametrize("dtype", [oracle.F32, oracle.BF16])
def test_ties_and_misaligned_rows(vsv, dtype):
    rng = np.random.default_rng(321 + dtype)
    b = custom_sampled(rng, len(GRID), 2, 5000, dtype, lambda i: GRID[i], seed=9, ties=True, ld=5003, shift=1)
    # (ties: 81 distinct values, so top-k cuts cross tie groups)
    out = run_custom(vsv, b)
    assert_same(out, oracle_custom(b))


def test_exact_whole_row_path(vsv):
    """Unfiltered sampling over a flat distribution: the draw usually lies
    beyond the captured candidates and the exact path decides."""
    rng = np.random.default_rng(2024)
    b = custom_sampled(rng, 6, 2, 152064, oracle.BF16, lambda i: (1.5, 0, 1.0, 0.0), seed=3, sigma=1.0)
    out = run_custom(vsv, b)
    assert_same(out, oracle_custom(b))
    assert int(host(out["slow_rows"])[0]) > 0


def test_invalid_parameters_are_flagged(vsv):
    import torch
    wl = synth.make("mixed", B=4, V=1000)
    d = upload(wl)
    T = d["temperature"].clone()
    T[1] = -1.0
    tp = d["top_p"].clone()
    tp[3] = 1.5
    out = vsv.verify_sampled(d["logits"], d["offsets"], d["owner"], d["drafts"], T, d["top_k"], tp, d["min_p"],
                             wl.seed)
    torch.cuda.synchronize()
    assert int(host(out["error_flag"])[0]) & vsv.FLAG_PARAMS


def test_large_mixed_draft_confidence(vsv):
    import torch
    wl = synth.make("mixed", B=16)
    d = upload(wl)
    conf, lse, flag = vsv.draft_confidence(d["draft_logits"], d["selected"])
    torch.cuda.synchronize()
    rc, rl = oracle.draft_confidence(wl.draft_logits, wl.dtype, wl.V, wl.selected)
    assert_lse_close(host(lse), rl)
    np.testing.assert_allclose(host(conf), rc, rtol=1e-5, atol=0)


def test_draft_confidence_without_rows_and_with_one_column(vsv):
    """Draft logits with no rows (from numpy such a tensor has zero strides)
    give empty outputs and no flag; a one-token vocabulary gives confidence
    1 and the logit itself as the log-sum-exp."""
    import torch
    empty = to_dev(np.zeros((0, 5), dtype=np.float32))
    conf, lse, flag = vsv.draft_confidence(empty)
    torch.cuda.synchronize()
    assert conf.numel() == 0 and lse.numel() == 0 and int(host(flag)[0]) == 0
    x = np.array([[1.5], [-2.0], [0.25]], dtype=np.float32)
    conf, lse, flag = vsv.draft_confidence(to_dev(x))
    torch.cuda.synchronize()
    rc, rl = oracle.draft_confidence(x, oracle.F32, 1)
    np.testing.assert_allclose(host(conf), rc, rtol=1e-6, atol=0)
    assert_lse_close(host(lse), rl)
    assert int(host(flag)[0]) == 0


@pytest.mark.parametrize("B,Kmax", [(300, 2), (600, 1)])
def test_many_requests_in_longest_first_order(vsv, B, Kmax):
    """A batch with more rows than CUs and at most two rows per workgroup
    slot goes out in the ordered queue (sampled requests' rows, then greedy
    ones), whose order each workgroup derives at its start: 300 requests
    give its 512 threads one request each, 600 give them two; a third of the
    requests are greedy."""
    rng = np.random.default_rng(4242 + B)
    params = lambda i: [(0.0, 0, 1.0, 0.0), (0.8, 40, 0.9, 0.0), (1.0, 0, 0.95, 0.05)][i % 3]
    b = custom_sampled(rng, B, Kmax, 4099, oracle.BF16, params, seed=17, offset=3)
    assert 256 < int(b["offsets"][-1]) <= 1024
    out = run_custom(vsv, b)
    assert_same(out, oracle_custom(b))
    assert int(host(out["error_flag"])[0]) == 0


@pytest.mark.parametrize("B", [12, 80])
def test_layout_errors_are_flagged(vsv, B):
    """Inconsistent owner maps and offsets set the layout flag; the launch
    still completes and writes inside the buffers. 80 requests (351 rows)
    take the ordered queue, whose order falls back to the plain row order
    for offsets that do not rise."""
    import torch
    wl = synth.make("ragged", B=B, V=1000)
    d = upload(wl)
    own = d["owner"].clone()
    own[3] = (own[3] + 1) % wl.B
    out = vsv.verify_sampled(d["logits"], d["offsets"], own, d["drafts"], d["temperature"], d["top_k"],
                             d["top_p"], d["min_p"], wl.seed)
    torch.cuda.synchronize()
    assert int(host(out["error_flag"])[0]) & vsv.FLAG_LAYOUT
    off = d["offsets"].clone()
    off[5] = off[4]                       # request 4 owns no rows: offsets not increasing
    out = vsv.verify_sampled(d["logits"], off, d["owner"], d["drafts"], d["temperature"], d["top_k"],
                             d["top_p"], d["min_p"], wl.seed)
    torch.cuda.synchronize()
    assert int(host(out["error_flag"])[0]) & vsv.FLAG_LAYOUT
    # the next well-formed call on the same workspace is unaffected
    good = run_sampled(vsv, with_margins(wl))
    assert_same(good, oracle_of(wl))


@pytest.mark.parametrize("dtype", [oracle.F32, oracle.BF16])
def test_top_p_cut_beyond_the_candidates(vsv, dtype):
    """Top-p alone over flat rows: the cut lies below the captured
    candidates in every row. Draws that land among the candidates for every
    survivor weight the cut allows are decided there; the rest take the
    whole-row path. Both happen here, and every row matches the oracle."""
    rng = np.random.default_rng(8080 + dtype)
    b = custom_sampled(rng, 24, 1, 152064, dtype, lambda i: (1.0, 0, 0.95, 0.0), seed=21, offset=2, sigma=3.0)
    R = int(b["offsets"][-1])
    out = run_custom(vsv, b)
    assert_same(out, oracle_custom(b))
    slow = int(host(out["slow_rows"])[0])
    print("top-p beyond the candidates: R=%d, whole-row path %d" % (R, slow), flush=True)
    assert 0 < slow < R
