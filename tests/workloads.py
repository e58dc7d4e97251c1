"""Test helpers: move synthetic workloads to the GPU, run the oracle on them,
compare results, and keep sampled rows away from rounding-sensitive
thresholds (tie margin) by re-drawing them."""
import math

import numpy as np
import pytest

import oracle
import synth

# Relative tolerance of float outputs (log-sum-exp, confidence).
RTOL = 1e-5
# Tie margins for sampled rows: normalised cumulative mass within DELTA_MASS
# of top_p or of u, or z within DELTA_Z of ln(min_p), triggers a re-draw.
DELTA_MASS = 1e-5
DELTA_Z = 1e-4


def cuda_or_skip():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch


def to_dev(arr):
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def upload(wl):
    d = dict(logits=to_dev(wl.logits), offsets=to_dev(wl.offsets), owner=to_dev(wl.owner),
             drafts=to_dev(wl.drafts))
    if wl.sampled:
        d.update(temperature=to_dev(wl.temperature), top_k=to_dev(wl.top_k), top_p=to_dev(wl.top_p),
                 min_p=to_dev(wl.min_p))
    if wl.draft_logits is not None:
        d.update(draft_logits=to_dev(wl.draft_logits), selected=to_dev(wl.selected))
    return d


def oracle_of(wl, requests=None):
    if wl.sampled:
        return oracle.verify_sampled(wl.logits, wl.dtype, wl.V, wl.offsets, wl.owner, wl.drafts,
                                     wl.temperature, wl.top_k, wl.top_p, wl.min_p, wl.seed, wl.offset)
    return oracle.verify_greedy(wl.logits, wl.dtype, wl.V, wl.offsets, wl.owner, wl.drafts,
                                relaxed_topk=wl.relaxed_topk)


def host(t):
    return t.detach().cpu().numpy()


def assert_lse_close(got, want, rtol=RTOL):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    tol = rtol * np.maximum(1.0, np.abs(want))
    bad = np.flatnonzero(~(np.abs(got - want) <= tol))
    assert bad.size == 0, "lse mismatch at rows %s: got %s want %s" % (bad[:5], got[bad[:5]], want[bad[:5]])


def assert_same(out, ref, check_lse=True):
    """GPU outputs vs oracle: bit-exact integers, RTOL on log-sum-exp."""
    acc = host(out["accepted_len"])
    assert np.array_equal(acc, ref["accepted_len"]), \
        "accepted_len differs at %s" % np.flatnonzero(acc != ref["accepted_len"])[:10]
    assert np.array_equal(host(out["next_token"]), ref["next_token"])
    offs = host(out["out_offsets"])
    assert np.array_equal(offs, ref["out_offsets"])
    total = int(ref["out_offsets"][-1])
    assert np.array_equal(host(out["out_tokens"])[:total], ref["out_tokens"])
    rt = host(out["row_token"])
    assert np.array_equal(rt, ref["row_token"]), "row_token differs at rows %s" % np.flatnonzero(rt != ref["row_token"])[:10]
    if check_lse:
        assert_lse_close(host(out["row_lse"]), ref["row_lse"])
    assert int(host(out["error_flag"])[0]) == 0


def margin_rows(wl, rows=None):
    """Sampled rows whose outcome would hinge on rounding (see DELTA_*)."""
    bad = []
    rows = range(wl.R) if rows is None else rows
    for r in rows:
        i = int(wl.owner[r])
        T = float(np.float32(wl.temperature[i]))
        if T == 0.0:
            continue
        j = r - int(wl.offsets[i])
        x = oracle.row_f64(wl.logits, wl.dtype, r, wl.V)
        u = oracle.row_uniform(wl.seed, i, j, wl.offset)
        tp, um, mp = oracle.sampled_row_margins(x, T, int(wl.top_k[i]), float(np.float32(wl.top_p[i])),
                                                float(np.float32(wl.min_p[i])), u)
        if tp < DELTA_MASS or um < DELTA_MASS or mp < DELTA_Z:
            bad.append(r)
    return bad


def with_margins(wl, max_rounds=20):
    """Re-draw sampled rows until every one clears the tie margins."""
    rows = None
    for _ in range(max_rounds):
        bad = margin_rows(wl, rows)
        if not bad:
            return wl
        synth.redraw_rows(wl, bad)
        rows = bad
    raise RuntimeError("rows keep violating the tie margin")
