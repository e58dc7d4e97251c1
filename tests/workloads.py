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
# The device sums the row's weights in float32 groups accumulated in float64
# (relative error of the total a few 1e-8 at the benchmark shapes) and the
# candidates' weights in float64; z is computed in float64 on both sides.
DELTA_MASS = 2e-7
DELTA_Z = 1e-9


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


def row_margins_ok(x, T, k, p, mp, u):
    tp, um, mpm = oracle.sampled_row_margins(x, T, k, p, mp, u)
    return tp >= DELTA_MASS and um >= DELTA_MASS and mpm >= DELTA_Z


def custom_sampled(rng, B, Kmax, V, dtype, params, seed, offset=0, ties=False, sigma=2.5, ld=None,
                   shift=0, hit=0.6):
    """A packed sampled batch with per-request (T, top_k, top_p, min_p) from
    `params(i)`. Drafts hit the oracle's own draw with probability `hit`, so
    acceptance chains occur; sampled rows are re-drawn until they clear the
    tie margins. Returns numpy arrays plus the [R, ld + shift] storage."""
    Ks = rng.integers(0, Kmax + 1, size=B)
    off = np.zeros(B + 1, dtype=np.int32)
    off[1:] = np.cumsum(Ks + 1)
    R = int(off[-1])
    owner = np.repeat(np.arange(B, dtype=np.int32), Ks + 1)
    ld = V if ld is None else ld
    P = [params(i) for i in range(B)]
    T = np.array([q[0] for q in P], dtype=np.float32)
    TK = np.array([q[1] for q in P], dtype=np.int32)
    TP = np.array([q[2] for q in P], dtype=np.float32)
    MP = np.array([q[3] for q in P], dtype=np.float32)
    store_dtype = np.uint16 if dtype == oracle.BF16 else np.float32
    store = np.zeros((R, ld + shift), dtype=store_dtype)
    drafts = np.zeros(R - B, dtype=np.int32)
    for i in range(B):
        for j in range(int(Ks[i]) + 1):
            r = int(off[i]) + j
            for attempt in range(200):
                if ties:
                    x = (rng.integers(-40, 41, size=V) * 0.125).astype(np.float32)
                else:
                    x = (rng.standard_normal(V) * sigma).astype(np.float32)
                row = np.zeros(ld + shift, dtype=np.float32)
                row[shift:shift + V] = x
                if dtype == oracle.BF16:
                    stored = synth.f32_to_bf16_bits(row)
                else:
                    stored = row
                xv = oracle.row_f64(stored[None, shift:], dtype, 0, V)
                Tf = float(np.float32(T[i]))
                if Tf == 0.0:
                    break
                u = oracle.row_uniform(seed, i, j, offset)
                if row_margins_ok(xv, Tf, int(TK[i]), float(np.float32(TP[i])), float(np.float32(MP[i])), u):
                    break
            else:
                raise RuntimeError("row %d keeps violating the tie margin" % r)
            store[r] = stored
            if j < Ks[i]:
                if Tf == 0.0:
                    tok = oracle.greedy_token(xv)
                else:
                    tok = oracle.sample_from_u(xv, Tf, int(TK[i]), float(np.float32(TP[i])),
                                               float(np.float32(MP[i])), u)
                drafts[r - i] = tok if rng.random() < hit else int(rng.integers(0, V))
    return dict(store=store, offsets=off, owner=owner, drafts=drafts, T=T, TK=TK, TP=TP, MP=MP,
                seed=seed, offset=offset, V=V, dtype=dtype, shift=shift)


def oracle_custom(b):
    return oracle.verify_sampled(b["store"][:, b["shift"]:], b["dtype"], b["V"], b["offsets"], b["owner"],
                                 b["drafts"], b["T"], b["TK"], b["TP"], b["MP"], b["seed"], b["offset"])
