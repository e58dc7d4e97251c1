"""Verification with probabilistic drafts on the GPU against the oracle's
rejection sampler (oracle/probabilistic.py).

Batches are ragged, with per-request target temperature (0 = greedy) and
filters, and a draft temperature per request (0 = the draft row's arg-max
was proposed). Draft rows are the target rows of the same position plus
noise, so acceptance and rejection both occur, and each draft token is drawn
from its draft row's law. Special cases: drafts whose law equals the
target's are always accepted; a greedy target reduces to greedy
verification."""
import numpy as np
import pytest

import oracle
import synth
from oracle.probabilistic import draft_probs, verify_probabilistic
from tests.workloads import cuda_or_skip, host, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vsv():
    cuda_or_skip()
    import draft_token_verification_packed_amd as m
    m.lib()
    return m


def _store(x, dtype):
    return synth.f32_to_bf16_bits(x) if dtype == oracle.BF16 else x.astype(np.float32)


def _batch(rng, B, Kmax, V, dtype, sigma=2.5, noise=0.3, params=None, same=False, ties=False, ninf=0):
    Ks = rng.integers(0, Kmax + 1, B)
    off = np.zeros(B + 1, dtype=np.int32)
    off[1:] = np.cumsum(Ks + 1)
    R = int(off[-1])
    owner = np.repeat(np.arange(B, dtype=np.int32), (Ks + 1).astype(np.int64))
    x = (rng.standard_normal((R, V)) * sigma).astype(np.float32)
    rows = [int(off[i]) + j for i in range(B) for j in range(int(Ks[i]))]   # draft rows, draft order
    y = x[rows] if same else (x[rows] + noise * rng.standard_normal((R - B, V))).astype(np.float32)
    if ties:      # integer grids: many ties, at the maxima too
        x = (rng.integers(-6, 7, (R, V)) * 0.5).astype(np.float32)
        y = (rng.integers(-6, 7, (R - B, V)) * 0.5).astype(np.float32)
    if ninf:      # every ninf-th draft logit is -inf
        y = np.array(y, dtype=np.float32)
        y[:, ::ninf] = -np.inf
    xs, ys = _store(x, dtype), _store(y.reshape(R - B, V), dtype)
    if params is None:
        def params(i):
            return (float(rng.choice([0.0, 0.7, 1.0])), int(rng.choice([0, 0, 20])),
                    float(rng.choice([1.0, 0.9])), float(rng.choice([0.0, 0.0, 0.05])),
                    float(rng.choice([0.0, 0.5, 1.0])))
    P = [params(i) for i in range(B)]
    T = np.array([p[0] for p in P], dtype=np.float32)
    TK = np.array([p[1] for p in P], dtype=np.int32)
    TP = np.array([p[2] for p in P], dtype=np.float32)
    MP = np.array([p[3] for p in P], dtype=np.float32)
    TD = np.array([p[4] for p in P], dtype=np.float32)
    drafts = np.zeros(R - B, dtype=np.int32)
    for i in range(B):
        for j in range(int(Ks[i])):
            q_row = int(off[i]) - i + j
            q = draft_probs(oracle.row_f64(ys, dtype, q_row, V), float(TD[i]))
            drafts[q_row] = int(rng.choice(V, p=q / q.sum()))
    return dict(xs=xs, ys=ys, off=off, owner=owner, drafts=drafts, T=T, TK=TK, TP=TP, MP=MP, TD=TD, V=V,
                dtype=dtype)


def _run(vsv, b, seed, offset):
    import torch
    out = vsv.verify_probabilistic(to_dev(b["xs"]), to_dev(b["off"]), to_dev(b["owner"]), to_dev(b["drafts"]),
                                   to_dev(b["ys"]), to_dev(b["T"]), to_dev(b["TK"]), to_dev(b["TP"]),
                                   to_dev(b["MP"]), to_dev(b["TD"]), seed, offset, vocab=b["V"])
    torch.cuda.synchronize()
    return out


def _oracle(b, seed, offset):
    return verify_probabilistic(b["xs"], b["dtype"], b["V"], b["off"], b["owner"], b["drafts"], b["ys"], b["T"],
                                b["TK"], b["TP"], b["MP"], b["TD"], seed, offset)


def _assert_same(out, ref):
    assert np.array_equal(host(out["accepted_len"]), ref["accepted_len"]), \
        (host(out["accepted_len"]), ref["accepted_len"])
    assert np.array_equal(host(out["next_token"]), ref["next_token"])
    assert np.array_equal(host(out["out_offsets"]), ref["out_offsets"])
    total = int(ref["out_offsets"][-1])
    assert np.array_equal(host(out["out_tokens"])[:total], ref["out_tokens"])
    rt = host(out["row_token"])
    assert np.array_equal(rt, ref["row_token"]), "row_token differs at rows %s" % np.flatnonzero(rt != ref["row_token"])
    assert int(host(out["error_flag"])[0]) == 0


@pytest.mark.parametrize("seed,B,Kmax,V,dtype", [
    (0, 12, 4, 1000, oracle.F32),
    (1, 10, 5, 4099, oracle.BF16),
    (2, 30, 3, 64, oracle.F32),
    (3, 8, 7, 2048, oracle.BF16),
    (4, 20, 2, 5, oracle.F32),
])
def test_matches_oracle(vsv, seed, B, Kmax, V, dtype):
    rng = np.random.default_rng(4200 + seed)
    b = _batch(rng, B, Kmax, V, dtype)
    print("probabilistic seed=%d B=%d Kmax=%d V=%d dtype=%d R=%d" % (seed, B, Kmax, V, dtype, int(b["off"][-1])),
          flush=True)
    ref = _oracle(b, 77 + seed, seed)
    _assert_same(_run(vsv, b, 77 + seed, seed), ref)
    # both outcomes occur
    K = np.diff(b["off"]) - 1
    assert np.any(ref["accepted_len"] < K) or seed == 4


def test_full_vocab_bf16(vsv):
    rng = np.random.default_rng(4300)
    b = _batch(rng, 3, 3, synth.VOCAB, oracle.BF16, sigma=3.0, noise=0.5,
               params=lambda i: [(0.7, 0, 0.95, 0.0, 0.7), (1.0, 50, 0.9, 0.05, 1.0), (0.0, 0, 1.0, 0.0, 1.0)][i])
    print("probabilistic full vocab R=%d" % int(b["off"][-1]), flush=True)
    _assert_same(_run(vsv, b, 5, 0), _oracle(b, 5, 0))


def test_draft_law_equal_to_target_accepts_everything(vsv):
    rng = np.random.default_rng(4400)
    b = _batch(rng, 16, 5, 3000, oracle.F32, same=True,
               params=lambda i: (float([0.5, 1.0, 1.5][i % 3]), 0, 1.0, 0.0, float([0.5, 1.0, 1.5][i % 3])))
    out = _run(vsv, b, 9, 3)
    K = np.diff(b["off"]) - 1
    assert np.array_equal(host(out["accepted_len"]), K)
    # p = q makes every draft row's residual max(0, p - q) pure rounding
    # noise on both sides, so a draft row's would-be replacement is not
    # unique; everything emitted (drafts, then the bonus row's draw) is
    ref = _oracle(b, 9, 3)
    for k in ("accepted_len", "next_token", "out_offsets", "out_tokens"):
        assert np.array_equal(host(out[k]), ref[k]), k
    bonus = b["off"][1:] - 1
    assert np.array_equal(host(out["row_token"])[bonus], ref["row_token"][bonus])
    assert int(host(out["error_flag"])[0]) == 0


def test_greedy_target_is_greedy_verification(vsv):
    rng = np.random.default_rng(4500)
    b = _batch(rng, 24, 4, 1500, oracle.BF16,
               params=lambda i: (0.0, 0, 1.0, 0.0, float([0.0, 1.0][i % 2])))
    out = _run(vsv, b, 1, 0)
    ref = oracle.verify_greedy(b["xs"], b["dtype"], b["V"], b["off"], b["owner"], b["drafts"])
    for k in ("accepted_len", "next_token", "out_offsets", "row_token"):
        assert np.array_equal(host(out[k]), ref[k]), k
    _assert_same(out, _oracle(b, 1, 0))


def test_flags_and_empty_batch(vsv):
    import torch
    rng = np.random.default_rng(4600)
    b = _batch(rng, 4, 3, 500, oracle.F32, params=lambda i: (1.0, 0, 1.0, 0.0, 1.0))
    b["TD"][1] = -1.0
    out = _run(vsv, b, 2, 0)
    assert int(host(out["error_flag"])[0]) & 8      # draft temperature out of range
    b = _batch(rng, 4, 3, 500, oracle.F32, params=lambda i: (1.0, 0, 1.0, 0.0, 1.0))
    if b["ys"].shape[0]:
        b["ys"][0, 7] = np.nan
        out = _run(vsv, b, 2, 0)
        assert int(host(out["error_flag"])[0]) & 4  # NaN in a draft row
    e = torch.zeros(0, 16, dtype=torch.float32, device="cuda")
    z = torch.zeros(1, dtype=torch.int32, device="cuda")
    ei = torch.zeros(0, dtype=torch.int32, device="cuda")
    ef = torch.zeros(0, dtype=torch.float32, device="cuda")
    out = vsv.verify_probabilistic(e, z, ei, ei, e, ef, ei, ef, ef, ef, 0, 0, vocab=16)
    torch.cuda.synchronize()
    assert int(host(out["error_flag"])[0]) == 0


def test_tied_maxima_and_minus_inf(vsv):
    """Draft rows with tied maxima (Td = 0 proposes the lowest arg-max) and
    draft rows holding -inf logits, against the oracle."""
    rng = np.random.default_rng(4700)
    b = _batch(rng, 12, 4, 700, oracle.F32, ties=True,
               params=lambda i: (float([0.0, 0.8, 1.0][i % 3]), 0, float([1.0, 0.9][i % 2]), 0.0,
                                 float([0.0, 0.7][i % 2])))
    print("probabilistic ties R=%d" % int(b["off"][-1]), flush=True)
    _assert_same(_run(vsv, b, 11, 0), _oracle(b, 11, 0))
    b = _batch(rng, 10, 4, 1200, oracle.BF16, ninf=7,
               params=lambda i: (float([0.7, 1.0][i % 2]), 0, 0.9, 0.0, float([0.0, 0.5, 1.0][i % 3])))
    _assert_same(_run(vsv, b, 12, 1), _oracle(b, 12, 1))
