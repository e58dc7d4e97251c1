"""Random small batches through both verify entry points, against the oracle,
and a run-twice bit comparison of the sampled path (a race smoke test).

Each case draws the batch size, ragged draft counts, vocabulary size,
element type, row alignment and per-request parameters from its seed, so
the launch rules (a row whole or cut into parts; ordered or plain sampled
queue) and the filters all get exercised on shapes nobody
picked by hand."""
import numpy as np
import pytest

import oracle
from tests.test_gpu_greedy import _custom
from tests.workloads import assert_same, cuda_or_skip, custom_sampled, host, oracle_custom, to_dev

pytestmark = pytest.mark.gpu

VOCABS = [1, 5, 64, 1000, 4099, 20000]


@pytest.fixture(scope="module")
def vsv():
    cuda_or_skip()
    import draft_token_verification_packed_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("seed", range(12))
def test_fuzz_greedy(vsv, seed):
    import torch
    rng = np.random.default_rng(9000 + seed)
    B = int(rng.integers(1, 400)) if seed % 4 == 0 else int(rng.integers(1, 60))
    Kmax = int(rng.integers(0, 8))
    V = int(rng.choice(VOCABS))
    dtype = int(rng.integers(0, 2))
    shift = int(rng.integers(0, 2))
    relaxed = int(rng.choice([1, 1, 2, 4])) if V >= 4 else 1
    store, off, owner, drafts = _custom(rng, B, Kmax, V, dtype, ld=V + int(rng.integers(0, 5)), shift=shift,
                                        ties=bool(seed % 3 == 0))
    print("fuzz greedy seed=%d B=%d Kmax=%d V=%d dtype=%d shift=%d relaxed=%d R=%d" %
          (seed, B, Kmax, V, dtype, shift, relaxed, int(off[-1])), flush=True)
    t = to_dev(store)[:, shift:]
    out = vsv.verify_greedy(t, to_dev(off), to_dev(owner), to_dev(drafts), relaxed_topk=relaxed, vocab=V)
    torch.cuda.synchronize()
    ref = oracle.verify_greedy(store[:, shift:], dtype, V, off, owner, drafts, relaxed_topk=relaxed)
    assert_same(out, ref)
    assert int(host(out["error_flag"])[0]) == 0


def _random_params(rng, V):
    def params(i):
        if rng.random() < 0.3:
            return (0.0, 0, 1.0, 0.0)
        T = float(rng.choice([0.3, 0.7, 1.0, 1.5]))
        tk = int(rng.choice([0, 0, 1, 5, 50])) if V > 1 else 0
        tp = float(rng.choice([1.0, 0.95, 0.8, 0.5]))
        mp = float(rng.choice([0.0, 0.0, 0.02, 0.2]))
        return (T, tk, tp, mp)
    return params


@pytest.mark.parametrize("seed", range(8))
def test_fuzz_sampled(vsv, seed):
    rng = np.random.default_rng(9500 + seed)
    B = int(rng.integers(1, 40))
    Kmax = int(rng.integers(0, 6))
    V = int(rng.choice(VOCABS[:5]))
    dtype = int(rng.integers(0, 2))
    shift = int(rng.integers(0, 2))
    b = custom_sampled(rng, B, Kmax, V, dtype, _random_params(rng, V), seed=100 + seed, offset=seed,
                       ld=V + 2, shift=shift)
    print("fuzz sampled seed=%d B=%d Kmax=%d V=%d dtype=%d shift=%d R=%d" %
          (seed, B, Kmax, V, dtype, shift, int(b["offsets"][-1])), flush=True)
    t = to_dev(b["store"])[:, b["shift"]:]
    out = vsv.verify_sampled(t, to_dev(b["offsets"]), to_dev(b["owner"]), to_dev(b["drafts"]), to_dev(b["T"]),
                             to_dev(b["TK"]), to_dev(b["TP"]), to_dev(b["MP"]), b["seed"], b["offset"], vocab=V)
    import torch
    torch.cuda.synchronize()
    assert_same(out, oracle_custom(b))


@pytest.mark.parametrize("B,K", [(24, 3), (300, 4)])
def test_sampled_run_twice_bit_identical(vsv, B, K):
    """Two calls on the same inputs give the same bits in every output:
    24 requests take the longest-first queue, 300 requests (1500 rows, more
    than two per workgroup slot) the plain one."""
    import torch
    rng = np.random.default_rng(77 + B)
    V = 2048
    R = B * (K + 1)
    x = (rng.standard_normal((R, V)) * 2.5).astype(np.float32)
    off = np.arange(0, R + 1, K + 1, dtype=np.int32)
    owner = np.repeat(np.arange(B, dtype=np.int32), K + 1)
    drafts = rng.integers(0, V, R - B).astype(np.int32)
    T = rng.choice(np.array([0.0, 0.7, 1.0], dtype=np.float32), B)
    d = [to_dev(a) for a in (x, off, owner, drafts, T, np.full(B, 40, np.int32), np.full(B, 0.9, np.float32),
                             np.full(B, 0.02, np.float32))]
    outs = []
    for _ in range(2):
        outs.append(vsv.verify_sampled(*d, 31, 0))
        torch.cuda.synchronize()
    for k in ("accepted_len", "next_token", "out_offsets", "out_tokens", "row_token", "row_lse"):
        assert np.array_equal(host(outs[0][k]), host(outs[1][k])), k


# Seeds of a wider random campaign (built as below) whose bfloat16 rows
# filtered by top-p alone drew the wrong token: their candidates reached
# far below the locator's bins (a window down to zero or below spans many
# more codes than the bins hold), and the bound on the weight of the first
# element outside the bins counted only the elements below tau.
@pytest.mark.parametrize("seed", [20036, 20079, 20556, 21444, 22093, 22251, 22665])
def test_fuzz_sampled_top_p_past_the_bins(vsv, seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    Kmax = int(rng.integers(0, 6))
    V = int(rng.choice(VOCABS[:5]))
    dtype = int(rng.integers(0, 2))
    shift = int(rng.integers(0, 2))
    b = custom_sampled(rng, B, Kmax, V, dtype, _random_params(rng, V), seed=seed, offset=seed % 7, ld=V + 2,
                       shift=shift, ties=bool(rng.random() < 0.3))
    print("campaign seed=%d B=%d Kmax=%d V=%d dtype=%d shift=%d R=%d" %
          (seed, B, Kmax, V, dtype, shift, int(b["offsets"][-1])), flush=True)
    t = to_dev(b["store"])[:, b["shift"]:]
    out = vsv.verify_sampled(t, to_dev(b["offsets"]), to_dev(b["owner"]), to_dev(b["drafts"]), to_dev(b["T"]),
                             to_dev(b["TK"]), to_dev(b["TP"]), to_dev(b["MP"]), b["seed"], b["offset"], vocab=V)
    import torch
    torch.cuda.synchronize()
    assert_same(out, oracle_custom(b))
