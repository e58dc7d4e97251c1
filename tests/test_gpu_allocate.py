"""GPU parity of adaptive verify allocation against the oracle.

Every output is compared element by element and must be bit-exact: verify
lengths, offsets, owners, source rows and packed drafts (integers), and the
float32 running products (IEEE products of the same operands in the same
order; +0 and -0 compare equal). The last tests chain allocation into
verification on the device and compare the chain with the oracle's."""
import numpy as np
import pytest

import oracle
import synth
from oracle.allocate import allocate_verify
from tests.workloads import cuda_or_skip, host, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vsv():
    cuda_or_skip()
    import draft_token_verification_packed_amd as m
    m.lib()
    return m


def check_allocation(vsv, B, K, G, kind, seed, with_drafts=True):
    import torch
    conf, drafts = synth.scores(B, K, seed, kind)
    print("allocate B=%d K=%d G=%d kind=%s seed=%d" % (B, K, G, kind, seed), flush=True)
    out = vsv.allocate_verify(to_dev(conf) if B * K else None, to_dev(drafts) if with_drafts and B * K else None,
                              B, K, G)
    torch.cuda.synchronize()
    ref = allocate_verify(conf, drafts, B, K, G)
    assert np.array_equal(host(out["verify_len"]), ref["verify_len"])
    assert np.array_equal(host(out["row_offsets"]), ref["row_offsets"])
    assert np.array_equal(host(out["row_owner"])[:G], ref["row_owner"])
    assert np.array_equal(host(out["row_source"])[:G], ref["row_source"])
    if with_drafts and G > B:
        assert np.array_equal(host(out["packed_drafts"])[:G - B], ref["packed_drafts"])
    if B * K:
        got_p = host(out["prefix"])[:B * K].reshape(B, K)
        assert np.array_equal(got_p, ref["prefix"])   # == treats -0 and +0 alike
    return out, ref


@pytest.mark.parametrize("kind", ["confidence", "uniform", "ties", "special", "tiny"])
@pytest.mark.parametrize("B,K", [(1, 1), (3, 4), (37, 5), (128, 4), (512, 7)])
def test_parity_over_budgets(vsv, kind, B, K):
    rng = np.random.default_rng([B, K, len(kind)])
    budgets = {B, B + 1, B * (K + 1), B * (K + 1) - 1, B + (B * K) // 2}
    budgets |= set(int(g) for g in rng.integers(B, B * (K + 1) + 1, size=3))
    for G in sorted(budgets):
        check_allocation(vsv, B, K, G, kind, seed=31 + G)


@pytest.mark.parametrize("B,K", [(8192, 2), (2048, 8), (1, 16384), (16384 // 7, 7)])
def test_largest_batches(vsv, B, K):
    for G in (B, B + (B * K) // 3, B * (K + 1)):
        check_allocation(vsv, B, K, G, "confidence", seed=5)


def test_no_drafts_and_no_positions(vsv):
    check_allocation(vsv, 64, 4, 200, "uniform", seed=2, with_drafts=False)
    check_allocation(vsv, 10, 0, 10, "uniform", seed=3)   # K = 0: one bonus row each


def test_repeated_calls_give_identical_results(vsv):
    import torch
    conf, drafts = synth.scores(512, 7, 9, "ties")
    c, d = to_dev(conf), to_dev(drafts)
    first = vsv.allocate_verify(c, d, 512, 7, 2048)
    for _ in range(5):
        again = vsv.allocate_verify(c, d, 512, 7, 2048)
        torch.cuda.synchronize()
        for k in ("verify_len", "row_offsets", "row_owner", "row_source", "packed_drafts"):
            assert torch.equal(first[k], again[k]), k


@pytest.mark.parametrize("seed", range(3))
def test_allocation_chains_into_verification(vsv, seed):
    # scores -> allocation -> gather of the chosen target rows -> greedy
    # verification, all on the device, equals the same chain in the oracle
    import torch
    B, K, V = 24, 5, 2048
    rng = np.random.default_rng(700 + seed)
    x = rng.normal(0.0, 2.0, size=(B * (K + 1), V)).astype(np.float32)
    am = x.argmax(axis=1)
    drafts = np.array([am[i * (K + 1) + j] if rng.uniform() < 0.7 else (am[i * (K + 1) + j] + 3) % V
                       for i in range(B) for j in range(K)], dtype=np.int32)
    conf = synth.scores(B, K, seed, "confidence")[0]
    G = B + int(rng.integers(0, B * K + 1))
    print("chain B=%d K=%d V=%d G=%d seed=%d" % (B, K, V, G, seed), flush=True)
    al = vsv.allocate_verify(to_dev(conf), to_dev(drafts), B, K, G)
    rows = to_dev(x).index_select(0, al["row_source"][:G].long()).contiguous()
    packed = al["packed_drafts"][:G - B] if G > B else None
    got = vsv.verify_greedy(rows, al["row_offsets"], al["row_owner"][:G].contiguous(),
                            packed.contiguous() if packed is not None else None)
    torch.cuda.synchronize()
    ref_al = allocate_verify(conf, drafts, B, K, G)
    ref = oracle.verify_greedy(x[ref_al["row_source"]], oracle.F32, V, ref_al["row_offsets"],
                               ref_al["row_owner"], ref_al["packed_drafts"])
    assert np.array_equal(host(got["accepted_len"]), ref["accepted_len"])
    assert np.array_equal(host(got["next_token"]), ref["next_token"])
    assert np.array_equal(host(got["out_offsets"]), ref["out_offsets"])
    n = int(ref["out_offsets"][-1])
    assert np.array_equal(host(got["out_tokens"])[:n], ref["out_tokens"])


def test_rejects_bad_arguments(vsv):
    import torch
    c = torch.zeros(12, dtype=torch.float32, device="cuda")
    for B, K, G in ((3, 4, 2), (3, 4, 16), (8193, 1, 8193), (2049, 8, 2049)):
        with pytest.raises((vsv.VSVError, ValueError)):
            vsv.allocate_verify(torch.zeros(max(B * K, 1), device="cuda"), None, B, K, G)
    out = vsv.allocate_verify(c, None, 0, 4, 0)   # empty batch: no-op
    assert out["verify_len"].numel() == 0
