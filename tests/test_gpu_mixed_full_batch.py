"""The whole large mixed batch (B=512, K=7, V=152064 bf16: 4096 verify rows,
3584 draft rows) on the GPU, every output compared with the oracle's.

The oracle's outputs are stored in tests/golden/mixed_b512_k7_v152064.npz by
tests/golden/make_mixed_golden.py, which calls only the oracle and the input
generator (a whole-batch oracle pass takes minutes). The inputs are rebuilt
here from the same recipe with the recorded re-draws and checked against the
recorded fingerprint, so the comparison is on exactly the batch the oracle
saw. At 4096 rows the sampled launch takes its plain row-queue order (more
than two rows per workgroup slot)."""
import os

import numpy as np
import pytest

import synth
from tests.workloads import assert_lse_close, cuda_or_skip, host, to_dev

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "mixed_b512_k7_v152064.npz")


@pytest.fixture(scope="module")
def vsv():
    cuda_or_skip()
    import draft_token_verification_packed_amd as m
    m.lib()
    return m


@pytest.fixture(scope="module")
def batch():
    from tests.golden.make_mixed_golden import fingerprint
    g = dict(np.load(GOLDEN, allow_pickle=False))
    attempts = dict(zip(g["attempt_rows"].tolist(), g["attempt_counts"].tolist()))
    wl = synth.make("mixed", attempts=attempts)
    assert fingerprint(wl) == str(g["fingerprint"]), "inputs differ from the ones the oracle saw"
    print("mixed batch rebuilt: %d re-drawn rows" % len(attempts), flush=True)
    d = dict(logits=to_dev(wl.logits), offsets=to_dev(wl.offsets), owner=to_dev(wl.owner),
             drafts=to_dev(wl.drafts), temperature=to_dev(wl.temperature), top_k=to_dev(wl.top_k),
             top_p=to_dev(wl.top_p), min_p=to_dev(wl.min_p), draft_logits=to_dev(wl.draft_logits),
             selected=to_dev(wl.selected))
    return wl, d, g


def _compare(out, g, prefix, lse=True):
    for k in ("accepted_len", "next_token", "out_offsets", "row_token"):
        got, want = host(out[k]), g[prefix + k]
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, "%s differs at %s (%d entries)" % (k, bad[:10], bad.size)
    total = int(g[prefix + "out_offsets"][-1])
    assert np.array_equal(host(out["out_tokens"])[:total], g[prefix + "out_tokens"])
    if lse:
        assert_lse_close(host(out["row_lse"]), g[prefix + "row_lse"])
    assert int(host(out["error_flag"])[0]) == 0


def test_mixed_full_batch_sampled(vsv, batch):
    import torch
    wl, d, g = batch
    print("verify_sampled on the whole mixed batch", flush=True)
    out = vsv.verify_sampled(d["logits"], d["offsets"], d["owner"], d["drafts"], d["temperature"], d["top_k"],
                             d["top_p"], d["min_p"], wl.seed, wl.offset, vocab=wl.V)
    torch.cuda.synchronize()
    _compare(out, g, "s_")


def test_mixed_full_batch_confidence(vsv, batch):
    import torch
    wl, d, g = batch
    print("draft_confidence on the whole mixed batch", flush=True)
    conf, lse, flag = vsv.draft_confidence(d["draft_logits"], d["selected"], vocab=wl.V)
    torch.cuda.synchronize()
    assert_lse_close(host(lse), g["c_lse"])
    c, want = host(conf).astype(np.float64), g["c_confidence"]
    bad = np.flatnonzero(~(np.abs(c - want) <= 1e-5 * want))
    assert bad.size == 0, "confidence differs at %s: %s vs %s" % (bad[:5], c[bad[:5]], want[bad[:5]])
    assert int(host(flag)[0]) == 0


def test_mixed_full_batch_probabilistic(vsv, batch):
    import torch
    wl, d, g = batch
    print("verify_probabilistic on the whole mixed batch", flush=True)
    out = vsv.verify_probabilistic(d["logits"], d["offsets"], d["owner"], d["drafts"], d["draft_logits"],
                                   d["temperature"], d["top_k"], d["top_p"], d["min_p"], d["temperature"],
                                   wl.seed, wl.offset, vocab=wl.V)
    torch.cuda.synchronize()
    _compare(out, g, "p_", lse=False)
