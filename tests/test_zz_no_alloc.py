"""The entry point that allocates nothing (vsv_verify_greedy_static, which
uses a library-owned scratch array per GPU instead of a caller workspace)
against the workspace entry point vsv_verify_greedy on the same inputs, and
both against the oracle: two calls in a row on the shared array, the second
on a smaller batch, so the second call runs on what the first left behind."""
import numpy as np
import pytest

import synth
from tests.workloads import assert_same, cuda_or_skip, host, oracle_of, upload

pytestmark = pytest.mark.gpu

KEYS = ("accepted_len", "next_token", "out_offsets", "out_tokens", "row_token", "row_lse", "error_flag")


@pytest.fixture(scope="module")
def vsv():
    cuda_or_skip()
    import draft_token_verification_packed_amd as m
    m.lib()
    return m


def _both(vsv, wl, relaxed=1):
    import torch
    d = upload(wl)
    print("static scratch: %s B=%d R=%d relaxed=%d" % (wl.key, wl.B, wl.R, relaxed), flush=True)
    ref = vsv.verify_greedy(d["logits"], d["offsets"], d["owner"], d["drafts"], relaxed_topk=relaxed, vocab=wl.V)
    got = vsv.verify_greedy_static(d["logits"], d["offsets"], d["owner"], d["drafts"], relaxed_topk=relaxed,
                                   vocab=wl.V)
    torch.cuda.synchronize()
    total = int(host(ref["out_offsets"])[-1])
    for k in KEYS:
        a, b = host(got[k]), host(ref[k])
        if k == "out_tokens":
            a, b = a[:total], b[:total]
        assert np.array_equal(a, b), k
    return got


def test_static_scratch_two_calls(vsv):
    # first call: 200 rows in three parts each (the parts' statistics in
    # the scratch); second: 20 rows, one workgroup per half row
    wl = synth.make("eagle", B=40)
    assert_same(_both(vsv, wl), oracle_of(wl))
    small = synth.make("tiny")
    assert_same(_both(vsv, small), oracle_of(small))


def test_static_scratch_relaxed_then_smaller(vsv):
    wl = synth.make("relaxed", B=64)
    wl.relaxed_topk = 4
    assert_same(_both(vsv, wl, relaxed=4), oracle_of(wl))
    small = synth.make("relaxed", B=8, V=4099)
    small.relaxed_topk = 4
    assert_same(_both(vsv, small, relaxed=4), oracle_of(small))


def test_static_scratch_limit(vsv):
    import torch
    R = vsv.STATIC_MAX_ROWS + 1
    logits = torch.zeros(R, 16, dtype=torch.float32, device="cuda")
    off = torch.tensor([0, R], dtype=torch.int32, device="cuda")
    owner = torch.zeros(R, dtype=torch.int32, device="cuda")
    drafts = torch.zeros(R - 1, dtype=torch.int32, device="cuda")
    with pytest.raises(vsv.VSVError) as e:
        vsv.verify_greedy_static(logits, off, owner, drafts)
    assert e.value.status == vsv.VSV_ELIMIT
