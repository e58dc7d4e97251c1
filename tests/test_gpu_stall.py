"""The batch scan's bounded wait. A dedicated GPU never reaches it, so the
host withholds one row's result word through the library's test hook: the
kernels still exit normally, the scan waits out its poll budget and flags
VSV_FLAG_STALLED. Checked: the flag, outputs that stay inside their buffers
and agree with the oracle wherever the withheld word plays no part, and a
next call on the same workspace that is exact again."""
import numpy as np
import pytest

import synth
from tests.workloads import assert_same, cuda_or_skip, host, oracle_of, upload, with_margins

pytestmark = pytest.mark.gpu

FLAG_STALLED = 16


@pytest.fixture(scope="module")
def vsv():
    cuda_or_skip()
    import draft_token_verification_packed_amd as m
    m.lib()
    yield m
    m.withhold_row_word(-1)


def check_stalled(out, ref, wl, row):
    """Flag set; every write inside its buffer; requests that do not own
    `row` exact; row outputs (written before the word) exact."""
    assert int(host(out["error_flag"])[0]) & FLAG_STALLED
    B, R = wl.B, wl.R
    acc = host(out["accepted_len"])
    offs = host(out["out_offsets"])
    toks = host(out["out_tokens"])
    K = np.diff(wl.offsets) - 1
    assert np.all((acc >= 0) & (acc <= K))
    assert offs[0] == 0 and np.array_equal(np.diff(offs), acc + 1) and offs[-1] <= R
    assert np.all(toks[offs[-1]:] == -1), "a write past the emitted tokens"
    assert np.array_equal(host(out["row_token"]), ref["row_token"])
    owner = int(wl.owner[row])
    keep = np.arange(B) != owner
    assert np.array_equal(acc[keep], ref["accepted_len"][keep])
    assert np.array_equal(host(out["next_token"])[keep], ref["next_token"][keep])
    for i in np.flatnonzero(keep):
        assert np.array_equal(toks[offs[i]:offs[i + 1]], ref["out_tokens"][ref["out_offsets"][i]:ref["out_offsets"][i + 1]])


def test_greedy_row_kernel_stall_then_recovers(vsv):
    import torch
    wl = synth.make("eagle", B=64)   # 320 rows: the row-per-workgroup kernel
    d = upload(wl)
    ref = oracle_of(wl)
    ws = vsv.workspace(wl.B, wl.R, False, d["logits"].device)
    row = 123
    print("greedy stall: B=%d R=%d withheld row %d" % (wl.B, wl.R, row), flush=True)
    try:
        vsv.withhold_row_word(row)
        out = vsv.verify_greedy(d["logits"], d["offsets"], d["owner"], d["drafts"], vocab=wl.V, ws=ws)
        torch.cuda.synchronize()
    finally:
        vsv.withhold_row_word(-1)
    check_stalled(out, ref, wl, row)
    again = vsv.verify_greedy(d["logits"], d["offsets"], d["owner"], d["drafts"], vocab=wl.V, ws=ws)
    torch.cuda.synchronize()
    assert_same(again, ref)


def test_sampled_stall_then_recovers(vsv):
    import torch
    wl = with_margins(synth.make("mixed", B=12))
    d = upload(wl)
    ref = oracle_of(wl)
    ws = vsv.workspace(wl.B, wl.R, True, d["logits"].device)
    row = wl.R - 2
    print("sampled stall: B=%d R=%d withheld row %d" % (wl.B, wl.R, row), flush=True)

    def call():
        return vsv.verify_sampled(d["logits"], d["offsets"], d["owner"], d["drafts"], d["temperature"], d["top_k"],
                                  d["top_p"], d["min_p"], wl.seed, wl.offset, vocab=wl.V, ws=ws)
    try:
        vsv.withhold_row_word(row)
        out = call()
        torch.cuda.synchronize()
    finally:
        vsv.withhold_row_word(-1)
    check_stalled(out, ref, wl, row)
    again = call()
    torch.cuda.synchronize()
    assert_same(again, ref)

