"""Calls issued on a stream that is not the current one: the binding must
allocate and zero the workspace and the outputs on that stream (so the
fills are ordered before the kernels) and mark the inputs as used there.
Results are compared with the oracle after synchronising that stream only."""
import pytest

import synth
from tests.workloads import assert_same, cuda_or_skip, oracle_of, upload, with_margins

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vsv():
    cuda_or_skip()
    import draft_token_verification_packed_amd as m
    m.lib()
    return m


def test_greedy_and_sampled_on_a_side_stream(vsv):
    import torch
    s = torch.cuda.Stream()
    g = synth.make("eagle", B=24)
    m = with_margins(synth.make("mixed", B=12))
    dg, dm = upload(g), upload(m)
    torch.cuda.synchronize()
    # a fresh cache entry: the side stream has not been used before
    vsv._ws_cache.clear()
    print("side stream: greedy R=%d, sampled R=%d" % (g.R, m.R), flush=True)
    og = vsv.verify_greedy(dg["logits"], dg["offsets"], dg["owner"], dg["drafts"], vocab=g.V, stream=s)
    om = vsv.verify_sampled(dm["logits"], dm["offsets"], dm["owner"], dm["drafts"], dm["temperature"],
                            dm["top_k"], dm["top_p"], dm["min_p"], m.seed, m.offset, vocab=m.V, stream=s)
    # the current stream keeps working meanwhile; nothing here waits for it
    busy = torch.randn(4096, 4096, device="cuda") @ torch.randn(4096, 4096, device="cuda")
    s.synchronize()
    assert_same(og, oracle_of(g))
    assert_same(om, oracle_of(m))
    ws = vsv._ws_cache[(torch.cuda.current_device(), s.cuda_stream)]
    assert ws.numel() >= vsv.workspace_bytes(m.B, m.R, True)
    del busy


def test_second_call_on_side_stream_grows_workspace(vsv):
    import torch
    s = torch.cuda.Stream()
    vsv._ws_cache.clear()
    small, big = synth.make("tiny"), synth.make("eagle", B=64)
    for wl in (small, big, small):
        d = upload(wl)
        out = vsv.verify_greedy(d["logits"], d["offsets"], d["owner"], d["drafts"], vocab=wl.V, stream=s)
        del d   # inputs freed while the side stream may still read them
        s.synchronize()
        assert_same(out, oracle_of(wl))
