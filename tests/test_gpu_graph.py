"""The entry points inside a captured HIP graph.

The calls allocate nothing and record no memset, and the words handed
between workgroups carry a tag derived from the workspace's call counter on
the device, so a captured call can be replayed: each replay is a new call.
A greedy call, a sampled call and the allocation-free greedy call are
captured together on a side stream, then replayed several times; between
replays the outputs are overwritten and the same calls run eagerly (which
advances the workspaces' counters), and every replay is checked against
the eager results and the oracle."""
import numpy as np
import pytest

import synth
from tests.workloads import assert_same, cuda_or_skip, host, oracle_of, upload, with_margins

pytestmark = pytest.mark.gpu

KEYS = ("accepted_len", "next_token", "out_offsets", "out_tokens", "row_token", "row_lse")


@pytest.fixture(scope="module")
def vsv():
    cuda_or_skip()
    import draft_token_verification_packed_amd as m
    m.lib()
    return m


def test_calls_replay_in_a_captured_graph(vsv):
    import torch
    wg = synth.make("eagle", B=8)
    ws_ = with_margins(synth.make("mixed", B=4))
    wt = synth.make("tiny")
    dg, ds, dt = upload(wg), upload(ws_), upload(wt)
    refs = [oracle_of(wg), oracle_of(ws_), oracle_of(wt)]
    dev = dg["logits"].device
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        wsg = vsv.workspace(wg.B, wg.R, False, dev, stream=s)
        wss = vsv.workspace(ws_.B, ws_.R, True, dev, stream=s)
        cg, og = vsv.prepare_greedy(dg["logits"], dg["offsets"], dg["owner"], dg["drafts"], ws=wsg, stream=s)
        cs, os_ = vsv.prepare_sampled(ds["logits"], ds["offsets"], ds["owner"], ds["drafts"], ds["temperature"],
                                      ds["top_k"], ds["top_p"], ds["min_p"], ws_.seed, ws_.offset, ws=wss, stream=s)
        ot = vsv.verify_greedy_static(dt["logits"], dt["offsets"], dt["owner"], dt["drafts"], stream=s)
        cg.run()
        cs.run()
    torch.cuda.synchronize()
    outs = [og, os_, ot]
    eager = [{k: o[k].clone() for k in KEYS} for o in outs]
    for o, ref in zip(outs, refs):
        assert_same(o, ref)
    print("graph: capturing greedy B=%d, sampled B=%d, static B=%d" % (wg.B, ws_.B, wt.B), flush=True)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        cg.run()
        cs.run()
        vsv.verify_greedy_static(dt["logits"], dt["offsets"], dt["owner"], dt["drafts"], out=ot, stream=s)
    for rep in range(4):
        for o in outs:
            for k in KEYS:
                o[k].fill_(-7)
            o["error_flag"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e, ref in zip(outs, eager, refs):
            n = int(host(e["out_offsets"])[-1])
            for k in KEYS:
                got, want = host(o[k]), host(e[k])
                if k == "out_tokens":
                    # only the emitted tokens are written; the rest keeps what it held
                    assert np.all(got[n:] == -7), "replay %d: a write past the emitted tokens" % rep
                    got, want = got[:n], want[:n]
                assert np.array_equal(got, want), "replay %d: %s differs" % (rep, k)
            assert int(host(o["error_flag"])[0]) == 0
            assert_same(o, ref)
        # eager calls between replays, on the same workspaces
        with torch.cuda.stream(s):
            cg.run()
            cs.run()
        torch.cuda.synchronize()
        assert_same(og, refs[0])
        assert_same(os_, refs[1])
    del g
