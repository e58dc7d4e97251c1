"""GPU parity of the relaxed acceptance variants (vsv_verify_greedy_relaxed)
against the oracle (oracle.verify_greedy_relaxed): the confidence-accept
margin, the from-position and after-tokens gates (per-request generated
counts), protected token ids, and top-K combined with them. Bit-exact
accepted lengths, next tokens, compacted outputs and row tokens; log-sum-exp
within 1e-5 relative."""
import numpy as np
import pytest

import oracle
import synth
from tests.workloads import assert_same, cuda_or_skip, host, to_dev, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vsv():
    cuda_or_skip()
    import draft_token_verification_packed_amd as m
    m.lib()
    return m


def _protected(rng, wl, n, from_argmax):
    """n token ids: some of them rows' greedy tokens or drafts, the rest random."""
    ids = set(int(t) for t in rng.integers(0, wl.V, size=max(0, n - 2 * from_argmax)))
    rows = rng.choice(wl.R, size=from_argmax, replace=False)
    for r in rows:
        ids.add(oracle.greedy_token(oracle.row_f64(wl.logits, wl.dtype, int(r), wl.V)))
    for q in rng.choice(max(1, wl.R - wl.B), size=from_argmax, replace=False):
        if wl.R > wl.B:
            ids.add(int(wl.drafts[int(q)]))
    return np.array(sorted(ids)[:n], dtype=np.int32)


def _run(vsv, wl, d, **kw):
    import torch
    dev = dict(kw)
    if dev.get("generated") is not None:
        dev["generated"] = to_dev(np.asarray(dev["generated"], dtype=np.int32))
    if dev.get("protected") is not None:
        dev["protected_ids"] = to_dev(np.asarray(dev.pop("protected"), dtype=np.int32))
    else:
        dev.pop("protected", None)
    out = vsv.verify_greedy_relaxed(d["logits"], d["offsets"], d["owner"], d["drafts"], vocab=wl.V, **dev)
    torch.cuda.synchronize()
    return out


def _oracle(wl, **kw):
    return oracle.verify_greedy_relaxed(wl.logits, wl.dtype, wl.V, wl.offsets, wl.owner, wl.drafts, **kw)


CASES = [
    dict(margin=5.25),
    dict(margin=5.25, from_position=1),
    dict(margin=1.5, after_tokens=6, generated="random"),
    dict(margin=5.25, protected=40),
    dict(topk=4, after_tokens=3, generated="random", protected=30),
    dict(topk=4, margin=0.75, from_position=2),
    dict(topk=1, margin=0.0, from_position=0),          # strict through the relaxed entry point
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_relaxed_variants_full_c4_shape(vsv, case):
    """The relaxed top-4 batch shape (B=128, K=4, V=152064 bf16)."""
    wl = synth.make("relaxed")
    d = upload(wl)
    rng = np.random.default_rng(9000 + case)
    kw = dict(CASES[case])
    if kw.get("generated") == "random":
        kw["generated"] = rng.integers(0, 9, size=wl.B).astype(np.int32)
    if "protected" in kw:
        kw["protected"] = _protected(rng, wl, kw["protected"], 8)
    print("relaxed case %d: %s" % (case, {k: (v if np.isscalar(v) else "array") for k, v in kw.items()}), flush=True)
    out = _run(vsv, wl, d, **kw)
    ref = _oracle(wl, **kw)
    assert_same(out, ref)
    if case == len(CASES) - 1:
        strict = oracle.verify_greedy(wl.logits, wl.dtype, wl.V, wl.offsets, wl.owner, wl.drafts)
        assert np.array_equal(ref["accepted_len"], strict["accepted_len"])


@pytest.mark.parametrize("B", [6, 40, 300])
def test_relaxed_margin_ties_and_shapes(vsv, B):
    """Integer-valued fp32 rows (many ties, and gaps equal to the margin
    exactly, which must be rejected on both sides), misaligned rows, drafts
    near the top; 6 and 300 requests cut each row in two, 40 keep rows
    whole."""
    rng = np.random.default_rng(9100 + B)
    V, ld, shift = 3001, 3010, 1
    Ks = rng.integers(0, 6, size=B)
    off = np.zeros(B + 1, dtype=np.int32)
    off[1:] = np.cumsum(Ks + 1)
    R = int(off[-1])
    owner = np.repeat(np.arange(B, dtype=np.int32), Ks + 1)
    store = np.zeros((R, ld + shift), dtype=np.float32)
    x = (rng.integers(-12, 13, size=(R, V)) * 0.25).astype(np.float32)
    store[:, shift:shift + V] = x
    drafts = np.zeros(R - B, dtype=np.int32)
    for i in range(B):
        for j in range(int(Ks[i])):
            r = int(off[i]) + j
            top = np.argsort(-x[r], kind="stable")[:12]
            drafts[r - i] = int(rng.choice(top))
    gen = rng.integers(0, 5, size=B).astype(np.int32)
    prot = np.array(sorted(set(int(t) for t in rng.integers(0, V, size=60))), dtype=np.int32)
    t = to_dev(store)[:, shift:]
    dev = dict(logits=t, offsets=to_dev(off), owner=to_dev(owner), drafts=to_dev(drafts))
    for kw in (dict(margin=0.5), dict(margin=0.75, from_position=1, after_tokens=3, generated=gen, protected=prot),
               dict(topk=3, margin=0.25, protected=prot)):
        print("relaxed ties B=%d: %s" % (B, sorted(kw)), flush=True)
        out = _run(vsv, synth_shape(V), dev, **kw)
        ref = oracle.verify_greedy_relaxed(store[:, shift:], oracle.F32, V, off, owner, drafts, **kw)
        assert_same(out, ref)


def synth_shape(V):
    class _S:
        pass
    s = _S()
    s.V = V
    return s


def test_relaxed_flags_and_empty(vsv):
    import torch
    wl = synth.make("tiny")
    drafts = wl.drafts.copy()
    drafts[0] = wl.V + 3                                   # out of range: mismatch and flag
    d = upload(wl)
    d["drafts"] = to_dev(drafts)
    out = _run(vsv, wl, d, margin=100.0)
    assert int(host(out["error_flag"])[0]) & vsv.FLAG_TOKEN
    assert int(host(out["accepted_len"])[0]) == 0
    e = torch.zeros(0, 16, dtype=torch.float32, device="cuda")
    z = torch.zeros(1, dtype=torch.int32, device="cuda")
    ei = torch.zeros(0, dtype=torch.int32, device="cuda")
    out = vsv.verify_greedy_relaxed(e, z, ei, ei, margin=1.0, vocab=16)
    torch.cuda.synchronize()
    assert int(host(out["error_flag"])[0]) == 0
