"""GPU parity of greedy verification and draft confidence against the oracle.

Bit-exact accepted lengths, next tokens, compacted offsets/tokens and row
tokens; log-sum-exp and confidence within 1e-5 relative."""
import numpy as np
import pytest

import oracle
import synth
from tests.workloads import assert_lse_close, assert_same, cuda_or_skip, host, oracle_of, to_dev, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vsv():
    cuda_or_skip()
    import draft_token_verification_packed_amd as m
    m.lib()
    return m


def run_greedy(vsv, wl, d=None, **kw):
    d = upload(wl) if d is None else d
    out = vsv.verify_greedy(d["logits"], d["offsets"], d["owner"], d["drafts"],
                            relaxed_topk=wl.relaxed_topk, vocab=wl.V, **kw)
    import torch
    torch.cuda.synchronize()
    return out


def test_tiny_greedy_closed_form(vsv):
    wl = synth.make("tiny")
    out = run_greedy(vsv, wl)
    assert host(out["accepted_len"]).tolist() == wl.planted.tolist()
    assert_same(out, oracle_of(wl))


# 4, 16, 32 and 128 requests (20, 80, 160, 640 rows) cut each row into 16,
# 8, 4 and 2 parts
@pytest.mark.parametrize("B", [4, 16, 32, 128])
def test_eagle_greedy_k4(vsv, B):
    wl = synth.make("eagle", B=B)
    assert_same(run_greedy(vsv, wl), oracle_of(wl))


@pytest.mark.parametrize("B", [8, 40, 128])
def test_relaxed_top4_k4(vsv, B):
    wl = synth.make("relaxed", B=B)
    ref = oracle_of(wl)
    assert_same(run_greedy(vsv, wl), ref)
    assert ref["accepted_len"].mean() > 1.0      # the relaxed rule accepts beyond arg-max hits


def _custom(rng, B, Kmax, V, dtype, ld=None, ties=False, pad_nan=True, shift=0):
    Ks = rng.integers(0, Kmax + 1, size=B)
    off = np.zeros(B + 1, dtype=np.int32)
    off[1:] = np.cumsum(Ks + 1)
    R = int(off[-1])
    owner = np.repeat(np.arange(B, dtype=np.int32), Ks + 1)
    ld = V if ld is None else ld
    if ties:
        x = rng.integers(-4, 5, size=(R, V)).astype(np.float32)
        x[rng.random((R, V)) < 0.05] = -0.0
    else:
        x = (rng.standard_normal((R, V)) * 3).astype(np.float32)
    full = np.full((R, ld + shift), np.nan if pad_nan else 0.0, dtype=np.float32)
    full[:, shift:shift + V] = x
    if dtype == oracle.BF16:
        store = synth.f32_to_bf16_bits(full)
    else:
        store = full
    drafts = np.empty(R - B, dtype=np.int32)
    for i in range(B):
        for j in range(int(Ks[i])):
            r = int(off[i]) + j
            xr = oracle.row_f64(store[:, shift:], dtype, r, V)
            drafts[r - i] = int(np.argmax(xr)) if rng.random() < 0.6 else int(rng.integers(0, V))
    return store, off, owner, drafts


@pytest.mark.parametrize("V", [1, 7, 8, 9, 33, 1000, 4099])
@pytest.mark.parametrize("dtype", [oracle.F32, oracle.BF16])
@pytest.mark.parametrize("shift", [0, 1])
def test_ragged_shapes_and_alignment(vsv, V, dtype, shift):
    rng = np.random.default_rng(V * 7 + dtype * 3 + shift)
    store, off, owner, drafts = _custom(rng, 9, 5, V, dtype, ld=V + 3, shift=shift)
    t = to_dev(store)[:, shift:]                    # shift = 1 misaligns every row start
    out = vsv.verify_greedy(t, to_dev(off), to_dev(owner), to_dev(drafts), vocab=V)
    ref = oracle.verify_greedy(store[:, shift:], dtype, V, off, owner, drafts)
    assert_same(out, ref)


@pytest.mark.parametrize("dtype", [oracle.F32, oracle.BF16])
@pytest.mark.parametrize("k", [1, 2, 4, 9])
def test_ties_and_signed_zero(vsv, dtype, k):
    rng = np.random.default_rng(100 + k + dtype)
    store, off, owner, drafts = _custom(rng, 12, 6, 3000, dtype, ties=True)
    out = vsv.verify_greedy(to_dev(store), to_dev(off), to_dev(owner), to_dev(drafts), relaxed_topk=k)
    assert_same(out, oracle.verify_greedy(store, dtype, 3000, off, owner, drafts, relaxed_topk=k))


def test_full_vocab_ragged(vsv):
    rng = np.random.default_rng(5)
    store, off, owner, drafts = _custom(rng, 6, 7, synth.VOCAB, oracle.BF16)
    out = vsv.verify_greedy(to_dev(store), to_dev(off), to_dev(owner), to_dev(drafts))
    assert_same(out, oracle.verify_greedy(store, oracle.BF16, synth.VOCAB, off, owner, drafts))


@pytest.mark.parametrize("B,k", [(1000, 1), (1000, 3), (1800, 1), (1800, 3)])
def test_many_rows(vsv, B, k):
    """About 5 B rows: beyond the 4096 rows the scan stages in LDS, and with
    1800 requests (about 9000 rows) more than 31 rows per CU of a 256-CU part,
    where every row gets a workgroup of its own."""
    rng = np.random.default_rng(B + k)
    store, off, owner, drafts = _custom(rng, B, 8, 640, oracle.BF16)
    assert int(off[-1]) > 4096
    out = vsv.verify_greedy(to_dev(store), to_dev(off), to_dev(owner), to_dev(drafts), relaxed_topk=k)
    assert_same(out, oracle.verify_greedy(store, oracle.BF16, 640, off, owner, drafts, relaxed_topk=k))


def test_single_row_requests_and_empty_batch(vsv):
    import torch
    rng = np.random.default_rng(6)
    store, off, owner, drafts = _custom(rng, 5, 0, 500, oracle.F32)
    out = vsv.verify_greedy(to_dev(store), to_dev(off), to_dev(owner), to_dev(drafts))
    ref = oracle.verify_greedy(store, oracle.F32, 500, off, owner, drafts)
    assert ref["accepted_len"].tolist() == [0] * 5
    assert_same(out, ref)
    empty = torch.zeros((0, 10), dtype=torch.float32, device="cuda")
    o = vsv.verify_greedy(empty, torch.zeros(1, dtype=torch.int32, device="cuda"),
                          torch.zeros(0, dtype=torch.int32, device="cuda"), None)
    torch.cuda.synchronize()
    assert o["accepted_len"].numel() == 0


def test_repeated_calls_reuse_workspace(vsv):
    wl = synth.make("eagle", B=32)
    d = upload(wl)
    a = run_greedy(vsv, wl, d)
    b = run_greedy(vsv, wl, d)
    for k in ("accepted_len", "next_token", "out_offsets", "out_tokens", "row_token", "row_lse"):
        assert np.array_equal(host(a[k]), host(b[k])), k
    assert_same(b, oracle_of(wl))


def test_device_error_flags(vsv):
    rng = np.random.default_rng(8)
    store, off, owner, drafts = _custom(rng, 4, 3, 300, oracle.F32, pad_nan=False)
    drafts2 = drafts.copy()
    drafts2[0] = 300                                 # out of range -> mismatch + flag
    out = vsv.verify_greedy(to_dev(store), to_dev(off), to_dev(owner), to_dev(drafts2))
    assert int(host(out["error_flag"])[0]) & vsv.FLAG_TOKEN
    assert int(host(out["accepted_len"])[0]) == 0
    bad = store.copy()
    bad[1, 7] = np.nan
    out = vsv.verify_greedy(to_dev(bad), to_dev(off), to_dev(owner), to_dev(drafts))
    assert int(host(out["error_flag"])[0]) & vsv.FLAG_LOGITS
    own2 = owner.copy()
    own2[2] = 3
    out = vsv.verify_greedy(to_dev(store), to_dev(off), to_dev(own2), to_dev(drafts))
    assert int(host(out["error_flag"])[0]) & vsv.FLAG_LAYOUT


@pytest.mark.parametrize("B", [8, 128])
def test_relaxed_batch_draft_confidence(vsv, B):
    import torch
    wl = synth.make("relaxed", B=B)
    d = upload(wl)
    conf, lse, flag = vsv.draft_confidence(d["draft_logits"], d["selected"])
    torch.cuda.synchronize()
    rc, rl = oracle.draft_confidence(wl.draft_logits, wl.dtype, wl.V, wl.selected)
    assert_lse_close(host(lse), rl)
    np.testing.assert_allclose(host(conf), rc, rtol=1e-5, atol=0)
    assert int(host(flag)[0]) == 0
    conf2, _, _ = vsv.draft_confidence(d["draft_logits"])
    torch.cuda.synchronize()
    rc2, _ = oracle.draft_confidence(wl.draft_logits, wl.dtype, wl.V)
    np.testing.assert_allclose(host(conf2), rc2, rtol=1e-5, atol=0)


def test_confidence_edge_rows(vsv):
    import torch
    rng = np.random.default_rng(9)
    y = (rng.standard_normal((5, 777)) * 2).astype(np.float32)
    y[0, :] = -np.inf
    y[0, 13] = 1.0                                   # one finite logit: confidence 1
    sel = np.array([13, 0, 776, 800, -1], dtype=np.int32)
    conf, lse, flag = vsv.draft_confidence(to_dev(y), to_dev(sel))
    torch.cuda.synchronize()
    c = host(conf)
    assert c[0] == pytest.approx(1.0, rel=1e-6)
    assert c[3] == 0.0 and c[4] == 0.0
    assert int(host(flag)[0]) & vsv.FLAG_TOKEN
    rc, rl = oracle.draft_confidence(y[:3], oracle.F32, 777, sel[:3])
    np.testing.assert_allclose(c[:3], rc, rtol=1e-5)


@pytest.mark.parametrize("dtype", [oracle.F32, oracle.BF16])
@pytest.mark.parametrize("B", [6, 60, 300])
def test_max_tied_between_head_and_body(vsv, dtype, B):
    """Rows misaligned by one element start with elements outside the 16-byte
    body; the row maximum is planted in one of them and again deep in the
    body, so the lowest index is a head element. 6, 60 and 300 requests cut
    the rows into halves, keep them whole and (bf16) halve them again; the
    sampled entry point with T = 0 streams the same rows as greedy rows."""
    import torch
    rng = np.random.default_rng(600 + B + dtype)
    V = 5000
    store, off, owner, drafts = _custom(rng, B, 4, V, dtype, ld=V + 3, ties=True, pad_nan=False, shift=1)
    top = synth.f32_to_bf16_bits(np.array([5.0], dtype=np.float32))[0] if dtype == oracle.BF16 else np.float32(5.0)
    store[:, 1 + 1] = top            # element 1 of every row: inside the misaligned head
    store[:, 1 + 3000] = top         # and the same value in the body
    R = int(off[-1])
    print("head tie B=%d R=%d dtype=%d" % (B, R, dtype), flush=True)
    t = to_dev(store)[:, 1:]
    out = vsv.verify_greedy(t, to_dev(off), to_dev(owner), to_dev(drafts), vocab=V)
    torch.cuda.synchronize()
    ref = oracle.verify_greedy(store[:, 1:], dtype, V, off, owner, drafts)
    assert (ref["row_token"] == 1).all()
    assert_same(out, ref)
    z = torch.zeros(B, dtype=torch.float32, device="cuda")
    s = vsv.verify_sampled(t, to_dev(off), to_dev(owner), to_dev(drafts), z, torch.zeros(B, dtype=torch.int32,
                           device="cuda"), torch.ones(B, device="cuda"), z, 1, vocab=V)
    torch.cuda.synchronize()
    assert_same(s, ref)


@pytest.mark.parametrize("dtype", [oracle.F32, oracle.BF16])
@pytest.mark.parametrize("B", [1, 3, 24])
def test_many_parts_ties_across_parts(vsv, dtype, B):
    """Small batches over a 152064-token vocabulary cut each row into up to
    16 parts; rows are misaligned by one element, so each has head and tail
    elements outside its 16-byte body. The row maximum is planted by rows in
    turn: twice in distant parts (the lower index must win the merge), once
    at the very last element (a tail element), at the first and the last
    element, and as a run of 81 equal values across the middle part boundary
    for every even part count. Drafts alternate, from one round of the four
    plantings to the next, between the lowest tied index and the highest (a
    tie that is not the greedy token is rejected)."""
    import torch
    rng = np.random.default_rng(7700 + B + dtype)
    V, shift = 152064, 1
    store, off, owner, _ = _custom_quick(rng, B, 6, V, dtype, ld=V + 3, shift=shift)
    R = int(off[-1])
    top = synth.f32_to_bf16_bits(np.array([40.0], dtype=np.float32))[0] if dtype == oracle.BF16 else np.float32(40.0)
    mid = V // 2
    plants = [[V // 3, 2 * V // 3], [V - 1], [0, V - 1], list(range(mid - 40, mid + 41))]
    chosen = []
    for r in range(R):
        idx = plants[r % len(plants)]
        store[r, shift + np.array(idx)] = top
        chosen.append(idx)
    drafts = np.empty(R - B, dtype=np.int32)
    for i in range(B):
        for j in range(int(off[i + 1] - off[i]) - 1):
            r = int(off[i]) + j
            idx = chosen[r]
            drafts[r - i] = idx[0] if (r // len(plants)) % 2 == 0 else idx[-1]
    print("many parts B=%d R=%d dtype=%d" % (B, R, dtype), flush=True)
    t = to_dev(store)[:, shift:]
    out = vsv.verify_greedy(t, to_dev(off), to_dev(owner), to_dev(drafts), vocab=V)
    torch.cuda.synchronize()
    ref = oracle.verify_greedy(store[:, shift:], dtype, V, off, owner, drafts)
    assert ref["row_token"].tolist() == [c[0] for c in chosen]
    assert_same(out, ref)


def _custom_quick(rng, B, Kmax, V, dtype, ld, shift):
    """A ragged batch of normal(0, 3) logits (drafts left to the caller)."""
    Ks = rng.integers(0, Kmax + 1, size=B)
    off = np.zeros(B + 1, dtype=np.int32)
    off[1:] = np.cumsum(Ks + 1)
    R = int(off[-1])
    owner = np.repeat(np.arange(B, dtype=np.int32), Ks + 1)
    full = np.zeros((R, ld + shift), dtype=np.float32)
    full[:, shift:shift + V] = (rng.standard_normal((R, V)) * 3).astype(np.float32)
    store = synth.f32_to_bf16_bits(full) if dtype == oracle.BF16 else full
    return store, off, owner, None
