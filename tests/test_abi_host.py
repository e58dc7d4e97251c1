"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point the header declares, and rejects bad arguments with a
status before anything is enqueued."""
import ctypes
import os
import re

import pytest

import draft_token_verification_packed_amd as vsv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vspec_verify.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(vsv.LIB_PATH):
        pytest.skip("library not built (run the package build first)")
    return vsv.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(vsv_\w+)\s*\(", text, re.M)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert set(vsv.SYMBOLS) <= set(names)
    assert {"vsv_verify_greedy", "vsv_verify_sampled", "vsv_draft_confidence"} <= set(names)


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings_and_version(L):
    assert L.vsv_status_string(0) == b"ok"
    for s in range(1, 6):
        assert len(L.vsv_status_string(s)) > 3
    assert L.vsv_version() >= 100


def test_workspace_bytes(L):
    assert L.vsv_workspace_bytes(0, 0, 0) >= 256
    b = L.vsv_workspace_bytes(128, 640, 0)
    assert b % 256 == 0 and b >= 640 * 4
    assert L.vsv_workspace_bytes(-1, 5, 0) == 0
    assert L.vsv_workspace_bytes(128, 640, 1) >= b


def _batch(**kw):
    b = dict(logits=0x10000, dtype=1, vocab=1024, ld=1024, num_requests=4, num_rows=20,
             row_offsets=0x20000, row_owner=0x30000, draft_tokens=0x40000)
    b.update(kw)
    return vsv.Batch(**b)


def _outs(**kw):
    o = dict(accepted_len=0x50000, next_token=0x60000, out_offsets=0x70000, out_tokens=0x80000,
             row_token=None, row_lse=None, error_flag=None)
    o.update(kw)
    return vsv.Outputs(**o)


def _greedy(L, batch, outs, ws=0x100000, ws_bytes=1 << 20, k=1):
    return L.vsv_verify_greedy(ctypes.byref(batch) if batch is not None else None, k,
                               ctypes.byref(outs) if outs is not None else None,
                               ctypes.c_void_p(ws) if ws else None, ws_bytes, None)


@pytest.mark.parametrize("bad", [
    dict(logits=None), dict(dtype=7), dict(vocab=0), dict(ld=1000), dict(num_rows=3),
    dict(num_requests=-1), dict(row_offsets=None), dict(row_owner=None), dict(draft_tokens=None),
    dict(logits=0x10001), dict(dtype=0, logits=0x10002), dict(num_requests=0, num_rows=5),
    # a row of 2 GiB or more (fp32 and bf16)
    dict(dtype=0, vocab=1 << 29, ld=1 << 29), dict(vocab=(1 << 30) - 1, ld=(1 << 30) - 1),
])
def test_invalid_batch_is_rejected_before_launch(L, bad):
    assert _greedy(L, _batch(**bad), _outs()) == 1


@pytest.mark.parametrize("bad", [dict(accepted_len=None), dict(next_token=None), dict(out_offsets=None),
                                 dict(out_tokens=None)])
def test_missing_required_output_is_rejected(L, bad):
    assert _greedy(L, _batch(), _outs(**bad)) == 1


def test_null_structs_and_workspace_errors(L):
    assert _greedy(L, None, _outs()) == 1
    assert _greedy(L, _batch(), None) == 1
    assert _greedy(L, _batch(), _outs(), ws=0) == 3
    assert _greedy(L, _batch(), _outs(), ws=0x100010) == 3       # misaligned
    assert _greedy(L, _batch(), _outs(), ws_bytes=64) == 3       # too small


def test_relaxed_topk_range(L):
    assert _greedy(L, _batch(), _outs(), k=0) == 1
    assert _greedy(L, _batch(), _outs(), k=1025) == 1


def test_empty_batch_is_a_noop(L):
    assert _greedy(L, _batch(num_requests=0, num_rows=0), _outs(), ws=0, ws_bytes=0) == 0 or \
        _greedy(L, _batch(num_requests=0, num_rows=0), _outs()) == 0
    assert _greedy(L, _batch(num_requests=0, num_rows=0, logits=None), _outs()) == 0


def test_sampled_rejects_missing_parameters(L):
    b, o = _batch(), _outs()
    st = L.vsv_verify_sampled(ctypes.byref(b), None, ctypes.c_void_p(8), ctypes.c_void_p(8),
                              ctypes.c_void_p(8), 1, 0, ctypes.byref(o), ctypes.c_void_p(0x100000), 1 << 20, None)
    assert st == 1


def _prob(L, b, o, draft=0x200000, dld=1024, params=(8, 8, 8, 8, 8)):
    return L.vsv_verify_probabilistic(ctypes.byref(b), ctypes.c_void_p(draft) if draft else None, dld,
                                      *[ctypes.c_void_p(p) if p else None for p in params], 1, 0, ctypes.byref(o),
                                      ctypes.c_void_p(0x100000), 1 << 20, None)


def test_probabilistic_validation(L):
    b, o = _batch(), _outs()
    for k in range(5):                                   # each parameter array, draft temperature last
        params = [8] * 5
        params[k] = 0
        assert _prob(L, b, o, params=params) == 1
    assert _prob(L, b, o, draft=0) == 1                  # draft rows needed when R > B
    assert _prob(L, b, o, draft=0x200001) == 1           # misaligned bf16 rows
    assert _prob(L, b, o, dld=1000) == 1                 # draft_ld < vocab
    assert _prob(L, _batch(), _outs(out_tokens=None)) == 1
    assert _prob(L, _batch(num_requests=0, num_rows=0), o, draft=0, params=(0, 0, 0, 0, 0)) == 0


def test_confidence_validation(L):
    f = L.vsv_draft_confidence
    assert f(ctypes.c_void_p(0x10000), 1, 100, 100, 0, None, None, None, None, None) == 0   # D = 0: no-op
    assert f(ctypes.c_void_p(0x10000), 1, 100, 100, -1, None, ctypes.c_void_p(8), None, None, None) == 1
    assert f(None, 1, 100, 100, 4, None, ctypes.c_void_p(8), None, None, None) == 1
    assert f(ctypes.c_void_p(0x10000), 1, 100, 99, 4, None, ctypes.c_void_p(8), None, None, None) == 1
    assert f(ctypes.c_void_p(0x10000), 1, 100, 100, 4, None, None, None, None, None) == 1
    assert f(ctypes.c_void_p(0x10000), 3, 100, 100, 4, None, ctypes.c_void_p(8), None, None, None) == 1
    assert f(ctypes.c_void_p(0x10001), 1, 100, 100, 4, None, ctypes.c_void_p(8), None, None, None) == 1


def test_workspace_init_validation(L):
    assert L.vsv_workspace_init(None, 256, None) == 1
    assert L.vsv_workspace_init(ctypes.c_void_p(0x1000), 6, None) == 1


def test_allocate_validation(L):
    f = L.vsv_allocate_verify
    p = ctypes.c_void_p(0x1000)

    def call(B, K, G, conf=p, drafts=None, vl=p, off=p, own=p, packed=None):
        return f(conf, drafts, B, K, G, vl, off, own, None, packed, None, None)

    assert call(0, 4, 0) == 0                      # empty batch: no-op
    assert call(0, 4, 1) == 1                      # G outside [B, B * (K + 1)]
    assert call(3, 4, 2) == 1 and call(3, 4, 16) == 1
    assert call(-1, 4, 0) == 1 and call(3, -1, 3) == 1
    assert call(8193, 1, 8193) == 1                # more requests than one workgroup holds
    assert call(2049, 8, 2049) == 1                # more positions than one workgroup holds
    assert call(3, 4, 5, conf=None) == 1           # scores needed when K > 0
    assert call(3, 4, 5, vl=None) == 1 and call(3, 4, 5, off=None) == 1 and call(3, 4, 5, own=None) == 1
    assert call(3, 4, 5, drafts=p) == 1            # drafts without packed output
    assert call(3, 4, 5, packed=p) == 1            # packed output without drafts


def test_static_entry_point_rejects_batches_beyond_its_scratch(L):
    """The entry point that allocates nothing refuses, before any HIP call,
    a batch larger than its fixed scratch serves (and a missing batch)."""
    out = vsv.Outputs(0x50000, 0x60000, 0x70000, 0x80000, None, None, None, None)
    R = vsv.STATIC_MAX_ROWS + 1
    b = _batch(num_requests=1, num_rows=R)
    assert L.vsv_verify_greedy_static(ctypes.byref(b), 1, ctypes.byref(out), None) == vsv.VSV_ELIMIT
    assert L.vsv_verify_greedy_static(None, 1, ctypes.byref(out), None) == 1
    text = open(HEADER).read()
    assert "#define VSV_STATIC_MAX_ROWS %d" % vsv.STATIC_MAX_ROWS in text


def test_relaxed_validation(L):
    """vsv_verify_greedy_relaxed refuses bad relaxation arguments before any
    launch (the batch itself is valid, with dummy pointers)."""
    ws = 0x100000
    out = vsv.Outputs(0x50000, 0x60000, 0x70000, 0x80000, None, None, None, None)
    b = _batch()
    nbytes = L.vsv_workspace_bytes(4, 20, 0)

    def call(**kw):
        r = dict(topk=1, margin=0.0, from_position=0, after_tokens=0, generated=None, protected_ids=None,
                 num_protected=0)
        r.update(kw)
        return L.vsv_verify_greedy_relaxed(ctypes.byref(b), ctypes.byref(vsv.Relax(**r)), ctypes.byref(out), ws,
                                           nbytes, None)
    assert L.vsv_verify_greedy_relaxed(ctypes.byref(b), None, ctypes.byref(out), ws, nbytes, None) == 1
    assert call(topk=0) == 1 and call(topk=1025) == 1
    assert call(margin=-1.0) == 1 and call(margin=float("nan")) == 1 and call(margin=float("inf")) == 1
    assert call(from_position=-1) == 1 and call(after_tokens=-2) == 1
    assert call(num_protected=vsv.MAX_PROTECTED + 1, protected_ids=0x90000) == 1
    assert call(num_protected=3) == 1                    # ids missing
    assert "#define VSV_MAX_PROTECTED %d" % vsv.MAX_PROTECTED in open(HEADER).read()


def test_withhold_hook_validation(L):
    assert L.vsv_test_withhold_row_word(-2) == 1
    assert L.vsv_test_withhold_row_word(5) == 0
    assert L.vsv_test_withhold_row_word(-1) == 0
    with pytest.raises(vsv.VSVError):
        vsv.withhold_row_word(-3)
