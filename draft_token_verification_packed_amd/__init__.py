"""Packed draft-token verification on MI355X: Python binding of libvspec_verify.

Argument marshalling only. Every step of verification runs in the HIP
kernels of `libvspec_verify.so` (built in-tree by `build.py`); PyTorch is used
for device memory and the current stream. There is no CPU fallback: if the
library is missing or cannot be loaded, every call raises.

Entry points mirror the C ABI in include/vspec_verify.h:
    verify_greedy(logits, row_offsets, row_owner, draft_tokens, relaxed_topk=1)
    verify_greedy_relaxed(logits, row_offsets, row_owner, draft_tokens, topk=1, margin=0.0,
                          from_position=0, after_tokens=0, generated=None, protected_ids=None)
    verify_greedy_static(logits, row_offsets, row_owner, draft_tokens, relaxed_topk=1)
    verify_sampled(logits, row_offsets, row_owner, draft_tokens,
                   temperature, top_k, top_p, min_p, seed, offset=0)
    draft_confidence(draft_logits, selected=None)
    allocate_verify(confidence, draft_tokens, num_requests, num_drafts, row_budget)
    Goodput(max_steps, window_size=20, update_interval=5, switch_min_gain=0.05)
        .observe(accepted_len, verify_len), .step(cost_ms, batch_size)   (host)
    goodput_select(prefix_acceptance, cost_ms, batch_size, current, switch_min_gain)
"""
import ctypes
import os

import torch  # load torch's HIP runtime first so the library binds to it

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvspec_verify.so")

VSV_F32 = 0
VSV_BF16 = 1
FLAG_LAYOUT = 1
FLAG_TOKEN = 2
FLAG_LOGITS = 4
FLAG_PARAMS = 8

_STATUS = {0: "VSV_OK", 1: "VSV_EINVAL", 2: "VSV_EUNSUPPORTED", 3: "VSV_EWORKSPACE", 4: "VSV_EHIP",
           5: "VSV_ELIMIT"}
VSV_ELIMIT = 5
STATIC_MAX_ROWS = 16384


class VSVError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s (%s): %s" % (_STATUS.get(status, status), status, msg))
        self.status = status


class Batch(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("ld", ctypes.c_int64), ("num_requests", ctypes.c_int32), ("num_rows", ctypes.c_int32),
                ("row_offsets", ctypes.c_void_p), ("row_owner", ctypes.c_void_p),
                ("draft_tokens", ctypes.c_void_p)]


class Outputs(ctypes.Structure):
    _fields_ = [("accepted_len", ctypes.c_void_p), ("next_token", ctypes.c_void_p),
                ("out_offsets", ctypes.c_void_p), ("out_tokens", ctypes.c_void_p),
                ("row_token", ctypes.c_void_p), ("row_lse", ctypes.c_void_p),
                ("error_flag", ctypes.c_void_p), ("slow_rows", ctypes.c_void_p)]


class Relax(ctypes.Structure):
    _fields_ = [("topk", ctypes.c_int32), ("margin", ctypes.c_float), ("from_position", ctypes.c_int32),
                ("after_tokens", ctypes.c_int32), ("generated", ctypes.c_void_p), ("protected_ids", ctypes.c_void_p),
                ("num_protected", ctypes.c_int32)]


MAX_PROTECTED = 256

SYMBOLS = ("vsv_workspace_bytes", "vsv_workspace_init", "vsv_verify_greedy", "vsv_verify_greedy_relaxed",
           "vsv_verify_greedy_static",
           "vsv_verify_sampled",
           "vsv_verify_probabilistic", "vsv_draft_confidence", "vsv_allocate_verify", "vsv_goodput_init", "vsv_goodput_observe",
           "vsv_goodput_step", "vsv_goodput_select", "vsv_status_string", "vsv_test_withhold_row_word", "vsv_version")

GOODPUT_MAX_STEPS = 32
GOODPUT_MAX_WINDOW = 64


class GoodputState(ctypes.Structure):
    _fields_ = [("max_steps", ctypes.c_int32), ("window_size", ctypes.c_int32), ("update_interval", ctypes.c_int32),
                ("switch_min_gain", ctypes.c_double), ("current", ctypes.c_int32), ("since", ctypes.c_int32),
                ("filled", ctypes.c_int32), ("head", ctypes.c_int32),
                ("reached", (ctypes.c_int32 * GOODPUT_MAX_STEPS) * GOODPUT_MAX_WINDOW),
                ("accepted", (ctypes.c_int32 * GOODPUT_MAX_STEPS) * GOODPUT_MAX_WINDOW),
                ("estimate", ctypes.c_double * GOODPUT_MAX_STEPS)]

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libvspec_verify.so is not built; run "
                           "`python -m draft_token_verification_packed_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t
    L.vsv_workspace_bytes.argtypes = [i32, i32, i32]
    L.vsv_workspace_bytes.restype = sz
    L.vsv_workspace_init.argtypes = [vp, sz, vp]
    L.vsv_workspace_init.restype = ctypes.c_int
    L.vsv_verify_greedy.argtypes = [ctypes.POINTER(Batch), i32, ctypes.POINTER(Outputs), vp, sz, vp]
    L.vsv_verify_greedy.restype = ctypes.c_int
    L.vsv_verify_greedy_relaxed.argtypes = [ctypes.POINTER(Batch), ctypes.POINTER(Relax), ctypes.POINTER(Outputs),
                                            vp, sz, vp]
    L.vsv_verify_greedy_relaxed.restype = ctypes.c_int
    L.vsv_verify_greedy_static.argtypes = [ctypes.POINTER(Batch), i32, ctypes.POINTER(Outputs), vp]
    L.vsv_verify_greedy_static.restype = ctypes.c_int
    L.vsv_verify_sampled.argtypes = [ctypes.POINTER(Batch), vp, vp, vp, vp, u64, u64,
                                     ctypes.POINTER(Outputs), vp, sz, vp]
    L.vsv_verify_sampled.restype = ctypes.c_int
    L.vsv_verify_probabilistic.argtypes = [ctypes.POINTER(Batch), vp, i64, vp, vp, vp, vp, vp, u64, u64,
                                           ctypes.POINTER(Outputs), vp, sz, vp]
    L.vsv_verify_probabilistic.restype = ctypes.c_int
    L.vsv_draft_confidence.argtypes = [vp, i32, i32, i64, i32, vp, vp, vp, vp, vp]
    L.vsv_draft_confidence.restype = ctypes.c_int
    L.vsv_allocate_verify.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    L.vsv_allocate_verify.restype = ctypes.c_int
    gp = ctypes.POINTER(GoodputState)
    L.vsv_goodput_init.argtypes = [gp, i32, i32, i32, ctypes.c_double]
    L.vsv_goodput_init.restype = ctypes.c_int
    L.vsv_goodput_observe.argtypes = [gp, vp, vp, i32]
    L.vsv_goodput_observe.restype = ctypes.c_int
    L.vsv_goodput_step.argtypes = [gp, vp, i32, ctypes.POINTER(i32)]
    L.vsv_goodput_step.restype = ctypes.c_int
    L.vsv_goodput_select.argtypes = [vp, vp, i32, i32, i32, ctypes.c_double]
    L.vsv_goodput_select.restype = i32
    L.vsv_status_string.argtypes = [ctypes.c_int]
    L.vsv_status_string.restype = ctypes.c_char_p
    L.vsv_test_withhold_row_word.argtypes = [i32]
    L.vsv_test_withhold_row_word.restype = ctypes.c_int
    L.vsv_version.argtypes = []
    L.vsv_version.restype = i32
    _lib = L
    return L


def _check(status):
    if status != 0:
        raise VSVError(status, lib().vsv_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return VSV_BF16
    if t.dtype == torch.float32:
        return VSV_F32
    raise TypeError("logits must be bfloat16 or float32")


def _vec(t, n, dtype, name):
    if t is None or not t.is_cuda or t.dtype != dtype or t.dim() != 1 or t.numel() != n or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s CUDA vector of length %d" % (name, dtype, n))
    return t


def _logits(t, vocab):
    # the column stride only matters when a row holds more than one element
    # (torch gives tensors without elements, or of one column, any strides)
    if not t.is_cuda or t.dim() != 2 or (t.stride(1) != 1 and t.shape[1] > 1 and t.numel() > 0):
        raise ValueError("logits must be a 2-D CUDA tensor with unit column stride")
    v = t.shape[1] if vocab is None else int(vocab)
    if v > t.shape[1]:
        raise ValueError("vocab exceeds the logits width")
    return _dtype_code(t), v, t.stride(0) if t.shape[0] > 1 else max(t.shape[1], 1)


def workspace_bytes(num_requests, num_rows, sampled=False):
    return int(lib().vsv_workspace_bytes(int(num_requests), int(num_rows), int(bool(sampled))))


_ws_cache = {}


def _resolve_stream(stream, device=None):
    if stream is not None:
        return stream
    return torch.cuda.current_stream(device)


def workspace(num_requests, num_rows, sampled=False, device=None, stream=None):
    """A zeroed workspace tensor, cached per (device, stream) and grown on demand.

    The buffer is allocated and zero-filled on the stream the calls run on,
    so the fill is ordered before them and the caching allocator hands its
    memory to no other stream. Calls on one stream run in order and each
    leaves the workspace ready for the next, so the cached buffer serves
    every later call on that stream. Calls that may overlap need workspaces
    of their own (pass `ws`).
    """
    need = workspace_bytes(num_requests, num_rows, sampled)
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    s = _resolve_stream(stream, dev)
    key = (dev.index, s.cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < need:
        size = max(need, 4096)
        size = (size + 3) // 4 * 4
        with torch.cuda.stream(s):
            ws = torch.empty(size, dtype=torch.uint8, device=dev)
        _check(lib().vsv_workspace_init(_ptr(ws), ws.numel(), ctypes.c_void_p(s.cuda_stream)))
        _ws_cache[key] = ws
    return ws


def _keep_alive(stream, *tensors):
    """Tell the caching allocator that `tensors` are used on `stream` when it
    is not the current stream, so their memory is not reused before the
    stream's work on them is done."""
    if stream is None or stream == torch.cuda.current_stream(stream.device):
        return
    for t in tensors:
        if t is not None and t.is_cuda:
            t.record_stream(stream)


def _prepare(logits, row_offsets, row_owner, draft_tokens, vocab, stream=None):
    dtype, V, ld = _logits(logits, vocab)
    R = logits.shape[0]
    B = row_offsets.numel() - 1
    _vec(row_offsets, B + 1, torch.int32, "row_offsets")
    _vec(row_owner, R, torch.int32, "row_owner")
    if R - B > 0:
        _vec(draft_tokens, R - B, torch.int32, "draft_tokens")
    dev = logits.device
    # outputs are allocated (and the ones with a fill are filled) on the
    # stream the call runs on, so the fills are ordered before the kernels
    with torch.cuda.stream(_resolve_stream(stream, dev)):
        out = _new_outputs(B, R, dev)
    batch = Batch(_ptr(logits), dtype, V, ld, B, R, _ptr(row_offsets), _ptr(row_owner),
                  _ptr(draft_tokens) if R - B > 0 else None)
    outs = _outputs_struct(out)
    return batch, outs, out, B, R


_OUT_KEYS = ("accepted_len", "next_token", "out_offsets", "out_tokens", "row_token", "row_lse", "error_flag",
             "slow_rows")


def _outputs_struct(out):
    return Outputs(*[_ptr(out[k]) for k in _OUT_KEYS])


def _new_outputs(B, R, dev):
    return dict(accepted_len=torch.empty(B, dtype=torch.int32, device=dev),
               next_token=torch.empty(B, dtype=torch.int32, device=dev),
               out_offsets=torch.empty(B + 1, dtype=torch.int32, device=dev),
               out_tokens=torch.full((max(R, 1),), -1, dtype=torch.int32, device=dev),
               row_token=torch.empty(R, dtype=torch.int32, device=dev),
               row_lse=torch.empty(R, dtype=torch.float32, device=dev),
               error_flag=torch.zeros(1, dtype=torch.int32, device=dev),
               slow_rows=torch.zeros(1, dtype=torch.int32, device=dev))


def verify_greedy(logits, row_offsets, row_owner, draft_tokens, relaxed_topk=1, vocab=None,
                  ws=None, stream=None):
    """Greedy verification of a packed batch; returns a dict of device tensors."""
    batch, outs, out, B, R = _prepare(logits, row_offsets, row_owner, draft_tokens, vocab, stream)
    ws = workspace(B, R, False, logits.device, stream) if ws is None else ws
    _keep_alive(stream, logits, row_offsets, row_owner, draft_tokens, ws)
    _check(lib().vsv_verify_greedy(ctypes.byref(batch), int(relaxed_topk), ctypes.byref(outs),
                                   _ptr(ws), ws.numel(), _stream(stream)))
    return out


def verify_greedy_relaxed(logits, row_offsets, row_owner, draft_tokens, topk=1, margin=0.0, from_position=0,
                          after_tokens=0, generated=None, protected_ids=None, vocab=None, ws=None, stream=None):
    """Greedy verification with relaxed acceptance (vsv_verify_greedy_relaxed):
    top-K and/or a logit margin, gated by draft position and by each
    request's generated-token count (`generated`, int32 [B] device or None),
    never relaxing a protected token (`protected_ids`, int32 device vector
    or None). Returns a dict of device tensors."""
    batch, outs, out, B, R = _prepare(logits, row_offsets, row_owner, draft_tokens, vocab, stream)
    if generated is not None:
        _vec(generated, B, torch.int32, "generated")
    nprot = 0
    if protected_ids is not None:
        nprot = protected_ids.numel()
        if nprot:
            _vec(protected_ids, nprot, torch.int32, "protected_ids")
    relax = Relax(int(topk), float(margin), int(from_position), int(after_tokens), _ptr(generated),
                  _ptr(protected_ids) if nprot else None, int(nprot))
    ws = workspace(B, R, False, logits.device, stream) if ws is None else ws
    _keep_alive(stream, logits, row_offsets, row_owner, draft_tokens, generated, protected_ids, ws)
    _check(lib().vsv_verify_greedy_relaxed(ctypes.byref(batch), ctypes.byref(relax), ctypes.byref(outs), _ptr(ws),
                                           ws.numel(), _stream(stream)))
    return out


def withhold_row_word(row):
    """Test hook (vsv_test_withhold_row_word): later row-per-workgroup verify
    launches leave row `row`'s result word unpublished, so their scan waits
    out its bounded poll and flags VSV_FLAG_STALLED; -1 turns it off."""
    _check(lib().vsv_test_withhold_row_word(int(row)))


def verify_greedy_static(logits, row_offsets, row_owner, draft_tokens, relaxed_topk=1, vocab=None, out=None,
                         stream=None):
    """Greedy verification through the entry point that allocates nothing
    (vsv_verify_greedy_static: library-owned scratch, at most STATIC_MAX_ROWS
    rows). `out`, if given, is a dict of output tensors as returned by
    verify_greedy and is written in place; otherwise outputs are allocated
    here. Returns the output dict."""
    batch, outs, res, B, R = _prepare(logits, row_offsets, row_owner, draft_tokens, vocab, stream)
    if out is not None:
        res = out
        outs = _outputs_struct(res)
    _keep_alive(stream, logits, row_offsets, row_owner, draft_tokens)
    _check(lib().vsv_verify_greedy_static(ctypes.byref(batch), int(relaxed_topk), ctypes.byref(outs),
                                          _stream(stream)))
    return res


def verify_sampled(logits, row_offsets, row_owner, draft_tokens, temperature, top_k, top_p, min_p,
                   seed, offset=0, vocab=None, ws=None, stream=None):
    """Sampled / mixed verification of a packed batch; returns a dict of device tensors."""
    batch, outs, out, B, R = _prepare(logits, row_offsets, row_owner, draft_tokens, vocab, stream)
    _vec(temperature, B, torch.float32, "temperature")
    _vec(top_k, B, torch.int32, "top_k")
    _vec(top_p, B, torch.float32, "top_p")
    _vec(min_p, B, torch.float32, "min_p")
    ws = workspace(B, R, True, logits.device, stream) if ws is None else ws
    _keep_alive(stream, logits, row_offsets, row_owner, draft_tokens, temperature, top_k, top_p, min_p, ws)
    _check(lib().vsv_verify_sampled(ctypes.byref(batch), _ptr(temperature), _ptr(top_k), _ptr(top_p),
                                    _ptr(min_p), int(seed) & (2**64 - 1), int(offset) & (2**64 - 1),
                                    ctypes.byref(outs), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def verify_probabilistic(logits, row_offsets, row_owner, draft_tokens, draft_logits, temperature, top_k, top_p,
                         min_p, draft_temperature, seed, offset=0, vocab=None, ws=None, stream=None):
    """Rejection-sampling verification with probabilistic drafts; draft_logits
    holds the R - B draft rows in the draft tokens' layout. Returns a dict of
    device tensors (row_lse and slow_rows are not written)."""
    batch, outs, out, B, R = _prepare(logits, row_offsets, row_owner, draft_tokens, vocab, stream)
    for t, n in ((temperature, "temperature"), (top_p, "top_p"), (min_p, "min_p"),
                 (draft_temperature, "draft_temperature")):
        _vec(t, B, torch.float32, n)
    _vec(top_k, B, torch.int32, "top_k")
    dld = 0
    if R - B > 0:
        dtype, V, _ = _logits(logits, vocab)
        ddt, _, dld = _logits(draft_logits, vocab if vocab is not None else logits.shape[1])
        if ddt != dtype or draft_logits.shape[0] != R - B or draft_logits.shape[1] < V:
            raise ValueError("draft_logits must be [R - B, >= vocab] of the logits' dtype")
        dld = draft_logits.stride(0) if draft_logits.shape[0] > 1 else max(draft_logits.shape[1], 1)
    ws = workspace(B, R, False, logits.device, stream) if ws is None else ws
    _keep_alive(stream, logits, row_offsets, row_owner, draft_tokens, draft_logits, temperature, top_k, top_p,
                min_p, draft_temperature, ws)
    _check(lib().vsv_verify_probabilistic(ctypes.byref(batch), _ptr(draft_logits) if R - B > 0 else None, int(dld),
                                          _ptr(temperature), _ptr(top_k), _ptr(top_p), _ptr(min_p),
                                          _ptr(draft_temperature), int(seed) & (2**64 - 1),
                                          int(offset) & (2**64 - 1), ctypes.byref(outs), _ptr(ws), ws.numel(),
                                          _stream(stream)))
    return out


def draft_confidence(draft_logits, selected=None, vocab=None, stream=None):
    """(confidence, lse, error_flag) device tensors for every draft row."""
    dtype, V, ld = _logits(draft_logits, vocab)
    D = draft_logits.shape[0]
    if selected is not None:
        _vec(selected, D, torch.int32, "selected")
    dev = draft_logits.device
    with torch.cuda.stream(_resolve_stream(stream, dev)):
        conf = torch.empty(D, dtype=torch.float32, device=dev)
        lse = torch.empty(D, dtype=torch.float32, device=dev)
        flag = torch.zeros(1, dtype=torch.int32, device=dev)
    _keep_alive(stream, draft_logits, selected)
    _check(lib().vsv_draft_confidence(_ptr(draft_logits), dtype, V, ld, D, _ptr(selected), _ptr(conf),
                                      _ptr(lse), _ptr(flag), _stream(stream)))
    return conf, lse, flag


def _alloc_outputs(B, K, G, dev, with_drafts):
    return dict(verify_len=torch.empty(B, dtype=torch.int32, device=dev),
                row_offsets=torch.empty(B + 1, dtype=torch.int32, device=dev),
                row_owner=torch.empty(max(G, 1), dtype=torch.int32, device=dev),
                row_source=torch.empty(max(G, 1), dtype=torch.int32, device=dev),
                packed_drafts=(torch.empty(max(G - B, 1), dtype=torch.int32, device=dev) if with_drafts else None),
                prefix=torch.empty(max(B * K, 1), dtype=torch.float32, device=dev))


def _alloc_args(confidence, draft_tokens, B, K, G, out, stream):
    if B * K > 0:
        _vec(confidence, B * K, torch.float32, "confidence")
        if draft_tokens is not None:
            _vec(draft_tokens, B * K, torch.int32, "draft_tokens")
    pd = out["packed_drafts"] if draft_tokens is not None and G > B else None
    return (_ptr(confidence) if B * K > 0 else None, (_ptr(draft_tokens) if pd is not None else None), int(B), int(K), int(G),
            _ptr(out["verify_len"]), _ptr(out["row_offsets"]), _ptr(out["row_owner"]),
            _ptr(out["row_source"]), _ptr(pd), _ptr(out["prefix"]), _stream(stream))


def allocate_verify(confidence, draft_tokens, num_requests, num_drafts, row_budget, stream=None):
    """Verify lengths and packed verify layout for a row budget; returns a dict of device tensors.

    `confidence` and `draft_tokens` are [B * K] request-major device vectors
    (`draft_tokens` may be None). The result's row_offsets, row_owner and
    packed_drafts are the batch layout the verify entry points take.
    """
    B, K, G = int(num_requests), int(num_drafts), int(row_budget)
    dev = confidence.device if confidence is not None else torch.device("cuda", torch.cuda.current_device())
    with torch.cuda.stream(_resolve_stream(stream, dev)):
        out = _alloc_outputs(B, K, G, dev, draft_tokens is not None)
    _keep_alive(stream, confidence, draft_tokens)
    _check(lib().vsv_allocate_verify(*_alloc_args(confidence, draft_tokens, B, K, G, out, stream)))
    return out


def _host_array(x, ctype, np_dtype):
    import numpy as np
    a = np.ascontiguousarray(np.asarray(x, dtype=np_dtype))
    return a, a.ctypes.data_as(ctypes.c_void_p)


class Goodput:
    """Goodput step selection over completed batches (host code; see
    vsv_goodput_* in the header). `observe` takes a batch's accepted and
    verified draft counts, `step` the full-round cost of every candidate
    step count 1 .. max_steps and returns the step count for the next batch."""

    def __init__(self, max_steps, window_size=20, update_interval=5, switch_min_gain=0.05):
        self.state = GoodputState()
        _check(lib().vsv_goodput_init(ctypes.byref(self.state), int(max_steps), int(window_size),
                                      int(update_interval), float(switch_min_gain)))

    def observe(self, accepted_len, verify_len):
        import numpy as np
        a, pa = _host_array(accepted_len, ctypes.c_int32, np.int32)
        k, pk = _host_array(verify_len, ctypes.c_int32, np.int32)
        if a.shape != k.shape or a.ndim != 1:
            raise ValueError("accepted_len and verify_len must be matching vectors")
        _check(lib().vsv_goodput_observe(ctypes.byref(self.state), pa, pk, int(a.size)))

    def step(self, cost_ms, batch_size):
        import numpy as np
        c, pc = _host_array(cost_ms, ctypes.c_double, np.float64)
        if c.size != self.state.max_steps:
            raise ValueError("cost_ms needs one cost per step count 1 .. max_steps")
        out = ctypes.c_int32(0)
        _check(lib().vsv_goodput_step(ctypes.byref(self.state), pc, int(batch_size), ctypes.byref(out)))
        return int(out.value)

    @property
    def estimate(self):
        return [self.state.estimate[j] for j in range(self.state.max_steps)]


def goodput_select(prefix_acceptance, cost_ms, batch_size, current, switch_min_gain=0.05):
    """One stateless scoring (vsv_goodput_select); -1 for invalid arguments."""
    import numpy as np
    p, pp = _host_array(prefix_acceptance, ctypes.c_double, np.float64)
    c, pc = _host_array(cost_ms, ctypes.c_double, np.float64)
    if p.size != c.size:
        raise ValueError("one prefix acceptance and one cost per step count")
    return int(lib().vsv_goodput_select(pp, pc, int(c.size), int(batch_size), int(current), float(switch_min_gain)))


class PreparedCall:
    """One entry-point call with every argument marshalled once.

    `run()` issues the C call on the stream captured at construction; the
    tensors passed in must stay alive (they are referenced here). Used where
    per-call Python overhead would otherwise show next to a ~30 us kernel.
    """

    def __init__(self, fn, args, keep):
        self._fn = fn
        self._args = args
        self._keep = keep

    def run(self):
        _check(self._fn(*self._args))


def prepare_greedy(logits, row_offsets, row_owner, draft_tokens, relaxed_topk=1, vocab=None,
                   out=None, ws=None, stream=None):
    batch, outs, res, B, R = _prepare(logits, row_offsets, row_owner, draft_tokens, vocab, stream)
    if out is not None:
        res = out
        outs = _outputs_struct(res)
    ws = workspace(B, R, False, logits.device, stream) if ws is None else ws
    _keep_alive(stream, logits, row_offsets, row_owner, draft_tokens, ws)
    args = (ctypes.byref(batch), int(relaxed_topk), ctypes.byref(outs), _ptr(ws), ws.numel(), _stream(stream))
    return PreparedCall(lib().vsv_verify_greedy, args, (batch, outs, res, ws, logits)), res


def prepare_sampled(logits, row_offsets, row_owner, draft_tokens, temperature, top_k, top_p, min_p,
                    seed, offset=0, vocab=None, out=None, ws=None, stream=None):
    batch, outs, res, B, R = _prepare(logits, row_offsets, row_owner, draft_tokens, vocab, stream)
    if out is not None:
        res = out
        outs = _outputs_struct(res)
    for t, dt, name in ((temperature, torch.float32, "temperature"), (top_k, torch.int32, "top_k"),
                        (top_p, torch.float32, "top_p"), (min_p, torch.float32, "min_p")):
        _vec(t, B, dt, name)
    ws = workspace(B, R, True, logits.device, stream) if ws is None else ws
    _keep_alive(stream, logits, row_offsets, row_owner, draft_tokens, temperature, top_k, top_p, min_p, ws)
    args = (ctypes.byref(batch), _ptr(temperature), _ptr(top_k), _ptr(top_p), _ptr(min_p),
            int(seed) & (2**64 - 1), int(offset) & (2**64 - 1), ctypes.byref(outs), _ptr(ws), ws.numel(),
            _stream(stream))
    return PreparedCall(lib().vsv_verify_sampled, args,
                        (batch, outs, res, ws, logits, temperature, top_k, top_p, min_p)), res


def prepare_allocate(confidence, draft_tokens, num_requests, num_drafts, row_budget, out=None, stream=None):
    B, K, G = int(num_requests), int(num_drafts), int(row_budget)
    if out is None:
        out = _alloc_outputs(B, K, G, confidence.device, draft_tokens is not None)
    args = _alloc_args(confidence, draft_tokens, B, K, G, out, stream)
    return PreparedCall(lib().vsv_allocate_verify, args, (confidence, draft_tokens, out)), out


def prepare_confidence(draft_logits, selected=None, vocab=None, out=None, stream=None):
    dtype, V, ld = _logits(draft_logits, vocab)
    D = draft_logits.shape[0]
    if selected is not None:
        _vec(selected, D, torch.int32, "selected")
    dev = draft_logits.device
    if out is None:
        out = (torch.empty(D, dtype=torch.float32, device=dev), torch.empty(D, dtype=torch.float32, device=dev),
               torch.zeros(1, dtype=torch.int32, device=dev))
    conf, lse, flag = out
    args = (_ptr(draft_logits), dtype, V, ld, D, _ptr(selected), _ptr(conf), _ptr(lse), _ptr(flag),
            _stream(stream))
    return PreparedCall(lib().vsv_draft_confidence, args, (draft_logits, selected, out)), out
