"""Seeded synthetic workloads for packed draft-token verification.

This module is the one thing the HIP path's tests and the CPU oracle both
consume. It only draws random numbers and lays them out; it holds none of the
verification arithmetic (no reductions, filters, sampling or acceptance).
Draft tokens are placed at given positions of NumPy's stable descending sort
of a row, which is workload construction; every expected value comes from the
oracle.

Every row is drawn from its own NumPy stream keyed by (seed, row, attempt),
so a single row can be re-drawn (attempt + 1) without touching the rest; the
tests use that to keep sampled rows away from rounding-sensitive thresholds.

The five workloads (tiny, eagle, ragged, relaxed, mixed) follow the shapes
and distributions of the verification batches being measured: B requests of K draft tokens (K + 1 verify rows each, the
bonus row last), a 152064-token vocabulary, N(0, sigma^2) logits in float32
or bfloat16 (round-to-nearest-even from float32), and drafts that hit the
target's arg-max with fixed per-position rates.
"""
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

F32 = 0
BF16 = 1
VOCAB = 152064


def f32_to_bf16_bits(a):
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.

    The upper half rounds up when the lower half is above one half, or
    exactly one half with an odd upper half (a carry out of the top wraps,
    as only NaN patterns can carry that far)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    hi = u >> np.uint32(16)
    lo = u & np.uint32(0xFFFF)
    up = (lo + (hi & np.uint32(1))) > np.uint32(0x8000)
    return (hi + up).astype(np.uint16)


@dataclass
class Workload:
    name: str
    key: str
    B: int
    V: int
    ld: int
    dtype: int
    offsets: np.ndarray            # int32 [B+1]
    owner: np.ndarray              # int32 [R]
    drafts: np.ndarray             # int32 [R-B]
    logits: np.ndarray             # float32 or uint16 (bf16 bits) [R, ld]
    sampled: bool = False
    temperature: Optional[np.ndarray] = None   # float32 [B]
    top_k: Optional[np.ndarray] = None         # int32 [B]
    top_p: Optional[np.ndarray] = None         # float32 [B]
    min_p: Optional[np.ndarray] = None         # float32 [B]
    seed: int = 0
    offset: int = 0
    relaxed_topk: int = 1
    draft_logits: Optional[np.ndarray] = None  # [D, ld] same dtype as logits
    selected: Optional[np.ndarray] = None      # int32 [D]
    planted: Optional[np.ndarray] = None       # per request, tiny greedy batch only
    attempts: Dict[int, int] = field(default_factory=dict)
    _spec: dict = field(default_factory=dict, repr=False)

    @property
    def R(self):
        return int(self.offsets[-1])

    @property
    def D(self):
        return 0 if self.draft_logits is None else int(self.draft_logits.shape[0])

    def logit_bytes(self):
        """Bytes of logits the path reads once: verify rows plus draft rows."""
        es = 2 if self.dtype == BF16 else 4
        return (self.R + self.D) * self.V * es


# Workload recipes by key. sigma: logits standard deviation; boost: added to
# the row's largest float32 draw before rounding; hit: per-position
# probability that a draft equals the row's arg-max; data_seed and
# philox_seed: the default seeds of the logits and of the sampler.
SPECS = {
    "tiny": dict(name="tiny greedy verify, B=4 K=4 V=1024 fp32", B=4, K=4, V=1024,
            dtype=F32, sigma=2.0, boost=0.0, mode="planted", data_seed=1001, philox_seed=2001),
    "eagle": dict(name="EAGLE greedy verify, B=128 K=4 V=152064 bf16", B=128, K=4, V=VOCAB,
            data_seed=1002, philox_seed=2002,
            dtype=BF16, sigma=3.0, boost=4.0, mode="hit",
            hit=(0.8, 0.7, 0.6, 0.5), miss="uniform"),
    "ragged": dict(name="ragged sampled verify, B=128 K~U{0..7} V=152064 fp32", B=128, K=None,
            data_seed=1003, philox_seed=2003,
            Kmax=7, V=VOCAB, dtype=F32, sigma=2.5, boost=0.0, mode="hit",
            hit=(0.75,), miss="rank", temps=(0.0, 0.5, 1.0), top_k=50, top_p=0.9,
            min_p=0.05, sampled=True),
    "relaxed": dict(name="relaxed top-4 verify + draft confidence, B=128 K=4 V=152064 bf16",
            data_seed=1004, philox_seed=2004,
            B=128, K=4, V=VOCAB, dtype=BF16, sigma=3.0, boost=0.0, mode="geometric",
            relaxed_topk=4, confidence=True),
    "mixed": dict(name="large mixed verify + draft confidence, B=512 K=7 V=152064 bf16",
            data_seed=1005, philox_seed=2005,
            B=512, K=7, V=VOCAB, dtype=BF16, sigma=3.0, boost=0.0, mode="hit",
            hit=(0.8, 0.7, 0.6, 0.5, 0.5, 0.5, 0.5), miss="rank", temps="alternate",
            alt_temp=0.7, top_k=0, top_p=0.95, min_p=0.0, sampled=True, confidence=True),
}


def _row_stream(seed, kind, r, attempt):
    return np.random.default_rng([int(seed), int(kind), int(r), int(attempt)])


def _draw_row(spec, seed, r, attempt, V, ld, pad):
    g = _row_stream(seed, 1, r, attempt)
    x = (g.standard_normal(V, dtype=np.float32) * np.float32(spec["sigma"])).astype(np.float32)
    if spec["boost"]:
        t = int(np.argmax(x))
        x[t] = np.float32(x[t] + np.float32(spec["boost"]))
    return _store(spec, x, ld, pad)


def _store(spec, x, ld, pad):
    V = x.shape[0]
    if spec["dtype"] == BF16:
        row = np.empty(ld, dtype=np.uint16)
        row[:V] = f32_to_bf16_bits(x)
        row[V:] = 0x7FC0 if pad else 0   # bf16 quiet NaN in the padding
    else:
        row = np.empty(ld, dtype=np.float32)
        row[:V] = x
        row[V:] = np.nan if pad else 0.0
    return row


def _as_f32(spec, row, V):
    if spec["dtype"] == BF16:
        return (row[:V].astype(np.uint32) << np.uint32(16)).view(np.float32)
    return row[:V]


def _place_draft(spec, row, V, seed, r, j, attempt):
    """Draft token for verify row r (local position j) from the row's values."""
    g = _row_stream(seed, 3, r, attempt)
    x = _as_f32(spec, row, V)
    mode = spec["mode"]
    if mode == "geometric":
        # rank min(G - 1, 8), G ~ Geometric(1/2) on {1, 2, ...}
        rank = min(int(g.geometric(0.5)) - 1, 8)
    else:
        hit = spec["hit"]
        p = hit[min(j, len(hit) - 1)]
        if g.random() < p:
            rank = 0
        elif spec.get("miss") == "rank":
            rank = int(g.integers(1, 8))
        else:
            rank = -1
    if rank == -1:
        top = int(np.argmax(x))
        t = int(g.integers(0, V - 1))
        return t + 1 if t >= top else t
    return _token_at_rank(x, rank)


def _token_at_rank(x, rank):
    """Token at 0-based position `rank` of the stable descending order of x."""
    if rank == 0:
        return int(np.argmax(x))
    kth = np.partition(x, x.shape[0] - 1 - rank)[x.shape[0] - 1 - rank]
    cand = np.flatnonzero(x >= kth)
    cand = cand[np.argsort(-x[cand], kind="stable")]
    return int(cand[rank])


def make(key, *, B=None, V=None, K=None, ld=None, seed=None, pad=False,
         attempts=None):
    """Build workload `key` (a key of SPECS); B, V, K and ld override the recipe."""
    spec = dict(SPECS[key])
    if B is not None:
        spec["B"] = B
    if V is not None:
        spec["V"] = V
    if K is not None:
        spec["K"] = K
        spec["Kmax"] = K
    Bn, Vn = spec["B"], spec["V"]
    ld = Vn if ld is None else ld
    seed = spec["data_seed"] if seed is None else seed
    attempts = dict(attempts or {})
    g = np.random.default_rng([seed, 0])

    if spec["K"] is None:
        Ks = g.integers(0, spec["Kmax"] + 1, size=Bn)
    else:
        Ks = np.full(Bn, spec["K"], dtype=np.int64)
    offsets = np.zeros(Bn + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(Ks + 1)
    R = int(offsets[-1])
    owner = np.repeat(np.arange(Bn, dtype=np.int32), (Ks + 1).astype(np.int64))

    wl = Workload(name=spec["name"], key=key, B=Bn, V=Vn, ld=ld,
                  dtype=spec["dtype"], offsets=offsets, owner=owner,
                  drafts=np.zeros(R - Bn, dtype=np.int32),
                  logits=np.empty((R, ld), dtype=np.uint16 if spec["dtype"] == BF16 else np.float32),
                  seed=spec["philox_seed"], offset=0,
                  relaxed_topk=spec.get("relaxed_topk", 1), attempts=attempts)
    wl._spec = dict(spec, pad=pad, data_seed=seed)

    if spec.get("sampled"):
        wl.sampled = True
        temps = spec["temps"]
        if temps == "alternate":
            T = np.where(np.arange(Bn) % 2 == 1, spec["alt_temp"], 0.0)
        else:
            T = np.asarray(temps)[g.integers(0, len(temps), size=Bn)]
        wl.temperature = T.astype(np.float32)
        wl.top_k = np.full(Bn, spec["top_k"], dtype=np.int32)
        wl.top_p = np.full(Bn, spec["top_p"], dtype=np.float32)
        wl.min_p = np.full(Bn, spec["min_p"], dtype=np.float32)

    if spec["mode"] == "planted":
        # one request (chosen by the seed) matches fully; every other has one
        # mismatch at a uniformly random position
        full = int(g.integers(0, Bn))
        planted = np.array([spec["K"] if i == full else int(g.integers(0, spec["K"]))
                            for i in range(Bn)], dtype=np.int32)
        wl.planted = planted

    _for_each(R, lambda r: _fill_row(wl, r))

    if spec.get("confidence"):
        D = R - Bn
        dl = np.empty((D, ld), dtype=wl.logits.dtype)

        def draft_row(q):
            gq = _row_stream(seed, 4, q, 0)
            y = (gq.standard_normal(Vn, dtype=np.float32) * np.float32(spec["sigma"])).astype(np.float32)
            dl[q] = _store(spec, y, ld, pad)

        _for_each(D, draft_row)
        wl.draft_logits = dl
        wl.selected = wl.drafts.copy()
    return wl


def _for_each(n, fn):
    """fn(0) .. fn(n - 1) on a few threads. Every row draws from its own
    stream and writes only its own slots, so the result does not depend on
    the order; NumPy releases the interpreter lock in the bulk work."""
    import concurrent.futures
    import os
    workers = min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 4)
    if n < 64 or workers < 2:
        for k in range(n):
            fn(k)
        return
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        for _ in ex.map(fn, range(n), chunksize=16):
            pass


def _fill_row(wl, r):
    spec = wl._spec
    seed = spec["data_seed"]
    a = wl.attempts.get(r, 0)
    wl.logits[r] = _draw_row(spec, seed, r, a, wl.V, wl.ld, spec["pad"])
    i = int(wl.owner[r])
    j = r - int(wl.offsets[i])
    K = int(wl.offsets[i + 1] - wl.offsets[i]) - 1
    if j == K:
        return
    if spec["mode"] == "planted":
        x = _as_f32(spec, wl.logits[r], wl.V)
        top = int(np.argmax(x))
        if j == int(wl.planted[i]):
            g = _row_stream(seed, 3, r, a)
            t = int(g.integers(0, wl.V - 1))
            d = t + 1 if t >= top else t
        else:
            d = top
    else:
        d = _place_draft(spec, wl.logits[r], wl.V, seed, r, j, a)
    wl.drafts[r - i] = d
    if wl.selected is not None:
        wl.selected[r - i] = d


def redraw_rows(wl, rows):
    """Re-draw the given verify rows (and their drafts) with attempt + 1."""
    for r in rows:
        wl.attempts[int(r)] = wl.attempts.get(int(r), 0) + 1
        _fill_row(wl, int(r))
    return wl


def scores(B, K, seed, kind="confidence", V=VOCAB):
    """Per-draft scores and draft tokens for adaptive verify allocation.

    Returns (scores float32 [B * K], drafts int32 [B * K]), request-major.
    Kinds:
      confidence  half the positions U(0.05, 0.95) (a draft near the top of
                  its distribution), half 10^U(-9, -1) (a draft far down it)
      uniform     U(0, 1)
      ties        drawn from {0, 0.25, 0.5, 1}, so products tie often
      special     U(-0.5, 1.5) with a few NaN and +-inf (outside [0, 1])
      tiny        U(0, 1e-12), so long products reach subnormals and 0
    """
    g = np.random.default_rng([seed, 7, B, K])
    n = B * K
    if kind == "confidence":
        near = g.uniform(0.05, 0.95, n)
        far = 10.0 ** g.uniform(-9.0, -1.0, n)
        s = np.where(g.uniform(size=n) < 0.5, near, far)
    elif kind == "uniform":
        s = g.uniform(0.0, 1.0, n)
    elif kind == "ties":
        s = g.choice(np.array([0.0, 0.25, 0.5, 1.0]), n)
    elif kind == "special":
        s = g.uniform(-0.5, 1.5, n)
        if n:
            for v in (np.nan, np.inf, -np.inf):
                s[g.integers(0, n, max(1, n // 50))] = v
    elif kind == "tiny":
        s = g.uniform(0.0, 1e-12, n)
    else:
        raise ValueError(kind)
    drafts = g.integers(0, V, n).astype(np.int32)
    return s.astype(np.float32), drafts
