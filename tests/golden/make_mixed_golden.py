"""Expected outputs of the whole large mixed batch (B=512, K=7, V=152064
bf16, even requests greedy, odd ones T = 0.7 with top_p 0.95), written by the
CPU oracle alone: `python tests/golden/make_mixed_golden.py`.

The batch is synth.make("mixed") with its rounding-sensitive rows re-drawn:
every row of a sampled request whose own draw, top-p cut or min-p cut lies
within the tie margins of tests/workloads.py, and every draft row whose
probabilistic acceptance or residual draw (draft law: softmax of the draft
row at the request's temperature) lies within DELTA_MASS of its threshold,
is re-drawn (attempt + 1) until none is. The file records those attempts,
fingerprints of the inputs they give, and the oracle's outputs for
  * vsv_verify_sampled on the batch (every row token, log-sum-exp, accepted
    length, next token and the compacted output),
  * vsv_draft_confidence on its 3584 draft rows with selected = the drafts,
  * vsv_verify_probabilistic on the batch with draft temperature = the
    request's temperature.
Nothing here runs or reads the HIP library."""
import hashlib
import multiprocessing
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402
from oracle.probabilistic import row_margins, row_uniforms, verify_probabilistic  # noqa: E402
from tests.workloads import DELTA_MASS, DELTA_Z  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "mixed_b512_k7_v152064.npz")

_WL = None


def fingerprint(wl):
    h = hashlib.sha256()
    for a in (wl.logits, wl.drafts, wl.draft_logits, wl.offsets, wl.temperature, wl.top_p):
        h.update(np.ascontiguousarray(a).view(np.uint8).tobytes())
    return h.hexdigest()


def _row_bad(r):
    wl = _WL
    i = int(wl.owner[r])
    T = float(np.float32(wl.temperature[i]))
    if T == 0.0:
        return False
    j = r - int(wl.offsets[i])
    K = int(wl.offsets[i + 1] - wl.offsets[i]) - 1
    x = oracle.row_f64(wl.logits, wl.dtype, r, wl.V)
    k, tp, mp = int(wl.top_k[i]), float(np.float32(wl.top_p[i])), float(np.float32(wl.min_p[i]))
    u, ua = row_uniforms(wl.seed, i, j, wl.offset)
    m_tp, m_u, m_mp = oracle.sampled_row_margins(x, T, k, tp, mp, u)
    if m_tp < DELTA_MASS or m_u < DELTA_MASS or m_mp < DELTA_Z:
        return True
    if j < K:
        y = oracle.row_f64(wl.draft_logits, wl.dtype, r - i, wl.V)
        am, rm = row_margins(x, y, T, k, tp, mp, T, int(wl.drafts[r - i]), u, ua)
        if am < DELTA_MASS or rm < DELTA_MASS:
            return True
    return False


def _init(wl):
    global _WL
    _WL = wl


def bad_rows(wl, rows, pool):
    flags = pool.map(_row_bad, rows, chunksize=8)
    return [r for r, f in zip(rows, flags) if f]


def main():
    t0 = time.time()
    wl = synth.make("mixed")
    rows = [r for r in range(wl.R) if wl.temperature[wl.owner[r]] > 0]
    ctx = multiprocessing.get_context("fork")
    for rnd in range(20):
        with ctx.Pool(min(8, os.cpu_count() or 1), initializer=_init, initargs=(wl,)) as pool:
            bad = bad_rows(wl, rows, pool)
        print("round %d: %d of %d rows inside a margin (%.0f s)" % (rnd, len(bad), len(rows), time.time() - t0),
              flush=True)
        if not bad:
            break
        synth.redraw_rows(wl, bad)
        rows = bad
    else:
        raise RuntimeError("rows keep violating the margins")
    td = wl.temperature.astype(np.float32)
    s = oracle.verify_sampled(wl.logits, wl.dtype, wl.V, wl.offsets, wl.owner, wl.drafts, wl.temperature,
                              wl.top_k, wl.top_p, wl.min_p, wl.seed, wl.offset)
    print("sampled oracle done (%.0f s)" % (time.time() - t0), flush=True)
    conf, clse = oracle.draft_confidence(wl.draft_logits, wl.dtype, wl.V, wl.selected)
    print("confidence oracle done (%.0f s)" % (time.time() - t0), flush=True)
    p = verify_probabilistic(wl.logits, wl.dtype, wl.V, wl.offsets, wl.owner, wl.drafts, wl.draft_logits,
                             wl.temperature, wl.top_k, wl.top_p, wl.min_p, td, wl.seed, wl.offset)
    print("probabilistic oracle done (%.0f s)" % (time.time() - t0), flush=True)
    att = sorted(wl.attempts.items())
    np.savez_compressed(
        OUT,
        attempt_rows=np.array([a for a, _ in att], dtype=np.int32),
        attempt_counts=np.array([c for _, c in att], dtype=np.int32),
        fingerprint=np.array(fingerprint(wl)),
        s_accepted_len=s["accepted_len"], s_next_token=s["next_token"], s_out_offsets=s["out_offsets"],
        s_out_tokens=s["out_tokens"], s_row_token=s["row_token"], s_row_lse=s["row_lse"],
        c_confidence=conf, c_lse=clse,
        p_accepted_len=p["accepted_len"], p_next_token=p["next_token"], p_out_offsets=p["out_offsets"],
        p_out_tokens=p["out_tokens"], p_row_token=p["row_token"])
    print("wrote %s: %d re-drawn rows (%.0f s)" % (OUT, len(att), time.time() - t0))


if __name__ == "__main__":
    main()
