"""Adaptive target-verify allocation: CPU oracle (test infrastructure only).

Only tests/, the smoke check and the benchmark's CPU baseline call this
module; the HIP library never does, and nothing here comes from it.

What the pages fix (xLLM docs, "Adaptive speculative inference": the table
of control switches, entry enable_adaptive_target_verify, and section
"Adaptive target verification from MTP logits"):

* every round still runs all draft steps, so each request has the same
  number K of draft tokens, and only the verify work is trimmed;
* the selected token's draft probability, exp(selected - logsumexp(draft)),
  is the predicted acceptance score of a draft position (it is not the true
  target acceptance probability);
* the host fixes the padded target-row budget ahead of the round, while the
  current round's scores stay on the device and decide the prefix allocation
  (how many leading drafts of each request the target verifies), followed by
  packing the verify rows.

Readings taken where the pages give no formula (each listed in the design
notes):

* A draft is accepted only if every earlier draft of its request is, so the
  predicted probability that draft j of request i is accepted is the running
  product of the request's scores through j. It is taken in float32, left to
  right, as the device takes the same integer decision in the same
  precision. Scores are first clamped to [0, 1] (NaN counts as 0).
* The budget G counts packed rows including every request's bonus row, so
  B <= G <= B * (K + 1). The G - B extra rows go to the positions with the
  largest products, ties broken by request, then position, ascending. This
  maximises the expected number of accepted drafts; since the products never
  grow along a request, the chosen positions of each request are a prefix.
* Packing: request i owns rows off[i] .. off[i+1] - 1 with off the exclusive
  scan of (k_i + 1); its row j is row j of the request in the full-width
  layout (index i * (K + 1) + j), and its draft tokens are its first k_i
  drafts, at off[i] - i + j as the verify entry points read them.

Parity-pinned by tests/test_oracle_allocate.py: brute-force optimality over
every allocation on tiny batches, closed forms for equal and unit scores,
nesting in the budget, and the packed layout checked by the verification
oracle itself.
"""
import numpy as np


def clamp_scores(conf):
    """Scores as float32 in [0, 1]; NaN becomes 0."""
    c = np.asarray(conf, dtype=np.float32).copy()
    c[np.isnan(c)] = 0.0
    return np.clip(c, np.float32(0.0), np.float32(1.0)).astype(np.float32)


def prefix_scores(conf, B, K):
    """Running products P[i, j] = c[i, 0] * ... * c[i, j] in float32."""
    c = clamp_scores(np.asarray(conf).reshape(B, K))
    P = np.zeros((B, K), dtype=np.float32)
    for i in range(B):
        run = np.float32(1.0)
        for j in range(K):
            run = np.float32(run * c[i, j])
            P[i, j] = run
    return P


def allocate_verify(conf, drafts, B, K, G):
    """Verify lengths and the packed verify layout for a row budget G."""
    if not (B <= G <= B * (K + 1)):
        raise ValueError("budget outside [B, B * (K + 1)]")
    P = prefix_scores(conf, B, K)
    M = G - B
    # every position ordered by (product desc, request asc, position asc)
    ii, jj = np.meshgrid(np.arange(B), np.arange(K), indexing="ij")
    order = np.lexsort((jj.ravel(), ii.ravel(), -P.ravel().astype(np.float64)))
    chosen = order[:M]
    k = np.zeros(B, dtype=np.int32)
    for q in chosen:
        k[q // K] += 1
    d = np.asarray(drafts, dtype=np.int32).reshape(B, K)
    off = np.zeros(B + 1, dtype=np.int32)
    for i in range(B):
        off[i + 1] = off[i] + k[i] + 1
    owner = np.zeros(G, dtype=np.int32)
    source = np.zeros(G, dtype=np.int32)
    packed = np.zeros(G - B, dtype=np.int32)
    for i in range(B):
        for j in range(k[i] + 1):
            owner[off[i] + j] = i
            source[off[i] + j] = i * (K + 1) + j
        for j in range(k[i]):
            packed[off[i] - i + j] = d[i, j]
    return dict(verify_len=k, row_offsets=off, row_owner=owner, row_source=source,
                packed_drafts=packed, prefix=P)
