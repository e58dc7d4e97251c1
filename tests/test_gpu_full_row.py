"""The exact whole-row path of sampled verification, against the oracle.

Rows take it when their draw or filter cut lies beyond the candidates the
capture keeps: plain temperature sampling and top-p alone over flat rows,
a hot temperature (draws deep in the tail), count cuts deep in the rank
order (top-k over most of the vocabulary), a min-p cut far below the
maximum, and heavy ties (each value held by about 1900 tokens, so the
search ends on a tie resolved in index order), for both element types and
a misaligned row start. Every case checks that the path ran."""
import numpy as np
import pytest

import oracle
from tests.test_gpu_sampled import run_custom
from tests.workloads import assert_same, cuda_or_skip, custom_sampled, host, oracle_custom

pytestmark = pytest.mark.gpu

V = 152064
CASES = {
    "plain-bf16": (oracle.BF16, (1.0, 0, 1.0, 0.0), dict(sigma=3.0)),
    "plain-f32": (oracle.F32, (1.0, 0, 1.0, 0.0), dict(sigma=3.0)),
    "top-p-f32": (oracle.F32, (1.0, 0, 0.95, 0.0), dict(sigma=3.0)),
    "hot-top-p-bf16": (oracle.BF16, (4.0, 0, 0.97, 0.0), dict(sigma=3.0)),
    "deep-top-k-f32": (oracle.F32, (1.0, 120000, 1.0, 0.0), dict(sigma=3.0)),
    "min-p-f32": (oracle.F32, (1.0, 0, 1.0, 0.001), dict(sigma=3.0)),
    "ties-bf16": (oracle.BF16, (1.0, 0, 0.9, 0.0), dict(ties=True)),
    "ties-f32-misaligned": (oracle.F32, (1.0, 0, 1.0, 0.0), dict(ties=True, shift=1, ld=V + 3)),
}


@pytest.fixture(scope="module")
def vsv():
    cuda_or_skip()
    import draft_token_verification_packed_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("case", sorted(CASES))
def test_full_row_path(vsv, case):
    dtype, params, kw = CASES[case]
    rng = np.random.default_rng(sum(map(ord, case)))
    b = custom_sampled(rng, 4, 2, V, dtype, lambda i: params, seed=11, offset=5, **kw)
    print("full-row case %s: R=%d" % (case, int(b["offsets"][-1])), flush=True)
    out = run_custom(vsv, b)
    assert_same(out, oracle_custom(b))
    assert int(host(out["slow_rows"])[0]) > 0, "no row took the whole-row path"
