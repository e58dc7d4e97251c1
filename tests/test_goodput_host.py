"""The library's goodput step selection (host code behind the C ABI) against
the oracle: identical estimates and step decisions over random histories,
the stateless scoring on random inputs, and argument errors. No GPU needed."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import draft_token_verification_packed_amd as vsv
from oracle.goodput import GoodputController, select

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(vsv.LIB_PATH):
        pytest.skip("library not built (run the package build first)")
    return vsv.lib()


def test_state_layout_matches_the_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "vspec_verify.h"\n'
                   'int main(void) { printf("%zu %zu %zu %zu\\n", sizeof(vsv_goodput), '
                   'offsetof(vsv_goodput, switch_min_gain), offsetof(vsv_goodput, reached), '
                   'offsetof(vsv_goodput, estimate)); return 0; }\n')
    exe = tmp_path / "layout"
    r = subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                        "-D__HIP_PLATFORM_AMD__", str(src), "-o", str(exe)], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("no host C compiler for the layout check: " + r.stderr[:200])
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    S = vsv.GoodputState
    assert got == [ctypes.sizeof(S), S.switch_min_gain.offset, S.reached.offset, S.estimate.offset]


@pytest.mark.parametrize("seed", range(8))
def test_controller_matches_oracle(L, seed):
    rng = np.random.default_rng(300 + seed)
    S = int(rng.integers(1, 9))
    W = int(rng.integers(1, 25))
    I = int(rng.integers(1, 7))
    m = float(rng.choice([0.0, 0.02, 0.05, 0.2]))
    lib_g = vsv.Goodput(S, W, I, m)
    ref = GoodputController(S, W, I, m)
    for t in range(60):
        B = int(rng.integers(0, 40))
        # verify lengths up to S + 2 (beyond max_steps is allowed), acceptance
        # drifting over time so that the best step count moves
        k = rng.integers(0, S + 3, B)
        p = 0.5 + 0.45 * np.sin(t / 7.0 + seed)
        a = np.array([min(int(rng.geometric(1.0 - p)) - 1, int(x)) for x in k], dtype=np.int64)
        lib_g.observe(a, k)
        ref.observe(a, k)
        assert lib_g.estimate == list(ref.estimate), t
        cost = np.cumsum(rng.uniform(0.5, 2.0, S)) + rng.uniform(1.0, 10.0)
        assert lib_g.step(cost, max(B, 1)) == ref.step(cost, max(B, 1)), t


def test_select_matches_oracle_on_random_inputs(L):
    rng = np.random.default_rng(9)
    for _ in range(2000):
        S = int(rng.integers(1, 33))
        pa = np.sort(rng.uniform(0, 1, S))[::-1].copy()
        if rng.uniform() < 0.2:
            pa[:] = np.round(pa * 4) / 4          # ties
        cost = rng.uniform(0.1, 5.0, S)
        if rng.uniform() < 0.2:
            cost[:] = np.ceil(cost)               # equal costs
        cur = int(rng.integers(1, S + 1))
        m = float(rng.choice([0.0, 0.05, 0.1]))
        B = int(rng.integers(1, 600))
        assert vsv.goodput_select(pa, cost, B, cur, m) == select(pa, cost, B, cur, m)


def test_argument_errors(L):
    with pytest.raises(vsv.VSVError):
        vsv.Goodput(0)
    with pytest.raises(vsv.VSVError):
        vsv.Goodput(33)
    with pytest.raises(vsv.VSVError):
        vsv.Goodput(4, window_size=65)
    with pytest.raises(vsv.VSVError):
        vsv.Goodput(4, update_interval=0)
    g = vsv.Goodput(4, 5, 1, 0.05)
    with pytest.raises(vsv.VSVError):
        g.observe([3], [2])                       # accepted more than verified
    with pytest.raises(vsv.VSVError):
        g.observe([-1], [2])
    assert g.state.filled == 0                    # rejected batches are not recorded
    with pytest.raises(vsv.VSVError):
        g.step([1.0, 2.0, 0.0, 4.0], 8)           # a cost that is not positive
    with pytest.raises(vsv.VSVError):
        g.step([1.0, 2.0, float("nan"), 4.0], 8)
    assert g.step([1.0, 2.0, 3.0, 4.0], 8) == 4   # nothing observed: stays at max_steps
    assert vsv.goodput_select([0.5, 0.2], [1.0, 1.0], 4, 3, 0.05) == -1   # current out of range
    assert vsv.goodput_select([0.5, 0.2], [1.0, -1.0], 4, 1, 0.05) == -1
