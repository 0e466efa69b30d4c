"""The bounds-checking debug build (libfkl_debug.so, FKL_DEBUG) on the GPU.

A child process loads the debug build (FKL_LIBRARY) and runs the cases of
tests/debug_cases.py: every kernel checks its global accesses against the
extents the host planned, and every entry point would return FKL_EDEVICE
naming the access class if one fell outside. The cases must all succeed and
give the release build's results, run here: the same integers exactly, and
floating-point outputs to within RTOL of each tensor's largest magnitude (the
checks change no arithmetic, but they move code between basic blocks, which
can change where the compiler fuses a multiply and an add: 1-ulp differences
were seen in row_kl). A planted case narrows the gradient block's extent from the
host (FKL_DEBUG_SHRINK_G=1): the debug build must skip those stores and
report the gradient block, with every kernel still ending normally. The
full-size case runs the headline shape and the builder's default pass at the
large head, whose plans (passes, slabs, candidate slices) the small cases do
not reach; it compares sums and largest magnitudes of the outputs.
"""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import output_projection_kl_amd as fkl
from output_projection_kl_amd.build import DEBUG_LIB_PATH

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
import debug_cases  # noqa: E402

RTOL = 1e-5


def test_debug_build_reports_nothing_and_matches_the_release_build(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(DEBUG_LIB_PATH):
        pytest.fail(f"{DEBUG_LIB_PATH} is missing: __graft_entry__.build() builds it")
    out = tmp_path / "debug.npz"
    env = dict(os.environ, FKL_LIBRARY=DEBUG_LIB_PATH)
    env.pop("FKL_DEBUG_SHRINK_G", None)
    print("[debug-build] child process with the debug library", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "debug_cases.py"), str(out), "--planted",
                        "--fullsize"], env=env, capture_output=True, text=True, timeout=300)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0, r.stderr[-3000:]
    dbg = dict(np.load(out))
    msg = str(dbg.pop("planted/planted_msg"))
    assert "bounds check failed" in msg and "gradient block" in msg, msg
    print("[debug-build] release build in this process", flush=True)
    rel = debug_cases.run_all(fullsize=True)
    assert set(rel) == set(dbg)
    for k in sorted(rel):
        a, b = np.asarray(rel[k]), np.asarray(dbg[k])
        assert a.shape == b.shape and a.dtype == b.dtype, k
        if a.dtype.kind in "iu":
            assert np.array_equal(a, b), k
        else:
            err = float(np.abs(a.astype(np.float64) - b).max()) if a.size else 0.0
            print(f"   {k}: max |release - debug| {err:.3g}", flush=True)
            assert err <= RTOL * max(1.0, float(np.abs(a).max())), (k, err)
