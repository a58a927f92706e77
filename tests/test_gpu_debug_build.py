"""The bounds-checked debug build (libhst_debug.so: HST_DEBUG, every check
recording into one device word, see csrc/hst_common.h) on the decode path.

A child process loads it (HST_LIBRARY=debug) and runs tests/debug_cases.py:
soft-LSH hashing and decode over a ragged bf16 batch and the fp32 tiny case,
the routed step on the ragged batch, attention over given rows, binary codes
and their decode step, and a stand-alone top-k with ties.  No check may fail, and every result must equal
the release library's on the same inputs (the checks only observe)."""
import os
import subprocess
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_debug_build_checks_pass_and_match_release(tmp_path):
    import hash_scored_top_amd as hst
    from tests.debug_cases import run_cases
    dbg = os.path.join(ROOT, "hash_scored_top_amd", "libhst_debug.so")
    assert os.path.exists(dbg), "libhst_debug.so is not built (build() builds it)"
    out = tmp_path / "dbg.npz"
    env = dict(os.environ, HST_LIBRARY="debug")
    print("[debug-build] child run", flush=True)
    p = subprocess.run([sys.executable, "-u", "-m", "tests.debug_cases", str(out)], cwd=ROOT, env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=110)
    print(p.stdout[-2000:], flush=True)
    assert p.returncode == 0, p.stdout[-2000:]
    got = dict(np.load(out))
    assert int(got.pop("debug_word")[0]) == 0
    # the release build in this process, same cases
    assert hst.LIB_PATH.endswith("libhst.so")
    ref = run_cases(hst)
    with pytest.raises(hst.HstError):
        hst.debug_status()  # the release library has no checks
    assert set(ref) == set(got)
    for k in ref:
        if k.endswith(("_out", "_lse", "_out_given", "_vn")):
            np.testing.assert_allclose(got[k], ref[k], rtol=1e-6, atol=1e-7, err_msg=k)
        else:
            assert np.array_equal(got[k], ref[k]), k
