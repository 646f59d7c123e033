"""Device-side bound checks of the debug build (libgmla_debug.so): in a child process on that
build, each case of debug_checks_cases.py reports exactly its expected flag bits (a token
position past the cache, a page-table entry outside the pool, none for in-range work), and every
output is identical to the normal build's, run on the same seeded inputs in this process."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
gm = pytest.importorskip("gated_mla_kv_amd")


@pytest.mark.gpu
def test_debug_build_flags_and_outputs(tmp_path):
    if not os.path.exists(gm.DEBUG_LIB_PATH):
        pytest.fail(f"{gm.DEBUG_LIB_PATH} is missing: build it with gated_mla_kv_amd.build.build()")
    import debug_checks_cases as C
    out = tmp_path / "debug.npz"
    env = dict(os.environ, GMLA_LIB=gm.DEBUG_LIB_PATH, PYTHONPATH=os.path.dirname(HERE))
    print("child: debug_checks_cases.py on libgmla_debug.so", flush=True)
    r = subprocess.run([sys.executable, os.path.join(HERE, "debug_checks_cases.py"), str(out)], env=env,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-3000:]
    rep = json.loads(r.stdout.strip().splitlines()[-1])
    assert rep["lib"] == "libgmla_debug.so" and rep["built"] is True, rep
    for name, (_, want) in C.CASES.items():
        assert rep["flags"][name] == want, (name, rep["flags"])
    # the normal build: no checks, no bits, and the same outputs
    print("parent: the same cases on libgmla.so", flush=True)
    flags, arrays, built = C.run_all()
    assert built is False and all(f == 0 for f in flags.values()), flags
    dbg = np.load(out)
    assert sorted(dbg.files) == sorted(arrays)
    for k, v in arrays.items():
        np.testing.assert_array_equal(dbg[k], v, err_msg=k)
