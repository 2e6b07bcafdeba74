"""The library's test and debug switches.

HHR_TEST_FAIL=<text> makes every launch whose name contains <text> ("*": all)
fail with HHR_E_HIP before anything is enqueued, so callers' error paths run
without a GPU; these tests are CPU-only and pass fake device pointers that
are never dereferenced.  HHR_DEBUG_SYNC=1 synchronizes and checks after
every launch; its GPU test runs the smoke check under it.  Both are read
once per process, so each case runs in a subprocess.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# A decode step and a qprep stage on fake, aligned pointers: every argument check passes, so the call
# reaches its first launch.
SNIPPET = textwrap.dedent("""
    import ctypes, sys
    sys.path.insert(0, {root!r})
    import hash_sparse_attention_amd as hsa
    L = hsa.lib()
    d = hsa.make_dims(1, 32, 8, 128, 16, 128, 131072, True)
    FAKE = ctypes.c_void_p(0x10000)
    n = hsa.workspace_bytes(d, 820, 4096)
    which = sys.argv[1]
    if which == "qprep":
        st = L.hhr_stage_qprep(ctypes.byref(d), FAKE, FAKE, FAKE, 820, 4096, FAKE, n, None)
    else:
        st = L.hhr_decode_step(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 820, 4096,
                               0.0, FAKE, None, FAKE, n, None)
    print(st)
    print(L.hhr_last_error().decode())
    try:
        hsa._check(st)
    except hsa.HHRError as e:
        print("raised", e.status)
""")


def run_snippet(which, env):
    r = subprocess.run([sys.executable, "-c", SNIPPET.format(root=ROOT), which], capture_output=True, text=True,
                       timeout=300, env={**os.environ, **env})
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stdout.strip().splitlines()


# Only the first launch of each call is targeted, so no case ever reaches a real launch on fake pointers.
@pytest.mark.parametrize("target,which,stage", [("qprep", "qprep", "qprep launch"),
                                                 ("*", "step", "qprep launch"),
                                                 ("qprep", "step", "qprep launch")])
def test_forced_failure_before_the_named_launch(target, which, stage):
    out = run_snippet(which, {"HHR_TEST_FAIL": target})
    assert out[0] == "8"  # HHR_E_HIP
    assert out[1] == f"{stage}: failed on purpose (HHR_TEST_FAIL={target})"
    assert out[2] == "raised 8"


def test_hip_error_path_of_the_binding():
    """The Python layer turns the status into HHRError with the library's message."""
    import hash_sparse_attention_amd as hsa
    with pytest.raises(hsa.HHRError) as e:
        hsa._check(8)
    assert e.value.status == 8 and str(e.value).startswith("HHR_E_HIP")


@pytest.mark.gpu
def test_smoke_under_debug_sync():
    """Every launch synchronized and checked: the smoke step still matches the oracle."""
    r = subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; g.smoke()"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300, env={**os.environ, "HHR_DEBUG_SYNC": "1"})
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
