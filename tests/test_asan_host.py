"""The host side of the C ABI (argument validation, error strings, the
per-device scratch lookup) under AddressSanitizer: build libsws_asan.so
(sws_api.hip's host code instrumented, GPU code unchanged) and run the
host-validation tests of test_abi.py against it in a child process with the
ASan runtime preloaded.  No GPU needed."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

hipcc_missing = not (os.path.exists("/opt/rocm/bin/hipcc") or shutil.which("hipcc"))


@pytest.mark.skipif(hipcc_missing, reason="hipcc is needed to build the sanitizer variant")
def test_abi_validation_under_host_asan():
    sys.path.insert(0, ROOT)
    from dynamic_block_sparse_sws_amd import build as B
    lib = B.build_asan()
    runtime = B.asan_runtime()
    env = dict(os.environ)
    env.update({"SWS_LIBRARY": lib, "LD_PRELOAD": runtime,
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1"})
    check = ("import dynamic_block_sparse_sws_amd as s; "
             "assert s.LIB_PATH.endswith('libsws_asan.so'); s.lib(); print('asan library loaded')")
    r = subprocess.run([sys.executable, "-c", check], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0 and "asan library loaded" in r.stdout, r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "AddressSanitizer" not in r.stderr
