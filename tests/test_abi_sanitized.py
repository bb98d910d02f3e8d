"""The C ABI tests (tests/test_abi.py), the host proxy's parity tests
(tests/test_proxy_parity.py) and the launch planner's tests
(tests/test_plan.py) run against a build whose host-side layer -- argument
validation, alias and alignment checks, byte-size helpers, the host
conversions, rq_proxy, the small-M planner -- is compiled with
AddressSanitizer and UndefinedBehaviorSanitizer (CPU only: no call reaches a
kernel).  Any sanitizer report fails the run."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_abi_under_address_and_undefined_sanitizers():
    from gemm_rwkv_amd import build
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc not available")
    lib = build.build_sanitized(verbose=False)
    rt = build.sanitizer_runtime()
    assert rt, "no AddressSanitizer runtime found"
    env = dict(os.environ)
    env.update({
        "RQ_LIBRARY": lib,
        "LD_PRELOAD": rt,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "HIP_VISIBLE_DEVICES": "",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        os.path.join(ROOT, "tests", "test_proxy_parity.py"),
                        os.path.join(ROOT, "tests", "test_plan.py"), "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
