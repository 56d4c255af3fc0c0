"""Host sanitizers (no GPU): the oracle's pin suites run against an
AddressSanitizer + UndefinedBehaviorSanitizer build of the oracle, and the C-ABI
validation tests run against a build of libhc.so whose host code carries the same
sanitizers. Every sanitizer finding aborts the child process, so the suites fail.

Each suite runs in a child process with the sanitizer runtime preloaded (the
Python interpreter itself is not instrumented) and leak checking off (the
interpreter keeps its allocations until exit).
"""
import os
import subprocess
import sys

import pytest
import torch

import oracle
from hyper_connection_residual_mixes_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = dict(ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(env, *tests):
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *(os.path.join(ROOT, "tests", t) for t in tests)],
                       cwd=ROOT, env=dict(os.environ, **SAN_ENV, **env), capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, f"sanitized run failed:\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    assert "passed" in r.stdout


def test_oracle_pins_under_asan_ubsan(tmp_path):
    gcc = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(gcc):
        pytest.skip("gcc's ASan runtime is not installed")
    lib = oracle.build(sanitize=True, out=str(tmp_path / "liboracle_hc_san.so"))
    _run(dict(HC_ORACLE_LIB=lib, LD_PRELOAD=gcc), "test_oracle_pins.py", "test_oracle_generic_hc.py")


@pytest.mark.skipif(torch.cuda.is_available(), reason="the ABI host tests pass fake device pointers")
def test_abi_validation_under_host_asan_ubsan(tmp_path):
    lib = hip_build.build_host_sanitized(str(tmp_path / "libhc_san.so"))
    _run(dict(HC_LIBRARY=lib, LD_PRELOAD=hip_build.sanitizer_runtime()), "test_abi_host.py")
