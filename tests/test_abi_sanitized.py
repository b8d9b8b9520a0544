"""The host validation of every entry point, run under AddressSanitizer and
UndefinedBehaviorSanitizer: the sources are rebuilt with the host side
instrumented, and the C-ABI rule tests (tests/test_abi_host.py) run against
that library in a child process with the sanitizer runtime preloaded.  Any
sanitizer report fails the child.  CPU only: no kernel is launched."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="the fake-pointer host checks run only without a GPU")
@pytest.mark.timeout(600)
def test_abi_rules_under_address_and_ub_sanitizers():
    from block_draft_head_amd import build as B
    out = os.path.join(ROOT, "block_draft_head_amd", "_build", "host_sanitized")
    lib = B.build_host_sanitized(out, jobs=min(8, os.cpu_count() or 1))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_handle" in syms, "the library is not instrumented"
    env = dict(os.environ)
    env.update(DFLASH2_LIBRARY=lib, LD_PRELOAD=B.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-x",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=500)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "skipped" not in r.stdout.split("\n")[-2], tail
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, tail
