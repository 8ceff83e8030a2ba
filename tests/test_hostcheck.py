"""The C ABI's host code (argument checks, workspace plans and carving, the no-allocation entry's
checks) under AddressSanitizer and UndefinedBehaviorSanitizer: builds the sanitized check program
(hierarchical_kv_indexer_amd/build.py --hostcheck) and runs it.  It needs hipcc but no GPU, and it
refuses to run where a GPU is present (its valid calls would launch kernels on fake addresses)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_host_code_under_sanitizers():
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc is not available")
    import torch
    if torch.cuda.is_available():
        pytest.skip("the sanitized check runs only on a machine without a GPU")
    from hierarchical_kv_indexer_amd import build
    exe = build.build_hostcheck()
    env = dict(os.environ)
    # the HIP runtime keeps allocations for the process's lifetime: leaks are not this check's subject
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env, cwd=ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert ", 0 failed" in out, out[-2000:]
