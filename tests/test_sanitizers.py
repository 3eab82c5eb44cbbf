"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only): the oracle built with gcc's sanitizers runs its pins, and the HIP
library built with clang's sanitizers on its host code (argument
validation, workspace carving, launch planning) runs the C-ABI and binding
checks, each suite in a process of its own with the runtime preloaded.  Any
sanitizer report aborts that process and fails the test."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
pytestmark = pytest.mark.slow


def _run(env_extra, tests):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", **env_extra)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu", *tests]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    return r.stdout


def test_oracle_pins_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    env = {"PKV_ORACLE_SANITIZE": "1"}
    subprocess.run([sys.executable, "-c", "import oracle.build as b; b.build()"], cwd=ROOT,
                   env=dict(os.environ, **env), check=True)
    pre = " ".join(subprocess.run(["gcc", "-print-file-name=" + n], capture_output=True, text=True,
                                  check=True).stdout.strip() for n in ("libasan.so", "libubsan.so"))
    out = _run(dict(env, LD_PRELOAD=pre), ["tests/test_oracle_pins.py", "tests/test_oracle_sampling.py"])
    assert "passed" in out


def test_library_host_code_under_asan_and_ubsan():
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang's ASan runtime is not installed")
    sys.path.insert(0, ROOT)
    from paged_kv_transformer_amd import build as hip_build
    lib = hip_build.build(sanitize=True)
    out = _run({"PKV_LIBRARY": lib, "LD_PRELOAD": rt[-1]},
               ["tests/test_abi_host.py", "tests/test_binding_checks.py"])
    assert "passed" in out
