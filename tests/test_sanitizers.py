"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two legs, each in a child process that preloads the sanitizer runtime its
library was built against (a finding aborts the child, so the test fails):

* the oracle (plain C) built by gcc with -fsanitize=address,undefined, running
  every pin of tests/test_oracle.py;
* the library's host code (argument checks, the host-built split partition,
  mla_split_plan, launch set-up) built by hipcc with the host half
  instrumented, running tests/test_abi.py, which drives those paths without a
  device.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_child(test_file, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", test_file)], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "passed" in r.stdout, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out


def test_oracle_under_asan_ubsan():
    import oracle

    lib = oracle.build_sanitized()
    asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc has no libasan")
    _run_child("test_oracle.py", {"LD_PRELOAD": asan, "MLA_ORACLE_LIBRARY": lib})


def test_library_host_code_under_asan_ubsan():
    from mla_latent_kv_fp8_amd import build

    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rts:
        pytest.skip("no clang ASan runtime under /opt/rocm/llvm")
    lib = build.build(sanitize=True)
    _run_child("test_abi.py", {"LD_PRELOAD": rts[-1], "LD_LIBRARY_PATH": os.path.dirname(rts[-1]),
                               "MLA_FP8_LIBRARY": lib})
