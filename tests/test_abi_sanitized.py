"""The C-ABI tests (tests/test_abi.py: argument validation, plans, workspace
layout, the prepared-call cache, no GPU) run again against a build of the
library whose host code is compiled with AddressSanitizer and
UndefinedBehaviorSanitizer (microscaled_mxfp4_block_amd.build_sanitized), in
a subprocess with the ASan runtime preloaded; any sanitizer report fails it.
CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_suite_under_host_sanitizers(tmp_path):
    from microscaled_mxfp4_block_amd import build_sanitized as S
    lib = S.LIB
    srcs = [os.path.join(S.B.CSRC, f) for f in os.listdir(S.B.CSRC)] + [os.path.join(ROOT, "include", "mx4.h")]
    if not os.path.exists(lib) or os.path.getmtime(lib) < max(os.path.getmtime(p) for p in srcs):
        S.build()
    env = dict(os.environ)
    env.update({
        "MX4_LIBRARY": lib,
        "LD_PRELOAD": S.asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=99",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=98",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                        "-p", "no:cacheprovider", "-k", "not fast_call"],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    out = r.stdout
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
