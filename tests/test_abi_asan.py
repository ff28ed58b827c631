"""The C-ABI layer under AddressSanitizer: tests/test_abi.py run against
libdsa_asan.so (abi.cpp's host code instrumented, the kernels unchanged),
in a child process with the sanitizer's runtime preloaded.  Any heap or
stack error in the host-side validation, workspace carving or error
reporting makes the sanitizer abort the child."""
import os
import subprocess
import sys

from sparse_attention_18_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_suite_under_address_sanitizer():
    lib = build.build_asan_library()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms, "libdsa_asan.so is not instrumented"
    env = dict(os.environ, LD_PRELOAD=build.asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from sparse_attention_18_amd import binding\n"
            "binding._LIB_PATH = %r\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_abi.py']))\n") % (ROOT, lib)
    res = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True, text=True,
                         timeout=600)
    assert "AddressSanitizer" not in res.stderr, res.stderr[-4000:]
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert " passed" in res.stdout
