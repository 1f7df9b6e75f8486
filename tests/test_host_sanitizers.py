"""The host-side validation and planning code of the C ABI (shape, alignment
and workspace checks, the layer's kernel and LDS plan, the scratch limit, the
per-entry-point launch counts) run under AddressSanitizer and
UndefinedBehaviorSanitizer: the library is rebuilt with host-only sanitizers
(device code as usual) and the C-ABI tests run against it in a child process
that preloads the sanitizer runtime.  Any sanitizer report aborts the child."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.slow


def test_c_abi_host_code_is_clean_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from quantized_moe_weight_amd import build as b
    lib = b.build(sanitize=True)
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in nm and "__ubsan_" in nm, "the library was not built with the sanitizers"
    env = dict(os.environ, LD_PRELOAD=b.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = ("import sys; sys.path[:0] = [{root!r}, {tests!r}]\n"
            "from quantized_moe_weight_amd import _lib\n"
            "_lib.load({lib!r})\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', {abi!r}]))\n").format(
        root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib, abi=os.path.join(ROOT, "tests", "test_abi.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
