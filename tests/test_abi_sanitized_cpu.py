"""The C ABI's argument validation under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only; no GPU needed). A child process with the ASan runtime preloaded loads
the sanitized build of the library (bit_quantized_lora_fp4_amd.build_sanitize, made by
__graft_entry__.build()) in place of the product library and runs the host-side ABI
tests against it: every rejected call, the workspace-size queries, the size helpers
and the status strings; any sanitizer report aborts the child."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_LIB = os.path.join(ROOT, "bit_quantized_lora_fp4_amd", "_build", "san", "libfourtune_san.so")
HEADER_TESTS = ["tests/test_abi_cpu.py"]

CHILD = """
import sys
sys.path.insert(0, {root!r})
from bit_quantized_lora_fp4_amd import abi
abi.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-s", "-p", "no:cacheprovider", *{tests!r}]))
"""


def test_abi_validation_under_sanitizers():
    if not os.path.exists(SAN_LIB):
        pytest.skip("sanitized library not built (__graft_entry__.build() builds it)")
    from bit_quantized_lora_fp4_amd.build_sanitize import asan_runtime
    env = dict(os.environ, LD_PRELOAD=asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = CHILD.format(root=ROOT, lib=SAN_LIB, tests=HEADER_TESTS)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "passed" in r.stdout
