"""The host-side C++ (page pool, working sets, fork, truncation, the prefix
registry and the batch packer, reached through a host-only context) run under
AddressSanitizer and UndefinedBehaviorSanitizer: the host ABI tests are run
again, in a child process, against libpie_asan.so (built by
`python -m paged_kv_forward_amd.build --sanitize`, host code instrumented) with
the clang ASan runtime preloaded.  Any report aborts the child and fails this
test.  No GPU is touched."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_abi_under_asan_and_ubsan():
    from paged_kv_forward_amd import build as b
    if not os.path.exists(b.LIB_ASAN) or os.path.getmtime(b.LIB_ASAN) < max(
            os.path.getmtime(os.path.join(b.CSRC, f)) for f in b.SOURCES):
        b.build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=b.asan_runtime(), PIE_LIBRARY=b.LIB_ASAN,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = ("import sys, ctypes; from paged_kv_forward_amd import _native as N; "
            "assert N.LIB_PATH.endswith('libpie_asan.so'); "
            "N.lib(); maps = open('/proc/self/maps').read(); "
            "assert 'libclang_rt.asan' in maps and 'libpie_asan.so' in maps; "
            "import pytest; sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', "
            "'tests/test_host_abi.py']))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    print(r.stdout[-3000:], r.stderr[-3000:])
    assert r.returncode == 0, "sanitized host ABI run failed"
    assert "passed" in r.stdout and "failed" not in r.stdout
