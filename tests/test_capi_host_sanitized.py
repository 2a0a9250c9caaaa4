"""The C ABI's host layer under AddressSanitizer and UndefinedBehaviorSanitizer.

``build()`` also compiles capi.cpp (every argument check, the int64 range and
alias arithmetic, the store bookkeeping) with g++ -fsanitize=address,undefined
into ``libattnres_hostsan.so``, whose launchers launch nothing.  These tests run
the host-side C-ABI suite (tests/test_capi_host.py) in a child process with that
build loaded and the ASan runtime preloaded; any sanitizer report aborts the
child.  CPU only.
"""

from __future__ import annotations

import os
import subprocess
import sys

import pytest

from depth_wise_attention_block_amd import build

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(build.HOSTSAN_LIB),
                                reason="libattnres_hostsan.so not built (build() compiles it)")


def _run(args, timeout=600):
    return subprocess.run([sys.executable, *args], cwd=REPO, env=build.sanitizer_env(), stdout=subprocess.PIPE,
                          stderr=subprocess.STDOUT, text=True, timeout=timeout)


def test_child_loads_the_sanitized_build():
    """The child's binding loads the sanitized host library, with the ASan runtime mapped."""
    code = ("import sys; sys.path.insert(0, '.'); from depth_wise_attention_block_amd import binding as B; "
            "B.lib(); maps = open('/proc/self/maps').read(); "
            "print('hostsan' if 'libattnres_hostsan.so' in maps else 'other', 'asan' if 'libasan' in maps else 'none', "
            "B.version())")
    p = _run(["-c", code])
    assert p.returncode == 0, p.stdout
    assert "hostsan asan" in p.stdout


def test_host_abi_suite_clean_under_asan_ubsan():
    p = _run(["-m", "pytest", "tests/test_capi_host.py", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"])
    assert p.returncode == 0, p.stdout[-4000:]
    assert "AddressSanitizer" not in p.stdout and "runtime error" not in p.stdout, p.stdout[-4000:]
    assert " passed" in p.stdout
