"""The C-ABI layer under host AddressSanitizer: api.cpp (argument validation,
layouts, error messages, the launch-timing records) is rebuilt with the
sanitizer and the host-side ABI tests run against that build in a child
process with the sanitizer runtime preloaded.  No GPU is used: the ABI tests
launch no kernel."""
import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT


def _libasan():
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_abi_host_tests_pass_under_host_asan(tmp_path):
    asan = _libasan()
    if asan is None:
        pytest.skip("no libasan.so for the host compiler")
    from grouped_gemm_mxfp8_amd._build import build_host_asan
    lib = build_host_asan(str(tmp_path))
    env = dict(os.environ)
    env.update({"MXMOE_LIB": lib, "LD_PRELOAD": asan,
                # the HIP runtime and the interpreter keep allocations to exit
                "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1"})
    # the child loads the sanitized build, with the sanitizer runtime
    probe = ("import grouped_gemm_mxfp8_amd as gm; gm.lib(); "
             "m = open('/proc/self/maps').read(); "
             "print(gm.LIB_PATH in m, 'libasan' in m)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.stdout.split() == ["True", "True"], (r.stdout, r.stderr[-2000:])
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    print(r.stdout[-2000:], r.stderr[-2000:])
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "AddressSanitizer" not in r.stderr
    assert " passed" in r.stdout
