"""The host ABI tests again, against a build whose host-side C++ (argument
checking, the codebook, the trace log, the device cache) carries
AddressSanitizer and UndefinedBehaviorSanitizer.

The sanitized library loads only into a process that preloads the clang ASan
runtime, so the ABI tests run in a child interpreter with that runtime
preloaded and QN_LIBRARY pointing at the sanitized build.  Any report (a heap
overflow, a use after free, undefined behaviour) ends the child with an error:
UndefinedBehaviorSanitizer is built not to recover.  Device code is never
instrumented, and nothing here runs a kernel.
"""

import os
import shutil
import subprocess
import sys

import pytest

from bit_nf4_quantized_08_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(not os.path.isfile(build.hipcc()) or shutil.which("python3") is None, reason="no hipcc")
def test_host_abi_under_address_and_undefined_behaviour_sanitizers():
    runtime = build.sanitizer_runtime()
    if runtime is None:
        pytest.skip("clang ASan runtime not found")
    lib = build.build_sanitized()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": runtime,
        "QN_LIBRARY": lib,
        # the interpreter itself is not instrumented and keeps memory until exit
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1:verify_asan_link_order=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    # the child really runs the instrumented build with the runtime in place
    probe = ("import ctypes; from bit_nf4_quantized_08_amd import lib; L = lib.load(); "
             "print(lib.LIB_PATH); print(hasattr(ctypes.CDLL(None), '__asan_init'))")
    p = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert p.returncode == 0, (p.stdout + p.stderr)[-4000:]
    assert p.stdout.split() == [lib, "True"], p.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_host_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
