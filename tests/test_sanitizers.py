"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code, on
the CPU.

* The fp64 oracle (plain gcc) is rebuilt with both sanitizers and every pin
  runs against it.
* libgdn is rebuilt with both sanitizers on its host code only (the argument
  validation, workspace layout and status code paths; device code is compiled
  as usual and never launched here), and the ABI and binding validation tests
  run against it.

Each run is a child process with the sanitizer runtime preloaded (a
sanitized shared library cannot be loaded into an uninstrumented Python
otherwise); any report aborts the child (no recovery), so the child must exit
0 and print no report.
"""
import glob
import os
import subprocess
import sys

import pytest

from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
ASAN_OPTIONS = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
UBSAN_OPTIONS = "halt_on_error=1:print_stacktrace=1"
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "UndefinedBehaviorSanitizer")


def _child(code, preload, cwd=ROOT, timeout=600):
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS=ASAN_OPTIONS,
               UBSAN_OPTIONS=UBSAN_OPTIONS)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         timeout=timeout, env=env, cwd=cwd)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    for r in REPORTS:
        assert r not in out, out[-4000:]
    return out


def _gcc_runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc has no %s here" % name)
    return path


PINS_CHILD = r"""
import sys
sys.path[:0] = [%r, %r]
import oracle, oracle_pins
lib = oracle.load(%r)
for pin in oracle_pins.ALL_PINS:
    pin(lib)
    print("pin ok", pin.__name__, flush=True)
"""


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = oracle_build.build(
        oracle_build.SRC, str(tmp_path / "liboracle_san.so"),
        extra=("-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=all"))
    out = _child(PINS_CHILD % (ROOT, TESTS, lib), _gcc_runtime("libasan.so"))
    assert out.count("pin ok") >= 10, out[-2000:]


ABI_CHILD = r"""
import ctypes, sys
sys.path[:0] = [%r, %r]
from gated_deltanet_chunkwise_amd import _binding
_binding._LIB_PATH = %r
_binding._LIB = None
_binding.load_library()
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "tests/test_abi.py",
                      "tests/test_binding_host.py"]))
"""


def _clang_asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        pytest.skip("no clang ASan runtime under /opt/rocm/llvm")
    return found[-1]


def test_host_validation_under_asan_ubsan(tmp_path):
    from gated_deltanet_chunkwise_amd import build as hip_build
    # sanitizers on the host pass only: each -fsanitize flag goes to the host
    # compiler through -Xarch_host (the device code is built as usual)
    flags = ["-O1", "-g",
             "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xarch_host", "-fno-omit-frame-pointer"]
    lib = hip_build.build(out=str(tmp_path / "libgdn_host_san.so"), extra=flags)
    out = _child(ABI_CHILD % (ROOT, TESTS, lib), _clang_asan_runtime())
    assert " passed" in out, out[-2000:]
