"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

capi.cpp, chooser.cpp and bank_model.cpp (argument checks, overflow and
overlap tests, the chooser's search, the bank model) are compiled with g++
and -fsanitize=address,undefined, linked with stand-ins for the kernel
launchers (tests/host_stubs.cpp), and the host tests of the C ABI
(tests/test_capi_host.py) run against that library in a child process with
the sanitizer runtime preloaded; any report fails the child (halt_on_error).
No GPU code is built or run: this is the host side only.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tiled_movement_amd", "csrc")
HOST_SOURCES = ["capi.cpp", "chooser.cpp", "bank_model.cpp"]


def _gxx():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.fail("g++ is needed for the sanitizer build")
    return gxx


def test_c_abi_host_tests_run_clean_under_asan_and_ubsan(tmp_path):
    gxx = _gxx()
    pkg = tmp_path / "tiled_movement_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "tiled_movement_amd", "__init__.py"), pkg / "__init__.py")
    flags = ["-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all",
             "-fsanitize=address,undefined", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
             f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]
    srcs = [os.path.join(CSRC, s) for s in HOST_SOURCES] + [os.path.join(ROOT, "tests", "host_stubs.cpp")]
    subprocess.run([gxx, *flags, "-shared", "-o", str(pkg / "libswz.so"), *srcs], check=True)
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    ubsan = subprocess.run([gxx, "-print-file-name=libubsan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ)
    # the sanitizer runtimes must come first; anything already preloaded stays
    env["LD_PRELOAD"] = " ".join(p for p in (asan, ubsan, env.get("LD_PRELOAD", "")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"  # the interpreter's own allocations
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    # the sanitized package first on the path; the tests import it as tiled_movement_amd
    env["PYTHONPATH"] = os.pathsep.join([str(tmp_path), ROOT, env.get("PYTHONPATH", "")])
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_capi_host.py")],
                       cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert str(pkg / "libswz.so") in subprocess.run(
        [sys.executable, "-c", "import tiled_movement_amd as T; print(T.LIB_PATH)"],
        cwd=str(tmp_path), env=env, capture_output=True, text=True).stdout  # it really loaded the sanitized build
