"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

area_host.cpp (validation, the integer schedule, workspace layouts, the entry
points) and area_sizes.cpp are compiled with g++ -fsanitize=address,undefined
together with tests/sanitize/launch_stub.cpp, which replaces every kernel
launcher by a host routine that touches the buffer regions the kernels would
read or write.  In a process with the sanitizer runtime preloaded, the
schedule, validation and workspace tests of test_host_abi.py run against this
library, then every device entry point runs on exactly-sized host buffers
(tests/sanitize/drive_entry_points.py).  Any out-of-bounds access,
overlapping workspace regions or undefined behaviour fails the test."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "resolution_diffusion_transformer_amd", "csrc")


def _runtime():
    out = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return out if out and os.path.isabs(out) and os.path.exists(out) else None


@pytest.fixture(scope="module")
def sanitized_library(tmp_path_factory):
    if not shutil.which("g++") or not _runtime():
        pytest.skip("g++ with the AddressSanitizer runtime is not available")
    lib = str(tmp_path_factory.mktemp("sanitize") / "libarea_host_sanitized.so")
    cmd = ["g++", "-std=c++17", "-shared", "-fPIC", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "area_host.cpp"), os.path.join(CSRC, "area_sizes.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "launch_stub.cpp"), "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return lib


def _env(lib):
    env = dict(os.environ)
    env.update(AREA_LIBRARY=lib, LD_PRELOAD=_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


def _clean(out):
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]


def test_host_abi_suite_under_sanitizers(sanitized_library):
    r = subprocess.run([sys.executable, "-c",
                        "import sys; sys.modules['torch'] = None; import pytest; "
                        "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu', "
                        "'tests/test_host_abi.py']))"],
                       cwd=ROOT, env=_env(sanitized_library), capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    _clean(out)
    assert r.returncode == 0, out[-4000:]


def test_every_entry_point_under_sanitizers(sanitized_library):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize", "drive_entry_points.py")],
                       cwd=ROOT, env=_env(sanitized_library), capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    _clean(out)
    assert r.returncode == 0 and "all entry points ok" in out, out[-4000:]
