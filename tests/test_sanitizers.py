"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C ABI's host side (the argument checks of every entry point, the
kernel-family choice, the block manager) and the CPU oracle are rebuilt with
gcc / g++ -fsanitize=address,undefined (-fno-sanitize-recover=all), and the
CPU suites that exercise them (test_abi.py, test_block_manager.py,
test_oracle_pins.py) run against those builds in a child process with the
sanitizer runtimes preloaded.  Kernel launches cannot happen in that build:
the stand-ins of tests/sanitize/host_stubs.cpp refuse them and count the
attempts, and the run checks that no test reached one.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_267_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _runtime(name: str) -> str:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else ""


@pytest.fixture(scope="module")
def sanitized_builds(tmp_path_factory):
    if not shutil.which("gcc") or not shutil.which("g++"):
        pytest.skip("gcc / g++ not available")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not installed")
    out = tmp_path_factory.mktemp("san")
    host = str(out / "libpa_host_san.so")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-Wall",
                    "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *SAN, "-o", host,
                    os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "dispatch.cpp"),
                    os.path.join(CSRC, "block_manager.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp")], check=True)
    ora = str(out / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                    "-D_DEFAULT_SOURCE", "-Wall", *SAN, "-o", ora,
                    os.path.join(ROOT, "oracle", "pa_oracle.c"), "-lm"], check=True)
    return host, ora, asan, ubsan


CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import pytest
import paged_kv_cache_267_amd as pa
import oracle
pa.LIB_PATH = {host!r}
oracle._LIB_PATH = {ora!r}
rc = pytest.main(["-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider", *{tests!r}])
launches = pa.lib().pa_host_stub_launches()
print(f"[sanitized] pytest rc={{rc}} refused launches={{launches}}", flush=True)
sys.exit(int(rc) if rc else (3 if launches else 0))
"""


def test_host_code_and_oracle_under_sanitizers(sanitized_builds):
    host, ora, asan, ubsan = sanitized_builds
    tests = [os.path.join(ROOT, "tests", t) for t in
             ("test_abi.py", "test_block_manager.py", "test_oracle_pins.py")]
    env = dict(os.environ)
    env["LD_PRELOAD"] = f"{asan}:{ubsan}"
    # the interpreter and torch are not instrumented and keep memory until exit
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = CHILD.format(root=ROOT, host=host, ora=ora, tests=tests)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=900)
    log = r.stdout + r.stderr
    print(log[-3000:])
    assert "ERROR: AddressSanitizer" not in log and "runtime error:" not in log, log[-3000:]
    assert r.returncode == 0, log[-3000:]
    assert "[sanitized] pytest rc=0 refused launches=0" in log
