"""The host side of the library under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: the host runtime (argument checks,
planning, allocation set-up) is rebuilt with both sanitizers and the CPU ABI
tests run against that build in a child Python with the sanitizer runtime
preloaded.  Any report (out-of-bounds access, use after free, undefined
behaviour such as an out-of-range enumeration value) ends the child with an
error and fails this test; the C header is also compiled as C99 and C++17."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tileq.h")


@pytest.mark.parametrize("cmd", [["gcc", "-std=c99", "-x", "c"],
                                 ["g++", "-std=c++17", "-x", "c++"]])
def test_header_compiles_as_c_and_cxx(cmd):
    if shutil.which(cmd[0]) is None:
        pytest.skip(cmd[0] + " not available")
    r = subprocess.run(cmd + ["-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only", HEADER],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    assert r.returncode == 0, r.stdout.decode(errors="replace")


@pytest.mark.slow
def test_abi_tests_under_asan_ubsan(tmp_path):
    from bit_rank_post_amd import build as B
    try:
        B.hipcc()
        rt = B.asan_runtime()
    except (RuntimeError, OSError, subprocess.CalledProcessError) as e:
        pytest.skip(f"sanitizer toolchain unavailable: {e}")
    lib = B.build_asan()
    log = str(tmp_path / "sanitizer")
    env = dict(os.environ, LD_PRELOAD=rt, TILEQ_LIB_PATH=lib,
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=0:log_path={log}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={log}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       timeout=600)
    reports = [os.path.join(tmp_path, f) for f in os.listdir(tmp_path)
               if f.startswith("sanitizer")]
    text = "".join(open(f).read()[:4000] for f in reports)
    assert r.returncode == 0 and not reports, (r.stdout.decode(errors="replace")[-3000:] + text)
    assert b"passed" in r.stdout
