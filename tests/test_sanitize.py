"""The C ABI layer's host code and the CPU oracle under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/sanitize/build.sh builds a C driver that
runs the ABI's validation paths (every bad problem, NULL or misaligned
pointer and short workspace, the allocation-free call beyond its scratch),
workspace sizing and many-row plans of valid problems, and the oracle on the
hand-worked d = 4 case and random integer inputs. No GPU is used."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/lib/llvm/bin/clang"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")

pytestmark = pytest.mark.skipif(not os.path.exists(CLANG), reason="no ROCm clang")


def _library_objects():
    from dsa_top_token_amd import build
    objs = [os.path.join(build.PKG, "_build", s + ".o") for s in build.SOURCES]
    if not all(os.path.exists(o) for o in objs):
        build.build_library()


def test_sanitizers_are_live(tmp_path):
    # the toolchain's sanitizers do fire: a heap overflow and a signed
    # overflow planted in a throwaway program are both reported
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\n#include <limits.h>\n"
                   "int main(int c, char** v) { volatile int* a = malloc(4 * sizeof(int));\n"
                   "  if (c > 1) { int x = INT_MAX; x += c; return x; }\n"
                   "  a[4] = 1; int r = a[4]; free((void*)a); return r; }\n")
    for san, args, report in (("address", [], "AddressSanitizer: heap-buffer-overflow"),
                              ("undefined", ["x"], "signed integer overflow")):
        exe = tmp_path / ("planted_" + san)
        subprocess.run([CLANG, "-O1", "-g", "-fsanitize=" + san, "-fno-sanitize-recover=all",
                        str(src), "-o", str(exe)], check=True)
        r = subprocess.run([str(exe), *args], capture_output=True, text=True, env=ENV)
        assert r.returncode != 0 and report in r.stderr, r.stderr


def test_abi_and_oracle_under_sanitizers():
    _library_objects()
    b = subprocess.run(["bash", os.path.join(SAN, "build.sh")], capture_output=True, text=True)
    assert b.returncode == 0, b.stdout + b.stderr
    r = subprocess.run([os.path.join(SAN, "_build", "host_check")], capture_output=True,
                       text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ALL CHECKS PASSED" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
