"""The CPU code of the path under AddressSanitizer and UndefinedBehaviorSanitizer
(host compilers only; no GPU code is built with them).

* The fp64 oracle (oracle/moe_oracle.c), driven by tests/sanitize/oracle_check.c
  over small problems, thread counts, token subsets and argument errors.
* The library's host code (csrc/api.cpp: argument checks, workspace carving,
  launch sequencing of every entry point), with the HIP runtime calls and the
  kernel launchers replaced by the stand-ins of tests/sanitize/host_stubs.cpp,
  driven by tests/sanitize/host_check.cpp over valid and invalid problems;
  the stand-ins check that every workspace array a launch is handed lies in
  the workspace.

Two control programs (a heap overflow, a signed overflow) show that each
sanitizer is active in these builds at all."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "w4a16_int4_grouped_moe_amd", "csrc")
ROCM_INC = "/opt/rocm/include"
FLAGS = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=undefined"]
ENV = dict(os.environ,
           ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")

pytestmark = pytest.mark.skipif(not (shutil.which("gcc") and shutil.which("g++")),
                                reason="host compilers not found")


def build(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-3000:]


def run(exe):
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    out = res.stdout + res.stderr
    return res.returncode, out


@pytest.mark.parametrize("kind,code,report", [
    ("address", "volatile int *p = malloc(8 * sizeof(int)); p[8] = 1; free((void *)p);",
     "AddressSanitizer: heap-buffer-overflow"),
    ("undefined", "volatile int x = INT_MAX; x = x + argc;", "signed integer overflow"),
])
def test_sanitizers_are_active(tmp_path, kind, code, report):
    src = tmp_path / "bad.c"
    src.write_text("#include <limits.h>\n#include <stdlib.h>\n"
                   f"int main(int argc, char **argv) {{ (void)argv; {code} return 0; }}\n")
    exe = str(tmp_path / "bad")
    build(["gcc", "-g", "-O1", f"-fsanitize={kind}", "-fno-sanitize-recover=all", str(src),
           "-o", exe])
    rc, out = run(exe)
    assert rc != 0 and report in out, out[-2000:]


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    build(["gcc", "-std=c11", *FLAGS, os.path.join(ROOT, "oracle", "moe_oracle.c"),
           os.path.join(SAN, "oracle_check.c"), "-o", exe, "-lm", "-lpthread"])
    rc, out = run(exe)
    assert rc == 0, out[-4000:]
    assert "failed: 0" in out and "runtime error" not in out and "Sanitizer" not in out, out


def test_host_code_under_sanitizers(tmp_path):
    if not os.path.isdir(ROCM_INC):
        pytest.skip("HIP headers not found")
    inc = ["-std=c++17", "-I", ROCM_INC, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-D__HIP_PLATFORM_AMD__"]
    objs = []
    # api.cpp as host C++: its one device declaration (the allocation-free
    # entry point's array) becomes a host array of the same size
    for src, extra in ((os.path.join(CSRC, "api.cpp"),
                        ["-D__align__(n)=__attribute__((aligned(n)))", "-DHIP_SYMBOL(x)=(&x)"]),
                       (os.path.join(SAN, "host_stubs.cpp"), []),
                       (os.path.join(SAN, "host_check.cpp"), [])):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        build(["g++", *inc, *FLAGS, *extra, "-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "host_check")
    build(["g++", "-fsanitize=address,undefined", *objs, "-o", exe])
    rc, out = run(exe)
    assert rc == 0, out[-4000:]
    assert "failed: 0" in out and "runtime error" not in out and "Sanitizer" not in out, out
