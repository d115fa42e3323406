"""Host code under AddressSanitizer and UBSan (CPU only, gcc/g++, no HIP).

The layout code of the library (csrc/layout.cpp) and the oracle (oracle/oracle.c)
are built for the host with both sanitizers and driven by a differential fuzzer
(tests/c/layout_fuzz.cpp): every offset, size, segment, bucket and memory figure
of 3000 random layouts must agree, and no sanitizer may report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "zero_partitioned_optimizer_amd")


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="host compilers not available")
def test_layout_differential_fuzz_under_sanitizers(tmp_path):
    """layout.cpp and oracle.c built for the host with AddressSanitizer and UBSan
    (gcc/g++, no HIP), compared on 3000 random layouts."""
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-g", "-O1"]
    obj = tmp_path / "oracle.o"
    subprocess.run(["gcc", "-std=c11", "-ffp-contract=off", *san, "-c",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", str(obj)],
                   check=True, capture_output=True, text=True)
    exe = tmp_path / "layout_fuzz"
    subprocess.run(["g++", "-std=c++17", *san, "-I", os.path.join(ROOT, "include"),
                    os.path.join(PKG, "csrc", "layout.cpp"),
                    os.path.join(ROOT, "tests", "c", "layout_fuzz.cpp"), str(obj), "-lm", "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([str(exe), "3000", "7"], capture_output=True, text=True, timeout=240, env=env)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "layout_fuzz ok" in res.stdout
