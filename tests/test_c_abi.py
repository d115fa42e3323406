"""The C ABI used from plain C programs (no Python, no torch): a host-only one in
the CPU suite, and a GPU one that runs the device-commit step through the HIP
runtime's C API and compares it with the oracle's C entry point bit for bit."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "zero_partitioned_optimizer_amd")
ROCM = "/opt/rocm"


def _lib():
    path = os.path.join(PKG, "libzero.so")
    if not os.path.exists(path):
        from zero_partitioned_optimizer_amd import build
        build.build()
    return path


def _compile(src, out, extra):
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", src), "-L", PKG, "-l:libzero.so",
           "-Wl,-rpath," + PKG, *extra, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_host_abi_from_c(tmp_path):
    _lib()
    exe = tmp_path / "abi_host"
    _compile("abi_host.c", exe, [])
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stderr
    assert "abi_host ok" in res.stdout


@pytest.mark.gpu
def test_device_step_from_c_matches_oracle(Z, tmp_path):
    _lib()
    import oracle
    oracle.build(force=False)
    exe = tmp_path / "step_parity"
    _compile("step_parity.c", exe,
             ["-D__HIP_PLATFORM_AMD__", "-I", f"{ROCM}/include", "-L", os.path.join(ROOT, "oracle"),
              "-l:liboracle.so", "-Wl,-rpath," + os.path.join(ROOT, "oracle"), "-L", f"{ROCM}/lib",
              "-lamdhip64", "-Wl,-rpath," + f"{ROCM}/lib", "-lm"])
    print("[gpu-test] C program: device-commit step vs oracle (S=100003, N=8, 3 steps)", flush=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(res.stdout, flush=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "step_parity ok" in res.stdout

