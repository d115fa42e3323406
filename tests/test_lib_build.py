"""Build-level checks of the gfx950 kernels (CPU only: hipcc cross-compiles).

Every kernel must run without private (scratch) memory: a spill or an argument
block copied to the stack turns the streaming step into a scratch-bound one."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
@pytest.mark.parametrize("source,kernel", [("step_kernels.hip", "k_step"),
                                           ("gather_kernels.hip", "k_gather")])
def test_kernels_use_no_scratch(tmp_path, source, kernel):
    from zero_partitioned_optimizer_amd import build as B
    src = os.path.join(B.CSRC, source)
    flags = [f for f in B.HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [B.hipcc(), *flags, "-I", os.path.join(ROOT, "include"), "-I", B.CSRC, "-c", src,
           "-o", str(tmp_path / "k.o"), "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True, check=True).stderr
    names = re.findall(r"Function Name: (\S+)", out)
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", out)]
    assert names and len(names) == len(scratch)
    assert any(kernel in n for n in names)
    bad = [(n, s) for n, s in zip(names, scratch) if s != 0]
    assert not bad, bad
