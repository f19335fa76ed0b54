"""Register budget of the persistent grouped GEMM (no GPU needed: the device
code is compiled for gfx950 here and its metadata read).

The kernel issues its MFMAs as inline asm, which the compiler does not know
to be MFMAs: any spill code it places around them (a store or move of an
accumulator register right after the MFMA that writes it) reads the result
before it lands, and the output goes wrong.  So no instantiation of the
kernel may spill registers.
"""
import os
import re
import shutil
import subprocess

import pytest

from sparse_mixture_experts_10_amd import build as B


def _hipcc():
    try:
        return B._hipcc()
    except RuntimeError:
        return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_persistent_gemm_spills_no_registers(tmp_path):
    src = os.path.join(B.CSRC, "gemm_bf16_persist.hip")
    out = tmp_path / "persist.s"
    flags = [f for f in B.FLAGS if f not in ("-fPIC",)]
    cmd = [_hipcc()] + flags + ["--cuda-device-only", "-S", "-x", "hip", src, "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    text = out.read_text()
    names = re.findall(r"^\s+\.name:\s+(\S*gemm_bf16_persist_kernel\S*)", text, flags=re.M)
    spills = re.findall(r"^\s+\.vgpr_spill_count:\s+(\d+)", text, flags=re.M)
    privs = re.findall(r"^\s+\.private_segment_fixed_size:\s+(\d+)", text, flags=re.M)
    assert len(names) >= 8, names
    assert len(spills) == len(names) == len(privs), (len(spills), len(names), len(privs))
    bad = [(n, int(s), int(p)) for n, s, p in zip(names, spills, privs) if int(s) or int(p)]
    assert not bad, f"instantiations that spill: {bad}"
