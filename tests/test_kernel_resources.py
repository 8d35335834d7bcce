"""Compile-only check of the gfx950 kernels (no GPU): every kernel the library
builds uses no scratch memory, i.e. no register spills.  FreeToken PR #897
qualifies its packed reader the same way ("Fresh R9700 stage-1 A/B": zero VGPR
and SGPR spills and zero scratch from the code-object metadata).  The figures
come from the compiler's resource-usage remarks for the same flags as the
library build."""
import os
import re
import subprocess

import pytest

from fp8_kv_cache_row_amd import build as B


def _resources(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".o")
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [B.HIPCC, *flags, *B.source_flags(src), "-c", "-I", B.INCLUDE, "-I", B.CSRC, src, "-o", str(out),
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|LDS Size \[bytes/block\]): (\d+)", line)
        if m and name:
            kernels[name][m.group(1).split()[0]] = int(m.group(2))
    return kernels


@pytest.mark.parametrize("src", B.sources(), ids=os.path.basename)
def test_no_kernel_spills(src, tmp_path):
    kernels = _resources(src, tmp_path)
    if os.path.basename(src) == "fp8kv_api.hip":
        assert not kernels
        return
    assert kernels, "no kernels reported"
    streaming = 0
    for name, res in kernels.items():
        print(f"{name[:90]:90s} VGPR {res.get('VGPRs')} AGPR {res.get('AGPRs')} LDS {res.get('LDS')}")
        assert res.get("ScratchSize") == 0, f"{name} uses {res.get('ScratchSize')} bytes of scratch per lane"
        assert res.get("VGPRs", 0) + res.get("AGPRs", 0) <= 512
        # Stage1<G, D, NT, MULTI, WINDOW, F, STREAM = true>, as mangled
        if re.search(r"Stage1ILi\d+ELi\d+ELi\d+ELb[01]ELb[01]ELi\d+ELb1E", name):
            # the streaming shape: three 4-wave workgroups per CU need <= 168 registers
            assert res.get("VGPRs", 0) + res.get("AGPRs", 0) <= 168, f"{name}: streaming shape over 168 registers"
            streaming += 1
    if os.path.basename(src) == "decode.hip":
        assert streaming == 20, (f"{streaming} streaming stage-1 instantiations "
                                 "(5 GQA ratios x 2 code formats x plain / non-temporal code loads)")
