"""Every HIP kernel of the library compiles for gfx950 without register
spills (no private scratch segment).  The pipelined kernels issue their LDS
operand reads as explicit instructions whose results the compiler treats as
ready at once; a spill of such a destination before the kernel's own wait
would store a value the read has not delivered yet, so a kernel that spills
is wrong, not merely slow.  CPU only: device-code compilation to assembly."""

import os
import re
import subprocess

import pytest

from block_scaled_fp4_topk_amd import build as b

KERNEL_SOURCES = [s for s in b.SOURCES if s.endswith(".hip")]


def kernel_resources(src):
    """{kernel symbol: (private segment bytes, LDS bytes)} from the device assembly."""
    out = os.path.join(b.BUILD, os.path.splitext(src)[0] + ".nospill.s")
    os.makedirs(b.BUILD, exist_ok=True)
    cmd = [b.hipcc(), *b._flags(), "-x", "hip", "-S", "--cuda-device-only", os.path.join(b.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    res, cur = {}, None
    for line in open(out):
        m = re.match(r"\s*\.amdhsa_kernel (\S+)", line)
        if m:
            cur = m.group(1)
            res[cur] = [None, None]
        m = re.match(r"\s*\.amdhsa_private_segment_fixed_size (\d+)", line)
        if m and cur:
            res[cur][0] = int(m.group(1))
        m = re.match(r"\s*\.amdhsa_group_segment_fixed_size (\d+)", line)
        if m and cur:
            res[cur][1] = int(m.group(1))
    os.remove(out)
    return res


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_register_spills(src):
    res = kernel_resources(src)
    assert res, f"no kernels found in {src}"
    spilling = {k: v[0] for k, v in res.items() if v[0]}
    assert not spilling, f"kernels with a private (spill) segment: {spilling}"
    for k, (_, lds) in res.items():
        assert lds is not None and lds <= 160 * 1024, (k, lds)
