"""The LDS-DMA waits of the small-M kernels (CPU: reads the gfx950 assembly of our
own skinny.hip, gemv.hip and block.hip).

A wave that pulls X into LDS with buffer_load ... lds then issues its first weight
batches and waits with s_waitcnt vmcnt(n), n being the number of loads issued after
the DMA: loads complete in issue order, so that wait means the DMA has landed while
the weight batches stay in flight.  If the compiler issued fewer loads than n (it
once merged four zero-word loads into one), the wave would read X before it
arrives.  This test compiles the kernels and checks every such wait.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _asm(tmp_path_factory, name):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / (name + ".s")
    csrc = os.path.join(ROOT, "int4_weight_only_02_amd", "csrc")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", csrc, "--cuda-device-only", "-S",
           os.path.join(csrc, name), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text().splitlines()


# source, the fewest DMA waits it must contain: the chunked and the DMA private modes
# in the single and the batched skinny kernels; the act-order instances of the M = 1
# kernel (X of the row by DMA, perm and the codes after it); the block kernel's
# instances of up to two groups per wave (each wave's X slice by DMA, then its scale,
# zero and code loads), single and batched
@pytest.mark.parametrize("name,least", [("skinny.hip", 24), ("gemv.hip", 2), ("block.hip", 12)])
def test_every_dma_wait_covers_the_dma(tmp_path_factory, name, least):
    skinny_asm = _asm(tmp_path_factory, name)
    kern, last_dma, after = None, None, 0
    checked = []
    for line in skinny_asm:
        m = re.match(r"^(_ZN\S+):", line)
        if m:
            kern, last_dma, after = m.group(1), None, 0
            continue
        t = line.strip()
        if t.startswith("buffer_load") and t.endswith(" lds"):
            last_dma, after = t, 0
        elif last_dma is not None and (t.startswith("buffer_load") or t.startswith("global_load")):
            after += 1
        elif last_dma is not None and t.startswith("s_waitcnt") and "vmcnt" in t:
            n = int(re.search(r"vmcnt\((\d+)\)", t).group(1))
            checked.append((kern, n, after))
            last_dma = None
    assert len(checked) >= least, checked
    bad = [c for c in checked if c[1] > c[2]]
    assert not bad, "waits that let the X DMA still be in flight: %s" % bad[:4]
