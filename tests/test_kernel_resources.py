"""Every gfx950 kernel of the library fits its registers: the device assembly that hipcc
writes for each HIP source reports no VGPR or SGPR spills and no private (scratch) segment.

A spill turns register traffic into scratch memory traffic inside the hot loops (it
happened once to the GEMM's bias epilogue); this runs on the CPU, where hipcc
cross-compiles, with the library's own compile flags."""
import concurrent.futures as cf
import os
import re
import subprocess
import tempfile

import pytest

from rotated_bit_linear_amd import build as B

SOURCES = [s for s in B.SOURCES if s.endswith(".hip")]


def _asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, src + ".s")
    flags = [f for f in B.FLAGS if f not in ("-fPIC",)]
    cmd = [B.HIPCC, *flags, "-x", "hip", "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr[-2000:]}")
    return open(out).read()


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not available")
def test_no_spills_and_no_scratch():
    with tempfile.TemporaryDirectory() as d, cf.ThreadPoolExecutor(4) as ex:
        texts = dict(zip(SOURCES, ex.map(lambda s: _asm(s, d), SOURCES)))
    seen = 0
    bad = []
    for src, text in texts.items():
        for block in text.split("- .agpr_count:")[1:]:
            name = re.search(r"\.name:\s+(\S+)", block).group(1)
            fields = {k: int(re.search(rf"\.{k}:\s+(\d+)", block).group(1))
                      for k in ("vgpr_spill_count", "sgpr_spill_count", "private_segment_fixed_size", "vgpr_count")}
            seen += 1
            if fields["vgpr_spill_count"] or fields["sgpr_spill_count"] or fields["private_segment_fixed_size"]:
                bad.append((src, name, fields))
    assert seen >= 40, seen            # every instantiation of every kernel was inspected
    assert not bad, bad
