"""Every kernel of the library compiles for gfx950 without register spills
(CPU only: the compiler's resource report, no GPU).

A spill moves registers to per-lane scratch memory in the middle of the hot
loops; the report's ScratchSize must be 0 bytes per lane for every kernel
of every source, for every instantiated operand/pool type and scan tile
width."""

import concurrent.futures as cf
import os
import re
import subprocess

import pytest

from linear_attention_state_kda_amd import build as B


def report(src):
    cmd = [B.hipcc(), "-x", "hip", "-c", "--cuda-device-only", os.path.join(B.CSRC, src), "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"] + [f for f in B.FLAGS if f != "-fPIC"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    names = re.findall(r"Function Name: (\S+)", r.stderr)
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", r.stderr)]
    vgprs = [int(x) for x in re.findall(r"VGPRs: (\d+)", r.stderr)]
    return list(zip(names, scratch, vgprs))


def test_no_kernel_spills():
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    srcs = [s for s in B.SOURCES if s.endswith(".hip")]
    with cf.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        reports = dict(zip(srcs, ex.map(report, srcs)))
    kernels = [(src, n, sc, vg) for src, rep in reports.items() for n, sc, vg in rep]
    assert any("kda_chunk_scan16" in n for _, n, _, _ in kernels)
    assert len([k for k in kernels if "kda_chunk_scan16" in k[1]]) == 18   # 2 inputs x 3 pools x 3 tile widths
    spilled = [(src, n, sc) for src, n, sc, _ in kernels if sc != 0]
    assert not spilled, spilled
    assert all(vg <= 512 for *_, vg in kernels)
