"""Every kernel instance the library builds runs without scratch memory: no register
spills to per-lane private memory (reflex-llm kernel notes, batched GEMM section and
its resource table: the batched kernels are kept at zero spill stores and loads).
Each HIP source is compiled for gfx950 with the library's own flags and the
compiler's resource-usage remarks; every kernel must report ScratchSize 0."""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from gemm_q4_q5_amd import build

KERNEL_SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]


def _usage(src, tmp):
    cmd = [build.HIPCC, *build.FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c",
           os.path.join(build.CSRC, src), "-o", os.path.join(tmp, src + ".o")]
    out = subprocess.run(cmd, capture_output=True, text=True, check=True).stderr
    names = re.findall(r"remark: Function Name: (\S+)", out)
    scratch = [int(v) for v in re.findall(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", out)]
    assert len(names) == len(scratch), f"{src}: could not pair the remarks"
    return list(zip(names, scratch))


@pytest.mark.skipif(not os.path.exists(build.HIPCC) and shutil.which("hipcc") is None, reason="no hipcc")
def test_no_kernel_uses_scratch(tmp_path):
    with cf.ThreadPoolExecutor(max_workers=len(KERNEL_SOURCES)) as ex:
        found = dict(zip(KERNEL_SOURCES, ex.map(lambda s: _usage(s, str(tmp_path)), KERNEL_SOURCES)))
    kernels = [(src, name, sc) for src, lst in found.items() for name, sc in lst]
    assert sum(1 for _, n, _ in kernels if "mma_kernel" in n) >= 100
    assert sum(1 for _, n, _ in kernels if "prefill_kernel" in n) == 6   # one per weight type, and the split Q6_K one
    spilling = [(src, name, sc) for src, name, sc in kernels if sc != 0]
    assert not spilling, f"{len(spilling)} kernels use scratch: {spilling[:5]}"
