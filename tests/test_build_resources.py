"""Every gfx950 kernel compiles without register spills or scratch memory.

Scratch accesses are vector-memory operations: in the MFMA kernels they would
count in the same counter as the global->LDS loads whose waits are computed
at compile time, so a spill would also add waits for in-flight loads. The
compiler's resource-usage remarks are read for every kernel of every HIP
source (compilation only; no GPU needed)."""
from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mlstm_matrix_memory_chunkwise_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def _usage(src):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-c", src,
           "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels = {}
    name = None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark: ([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
        if m and name:
            kernels[name][m.group(1).strip()] = int(m.group(2))
    return kernels


def test_no_spills_or_scratch():
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = dict(zip(srcs, ex.map(_usage, srcs)))
    bad = []
    n = 0
    for src, kernels in results.items():
        for name, u in kernels.items():
            n += 1
            if u.get("VGPRs Spill", 0) or u.get("ScratchSize", 0):
                bad.append((os.path.basename(src), name, u.get("VGPRs Spill"), u.get("ScratchSize")))
    assert n > 0, "no kernels found in the compiler's resource remarks"
    assert not bad, bad
