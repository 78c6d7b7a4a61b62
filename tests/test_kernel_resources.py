"""Every gfx950 kernel of the library runs without scratch memory.

Scratch (per-lane private memory) appears when the compiler spills registers
or keeps an array indexed at run time in memory; a kernel that needs it
reserves it for every wave it launches, and the loads and stores it adds sit
on the hot loops.  The compiler's resource report of a device-only compile of
each source is read here (no GPU needed)."""
import concurrent.futures as cf
import os
import re
import subprocess

import pytest

from expert_ffn_layer_router_amd import build

pytestmark = pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc") and not os.environ.get("HIPCC"),
                                reason="hipcc not installed")


def _report(src):
    cmd = [build._hipcc(), *build.HIPCC_FLAGS, "--cuda-device-only", "-c", "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage", os.path.join(build.CSRC, src)]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert res.returncode == 0, res.stdout[-2000:]
    kernels, name = {}, None
    for line in res.stdout.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            kernels[name] = int(m.group(1))
    return kernels


def test_no_kernel_uses_scratch():
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        reports = dict(zip(build.SOURCES, ex.map(_report, build.SOURCES)))
    assert sum(len(r) for r in reports.values()) >= 20, "the resource report lists the kernels"
    spilled = {f"{src}: {k}": v for src, r in reports.items() for k, v in r.items() if v}
    assert not spilled, f"kernels with scratch: {spilled}"
