"""Code generation of the gfx950 kernels, checked on the CPU (hipcc cross-compiles).

Every kernel must use no scratch memory: no VGPR spills and no stack frame
(SGPR spills that land in VGPR lanes are allowed: they touch no memory).  A
helper that the compiler stops inlining (a device-function call with its own
stack) shows up here as scratch; that once slowed the greedy row kernel by 18%
without changing any result.
"""
import os
import re
import shutil
import subprocess

import pytest

from draft_verification_vocab_amd import _build

EXPECTED = ("verify_rows", "verify_rows_level", "verify_accept", "verify_draw", "verify_locate",
            "draft_sample_kernel", "build_kernel", "tree_walk", "accept_metrics_kernel")


def _resource_usage(src):
    flags = [f for f in _build.FLAGS if f not in ("-fPIC", "-shared", "-Wall")]
    cmd = [_build.HIPCC, *flags, "--cuda-device-only", "-c", "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage", src]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels, cur = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark: +(ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill): (\d+)", line)
        if m and cur:
            kernels[cur][m.group(1)] = int(m.group(2))
    return kernels


@pytest.mark.skipif(not os.path.exists(_build.HIPCC) and shutil.which("hipcc") is None,
                    reason="hipcc not available")
def test_kernels_use_no_scratch():
    from concurrent.futures import ThreadPoolExecutor
    seen = {}
    srcs = _build.sources()
    with ThreadPoolExecutor(max_workers=max(1, min(len(srcs), os.cpu_count() or 1, 8))) as ex:
        for usage in ex.map(_resource_usage, srcs):
            seen.update(usage)
    for name in EXPECTED:
        assert any(name in k for k in seen), f"no kernel named like {name}"
    for k, usage in seen.items():
        assert usage.get("ScratchSize [bytes/lane]") == 0, (k, usage)
        assert usage.get("VGPRs Spill") == 0, (k, usage)
