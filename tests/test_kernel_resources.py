"""Compile-time resources of the gfx950 kernels (CPU only: hipcc -S).

Every kernel must run without scratch memory: a private segment makes each
launch set up scratch, and in this code it has meant the whole argument block
copied to scratch (the optimizer gives up proving it read-only once the
kernel grows).  The greedy streaming kernels must keep two waves per SIMD at
512 threads (at most 256 VGPRs) and four at 256 (at most 128)."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "commit_step_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")


SOURCES = ["token_stats.hip", "token_stats_full.hip", "transfer.hip", "uniform.hip",
           "read_probe.hip"]


def _parse(path):
    found, cur = {}, None
    for line in open(path).read().splitlines():     # the amdhsa metadata, one kernel at a time
        m = re.match(r"\s+\.name:\s+(_Z\S+)$", line)
        if m:
            cur = found.setdefault(m.group(1), {})
            continue
        m = re.match(r"\s+\.(private_segment_fixed_size|vgpr_count|sgpr_count):\s+(\d+)$", line)
        if m and cur is not None:
            cur[m.group(1)] = int(m.group(2))
    return found


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    """Every source compiled to gfx950 assembly, in parallel."""
    from commit_step_amd.build import FLAGS
    flags = [f for f in FLAGS if f not in ("-shared", "-fPIC")]
    tmp = tmp_path_factory.mktemp("asm")
    procs = {}
    for src in SOURCES:
        out = tmp / (src + ".s")
        procs[src] = (out, subprocess.Popen(
            [HIPCC, *flags, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
             "--cuda-device-only", "-S", "-o", str(out), os.path.join(CSRC, src)],
            stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
    result = {}
    for src, (out, pr) in procs.items():
        pr.communicate()
        assert pr.returncode == 0, f"hipcc -S failed for {src}"
        result[src] = _parse(out)
    return result


@pytest.mark.parametrize("src", SOURCES)
def test_no_scratch_and_vgpr_budget(src, kernels):
    ks = kernels[src]
    assert ks, f"no kernels found in {src}"
    for name, r in ks.items():
        assert r["private_segment_fixed_size"] == 0, f"{name} uses scratch: {r}"
        # greedy (SAMPLE = false) 16-byte-load stream kernels: 512-thread groups (one per
        # CU, 2 waves per SIMD) within 256 VGPRs; 256-thread groups (several per CU) keep
        # 4 waves per SIMD, within 128
        m = re.search(r"token_stats_kernelI[tf]Li(\d+)ELi\d+ELb0ELb1ELb[01]E", name)
        if m:
            budget = 256 if m.group(1) == "512" else 128
            assert r["vgpr_count"] <= budget, f"{name}: {r}"
