"""Compile-time resources of the gfx950 kernels (CPU only: hipcc -S).

Every kernel must run without scratch memory: a private segment makes each
launch set up scratch, and in this code it has meant the whole argument block
copied to scratch (the optimizer gives up proving it read-only once the
kernel grows).  The greedy streaming kernels must keep two waves per SIMD at
512 threads (at most 256 VGPRs) and four at 256 (at most 128).  Every
kernel's static LDS plus the most dynamic LDS its launcher can ask for must
fit the 160 KiB a gfx950 workgroup may hold: a launch beyond it is not an
error the runtime returns but an aborted queue."""
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
    """Per-kernel fields of the amdhsa metadata: the kernels are a YAML list
    whose items open with '  - ' at two spaces, each item's keys in
    alphabetical order (so fields before `.name` belong to the same item)."""
    text = open(path).read()
    meta = text[text.index("amdhsa.kernels:"):text.index("amdhsa.target")]
    found = {}
    for block in re.split(r"\n  - ", meta)[1:]:
        m = re.search(r"^\s+\.name:\s+(_Z\S+)$", block, re.M)
        if not m:
            continue
        fields = {}
        for key in ("private_segment_fixed_size", "group_segment_fixed_size", "vgpr_count",
                    "sgpr_count"):
            f = re.search(r"^\s+\." + key + r":\s+(\d+)$", block, re.M)
            fields[key] = int(f.group(1)) if f else None
        found[m.group(1)] = fields
    return found


def _const(path, pattern):
    m = re.search(pattern, open(path).read(), re.M)
    assert m, f"{pattern} not found in {path}"
    return int(m.group(1))


MAX_L = _const(os.path.join(ROOT, "include", "dllm_commit.h"), r"^#define DLLM_MAX_L (\d+)")
MAX_SLICES = _const(os.path.join(CSRC, "token_stats_dev.h"), r"kMaxSlices = (\d+);")
PARTIAL_BYTES = 32      # sizeof(Partial), asserted in token_stats_dev.h
LDS_LIMIT = 160 * 1024  # LDS per workgroup on gfx950


def _rule_lds(L, nt):
    """Dynamic LDS of the ranking rules for a batch row of L positions run by
    nt threads (rule_smem_bytes in rules_dev.h: position lists of 20 bytes
    per slot of the power-of-two padded row plus 12 bytes per thread, or the
    8-byte sort keys, whichever is larger, plus 512 bytes of flags)."""
    npow = 64
    while npow < L:
        npow *= 2
    return ((max(npow * 20 + nt * 12, npow * 8) + 7) & ~7) + 512


def _max_dynamic_lds(name):
    """The largest dynamic LDS request the library makes for this kernel."""
    m = re.search(r"token_stats_kernelI[tf]Li(\d+)E", name)
    if m:   # ranking rules fused into the last group of a batch row, or slice partials
        return max(_rule_lds(MAX_L, int(m.group(1))), MAX_SLICES * PARTIAL_BYTES)
    m = re.search(r"batch_rule_kernelILi(\d+)E", name)
    if m:
        return _rule_lds(MAX_L, int(m.group(1)))
    return 0


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


@pytest.mark.parametrize("src", SOURCES)
def test_lds_fits_workgroup(src, kernels):
    ks = kernels[src]
    assert ks, f"no kernels found in {src}"
    for name, r in ks.items():
        assert r["group_segment_fixed_size"] is not None, f"{name}: no LDS size in metadata"
        need = r["group_segment_fixed_size"] + _max_dynamic_lds(name)
        assert need <= LDS_LIMIT, f"{name}: {need} bytes of LDS ({r})"


def test_parse_attributes_fields_to_their_own_kernel(tmp_path):
    """Keys sorted before `.name` in a metadata item belong to that item."""
    meta = """\t.amdgpu_metadata
---
amdhsa.kernels:
  - .args: []
    .group_segment_fixed_size: 100
    .name:           _Z1av
    .private_segment_fixed_size: 0
    .sgpr_count:     10
    .vgpr_count:     20
  - .args: []
    .group_segment_fixed_size: 200
    .name:           _Z1bv
    .private_segment_fixed_size: 16
    .sgpr_count:     30
    .vgpr_count:     40
amdhsa.target:   amdgcn-amd-amdhsa--gfx950
"""
    p = tmp_path / "k.s"
    p.write_text(meta)
    got = _parse(str(p))
    assert got["_Z1av"] == {"private_segment_fixed_size": 0, "group_segment_fixed_size": 100,
                            "vgpr_count": 20, "sgpr_count": 10}
    assert got["_Z1bv"] == {"private_segment_fixed_size": 16, "group_segment_fixed_size": 200,
                            "vgpr_count": 40, "sgpr_count": 30}
