"""Build libdllm_commit.so for gfx950 with hipcc (in-tree, next to this file).

Usage: python -m commit_step_amd.build [--stages]   (or call build()).
--stages builds libdllm_commit_stages.so instead: the same library with stage
timestamps recorded by the statistics kernels (dllm_stage_timestamps), for
commit_step_amd.stage_timing.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = ["csrc/token_stats.hip", "csrc/token_stats_full.hip", "csrc/transfer.hip",
           "csrc/uniform.hip", "csrc/read_probe.hip"]
LIB = os.path.join(HERE, "libdllm_commit.so")
STAGES_LIB = os.path.join(HERE, "libdllm_commit_stages.so")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no implicit fused multiply-add: every rounding step is the one written
    "-ffp-contract=off",
    # packed FP32 instructions stay off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def _filter(out):
    return [ln for ln in out.strip().splitlines() if "argument unused during compilation" not in ln
            and "packed-fp32-ops" not in ln]


def build(verbose=True, stages=False):
    """Compile the HIP sources into commit_step_amd/libdllm_commit.so (with
    stages: libdllm_commit_stages.so, stage timestamps on): one object per
    source, compiled in parallel, then one link."""
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    cflags = [f for f in FLAGS if f != "-shared"] + (["-DDLLM_STAGE_TIMESTAMPS"] if stages else [])
    lib = STAGES_LIB if stages else LIB
    tag = ".stages" if stages else ""
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(HERE, os.path.basename(src) + tag + ".o")
        cmd = [hipcc(), *cflags, *inc, "-c", "-o", obj, os.path.join(HERE, src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        objs.append(obj)
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                      text=True))
    failed = []
    for src, pr in zip(SOURCES, procs):
        out, _ = pr.communicate()
        lines = _filter(out)
        if pr.returncode != 0:
            failed.append(f"{src}:\n" + "\n".join(lines))
        elif verbose and lines:
            print("\n".join(lines), flush=True)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
    tmp = lib + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + "\n".join(_filter(r.stdout + r.stderr)))
    for obj in objs:
        os.remove(obj)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    build(stages="--stages" in sys.argv[1:])
    sys.exit(0)
