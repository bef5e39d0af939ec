"""The stage-timestamp build (libdllm_commit_stages.so) on the GPU: its
launches compute the same bits as the product library, and the completing
workgroup's stages come in the order it passes them."""
import os

import pytest
import torch

import commit_step_amd as dc

pytestmark = pytest.mark.gpu

st = pytest.importorskip("commit_step_amd.stage_timing")
STAGES_SO = os.path.join(os.path.dirname(os.path.abspath(dc.__file__)), "libdllm_commit_stages.so")


@pytest.mark.skipif(not os.path.exists(STAGES_SO),
                    reason="stage build absent (python -m commit_step_amd.build --stages)")
@pytest.mark.parametrize("workload", ["tiny", "llada_step"])
def test_stage_build_matches_and_orders_stages(workload):
    torch.cuda.set_device(0)
    prod = dc.load_library()
    stages = dc.load_library(stages=True)
    launch_p, _, keep_p = st.setup(workload, prod, 0)
    launch_s, _, keep_s = st.setup(workload, stages, 0)
    assert launch_p(0) == 0
    ts = st.one_launch(stages, launch_s, 0, burst=3)
    torch.cuda.synchronize()
    for name in keep_p["outs"]:
        assert torch.equal(keep_p["outs"][name], keep_s["outs"][name]), name
    m = st.metrics(ts)
    assert m["workgroups"] >= 64
    chain = [m["completer_" + n] for n in st.CHAIN if "completer_" + n in m]
    assert len(chain) >= 4 and chain == sorted(chain), m
    assert m["stream_end_last"] > 0 and m["completer_batch_done"] >= m["stream_end_last"]
    # the product library has no records to give
    assert prod.dllm_stage_timestamps(None, 0, 1) != 0
