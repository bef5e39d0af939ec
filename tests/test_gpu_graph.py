"""The commit step captured in a HIP graph and replayed.

The library records no memset (the workspace is cleared by its own kernels),
so a captured sequence must replay exactly: every replay, with eager work on
the same workspace between replays, gives the eager results bit for bit.
"""
import numpy as np
import pytest
import torch

import commit_step_amd as dc
from gpu_util import log, to_dev
from workloads import random_logits

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager_results():
    dev = torch.device("cuda:0")
    B, L, V, mask_id, steps = 1, 32, 126464, 126463, 4           # split rows, top-k, canvas
    logits = [to_dev(random_logits(70 + s, B, L, V, "bf16", 3.0, 0.4, 8.0, 16.0, (mask_id,))[0], "bf16")
              for s in range(steps)]
    B2, L2, V2 = 1, 64, 30000                                     # entropy_bound + edit, split rows
    bits2, rng = random_logits(80, B2, L2, V2, "bf16", 2.0, 0.5, 6.0, 14.0)
    lg2 = to_dev(bits2, "bf16")
    cand2 = torch.from_numpy(rng.random((B2, L2)) < 0.6).to(dev)
    tok2 = torch.from_numpy(rng.integers(0, V2, size=(B2, L2)).astype(np.int32)).to(dev)
    other = to_dev(random_logits(90, 2, 40, 30000, "bf16", 2.0, 0.5, 5.0, 12.0)[0], "bf16")
    other_cand = torch.ones((2, 40), dtype=torch.bool, device=dev)

    lib = dc.load_library()
    need = max(int(lib.dllm_token_stats_workspace_size(dc.DLLM_BF16, *s))
               for s in [(B, L, V), (B2, L2, V2), (2, 40, 30000)])
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    init = torch.full((B, L), mask_id, dtype=torch.int32, device=dev)
    tok = init.clone()
    k = torch.full((B,), 3, dtype=torch.int32, device=dev)
    x0 = torch.empty((B, L), dtype=torch.int32, device=dev)
    pr = torch.empty((B, L), dtype=torch.float32, device=dev)
    en = torch.empty((B, L), dtype=torch.float32, device=dev)
    cnt = torch.empty((B, 2), dtype=torch.int32, device=dev)
    hist = {"tok": torch.empty((steps, B, L), dtype=torch.int32, device=dev),
            "cnt": torch.empty((steps, B, 2), dtype=torch.int32, device=dev),
            "commit": torch.empty((steps, B, L), dtype=torch.bool, device=dev),
            "x0": torch.empty((steps, B, L), dtype=torch.int32, device=dev),
            "prob": torch.empty((steps, B, L), dtype=torch.float32, device=dev)}
    out2 = (torch.empty((B2, L2), dtype=torch.int32, device=dev),
            torch.empty((B2, L2), dtype=torch.float32, device=dev),
            torch.empty((B2, L2), dtype=torch.float32, device=dev))
    masks2 = {}

    def sequence():
        tok.copy_(init)
        for s in range(steps):
            rule = dc.Rule.topk(tok == mask_id, k)
            dc.commit_step(logits[s], tok, [rule], suppress_ids=(mask_id,), out=(x0, pr, en),
                           counts=cnt, workspace=ws)
            hist["tok"][s].copy_(tok)
            hist["cnt"][s].copy_(cnt)
            hist["commit"][s].copy_(rule.out)
            hist["x0"][s].copy_(x0)
            hist["prob"][s].copy_(pr)
        eb, ed = dc.Rule.entropy_bound(cand2, 0.5), dc.Rule.edit(~cand2, tok2, 0.9)
        dc.token_stats(lg2, rules=[eb, ed], out=out2, workspace=ws)
        masks2["eb"], masks2["ed"] = eb.out, ed.out

    sequence()
    torch.cuda.synchronize()
    want = {name: t.clone() for name, t in hist.items()}
    want.update({f"stats{i}": t.clone() for i, t in enumerate(out2)})
    want.update({name: t.clone() for name, t in masks2.items()})
    assert int(torch.count_nonzero(ws)) == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sequence()                                   # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sequence()
    torch.cuda.synchronize()

    for rep in range(4):
        # eager work between replays: clear the outputs, and a call of another shape on
        # the same workspace (which must leave it zero-filled for the replay)
        for t in list(hist.values()) + list(out2):
            t.fill_(7)
        r = dc.Rule.entropy_bound(other_cand, 0.4)
        dc.token_stats(other, rules=[r], workspace=ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {name: t for name, t in hist.items()}
        got.update({f"stats{i}": t for i, t in enumerate(out2)})
        got.update(masks2)
        for name, t in want.items():
            assert torch.equal(got[name], t), f"replay {rep}: {name} differs from the eager run"
        assert int(torch.count_nonzero(ws)) == 0, f"replay {rep}: workspace left dirty"
    log("graph replays match the eager run")


def test_graph_with_the_default_workspace_of_the_capture_stream():
    """No workspace= argument: the call takes its stream's default workspace,
    created by an eager call on the capture stream before the capture."""
    dev = torch.device("cuda:0")
    B, L, V = 2, 48, 30000                                       # split rows
    lg = to_dev(random_logits(95, B, L, V, "bf16", 2.0, 0.5, 6.0, 14.0)[0], "bf16")
    cand = torch.ones((B, L), dtype=torch.bool, device=dev)
    out = (torch.empty((B, L), dtype=torch.int32, device=dev),
           torch.empty((B, L), dtype=torch.float32, device=dev),
           torch.empty((B, L), dtype=torch.float32, device=dev))
    masks = {}

    def call():
        r = dc.Rule.entropy_bound(cand, 0.5)
        dc.token_stats(lg, rules=[r], out=out)
        masks["eb"] = r.out

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        call()                                       # creates the capture stream's workspace
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    want = [t.clone() for t in out] + [masks["eb"].clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        call()
    graph_mask = masks["eb"]                         # the captured call's output
    torch.cuda.synchronize()
    for rep in range(3):
        for t in out:
            t.fill_(7)
        call()                                       # eager call on the default stream
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = list(out) + [graph_mask]
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager run"
    log("default-workspace graph replays match the eager run")
