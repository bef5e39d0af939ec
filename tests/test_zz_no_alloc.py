"""dllm_commit_step_static (no workspace argument, nothing allocated) against
dllm_commit_step with a workspace, through the C ABI: same kernels, so every
output matches bit for bit, on consecutive calls of different shapes that
share the library's static array (split rows included, so its counters and
partials are used and must be left zero-filled for the next call)."""
import ctypes

import numpy as np
import pytest
import torch

import commit_step_amd as dc
from gpu_util import log, to_dev
from workloads import random_logits

pytestmark = pytest.mark.gpu

DLLM_ERR_UNSUPPORTED = -5
STATIC_BYTES = 1 << 20


def _step(lib, static, logits, B, L, V, mask_id, k, edit_tau, seed_tok):
    """One commit step with a top-k rule and an edit rule on a fresh canvas;
    returns every output as numpy."""
    dev = logits.device
    rng = np.random.default_rng(seed_tok)
    tok_np = np.full((B, L), mask_id, dtype=np.int32)
    done = rng.random((B, L)) < 0.4
    tok_np[done] = rng.integers(0, V - 1, size=int(done.sum()))
    tok = torch.from_numpy(tok_np).to(dev)
    cand = (tok == mask_id).to(torch.uint8)
    editable = (tok != mask_id).to(torch.uint8)
    kk = torch.full((B,), k, dtype=torch.int32, device=dev)
    x0 = torch.full((B, L), -7, dtype=torch.int32, device=dev)
    pr = torch.full((B, L), -7.0, dtype=torch.float32, device=dev)
    en = torch.full((B, L), -7.0, dtype=torch.float32, device=dev)
    cnt = torch.full((B, 2), -7, dtype=torch.int32, device=dev)
    out_k = torch.zeros((B, L), dtype=torch.uint8, device=dev)
    out_e = torch.zeros((B, L), dtype=torch.uint8, device=dev)
    rules = (dc._CRule * 2)()
    rules[0].kind, rules[0].mask, rules[0].out, rules[0].k = dc.RULE_TOPK, cand.data_ptr(), \
        out_k.data_ptr(), kk.data_ptr()
    rules[1].kind, rules[1].mask, rules[1].out, rules[1].param = dc.RULE_EDIT, \
        editable.data_ptr(), out_e.data_ptr(), edit_tau
    cv = dc._CCanvas()
    cv.tokens, cv.counts, cv.skip_rows = tok.data_ptr(), cnt.data_ptr(), 1
    sup = (ctypes.c_int32 * 1)(mask_id)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (logits.data_ptr(), dc.DLLM_BF16, B, L, V, V, 0.0, 0, 0, sup, 1, x0.data_ptr(),
            pr.data_ptr(), en.data_ptr(), None, rules, 2, ctypes.byref(cv))
    if static:
        rc = lib.dllm_commit_step_static(*args, stream)
    else:
        need = int(lib.dllm_token_stats_workspace_size(dc.DLLM_BF16, B, L, V))
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
        rc = lib.dllm_commit_step(*args, ws.data_ptr(), ws.numel(), stream)
    assert rc == 0, lib.dllm_last_error().decode()
    torch.cuda.synchronize()
    if not static:
        assert int(torch.count_nonzero(ws)) == 0
    return {n: t.cpu().numpy() for n, t in (("x0", x0), ("prob", pr), ("entropy", en),
                                            ("counts", cnt), ("topk", out_k), ("edit", out_e),
                                            ("tokens", tok))}


def test_static_entry_matches_the_workspace_entry():
    lib = dc.load_library()
    shapes = [(2, 40, 126464, 5), (1, 24, 50000, 9), (3, 8, 30000, 11), (2, 40, 126464, 13)]
    for i, (B, L, V, seed) in enumerate(shapes):
        need = int(lib.dllm_token_stats_workspace_size(dc.DLLM_BF16, B, L, V))
        assert 0 < need <= STATIC_BYTES
        log(f"static scratch call {i}: B={B} L={L} V={V} (workspace need {need} bytes)")
        mask_id = V - 1
        bits, _ = random_logits(seed, B, L, V, "bf16", 2.5, 0.5, 6.0, 14.0, (mask_id,))
        logits = to_dev(bits, "bf16")
        want = _step(lib, False, logits, B, L, V, mask_id, 3, 0.8, seed)
        got = _step(lib, True, logits, B, L, V, mask_id, 3, 0.8, seed)
        for name, w in want.items():
            assert np.array_equal(got[name].view(np.uint8), w.view(np.uint8)), \
                f"call {i}: {name} differs from dllm_commit_step"
        assert want["topk"].sum() >= B
    log("static scratch entry matches the workspace entry")


def test_static_entry_rejects_shapes_beyond_its_array():
    lib = dc.load_library()
    B, L, V = 300000, 1, 64        # batch-row counters alone need more than 1 MiB
    need = int(lib.dllm_token_stats_workspace_size(dc.DLLM_BF16, B, L, V))
    assert need > STATIC_BYTES
    cv = dc._CCanvas()
    dummy = torch.zeros(16, dtype=torch.uint8, device="cuda")
    p = dummy.data_ptr()
    rc = lib.dllm_commit_step_static(p, dc.DLLM_BF16, B, L, V, V, 0.0, 0, 0, None, 0, p, p, p,
                                     None, None, 0, ctypes.byref(cv),
                                     torch.cuda.current_stream().cuda_stream)
    assert rc == DLLM_ERR_UNSUPPORTED
    assert b"static" in lib.dllm_last_error()
