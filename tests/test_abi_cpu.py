"""The C-ABI library loads and exports what include/dllm_commit.h declares;
host-only logic (block_ranges, argument validation) is checked on the CPU.
No kernel is launched here."""
import ctypes
import glob
import math
import os
import re
from itertools import product

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    import commit_step_amd
    path = commit_step_amd.library_path()
    if not os.path.exists(path):
        from commit_step_amd.build import build
        build(verbose=False)
    return commit_step_amd.load_library()


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(dllm_\w+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ["dllm_token_stats", "dllm_transfer_threshold", "dllm_transfer_topk",
              "dllm_transfer_factor", "dllm_transfer_entropy_bound", "dllm_transfer_edit",
              "dllm_transfer_schedule", "dllm_block_ranges", "dllm_block_causal_mask"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in _declared_functions():
        assert hasattr(lib, n), f"{n} is declared but not exported"


def test_block_ranges_host_parity(lib):
    import commit_step_amd as dc
    for P, G, bl, align in product([0, 1, 31, 32, 77, 100, 1000], [0, 1, 31, 32, 33, 435, 4096],
                                   [1, 7, 32, 1000], [False, True]):
        assert dc.block_ranges(P, G, bl, align) == oracle.block_ranges(P, G, bl, align)
    # partial buffer: the count is still returned, only cap pairs are written
    buf = (ctypes.c_int64 * 4)()
    assert lib.dllm_block_ranges(77, 435, 32, 1, buf, 2) == 14
    assert list(buf) == [64, 96, 96, 128]


def _err(lib):
    return lib.dllm_last_error().decode()


def test_token_stats_argument_errors(lib):
    P = ctypes.c_void_p
    fake = P(16)   # never dereferenced: every call below fails validation first

    def call(dtype=1, B=1, L=1, V=8, stride=8, T=0.0, step=0, sup=None, nsup=0, rules=None,
             nrules=0):
        return lib.dllm_token_stats(fake, dtype, B, L, V, stride, T, 0, step, sup, nsup, fake,
                                    fake, fake, None, rules, nrules, fake, 1 << 20, None)

    assert call(dtype=7) == -2 and "dtype" in _err(lib)
    assert call(B=-1) == -1
    assert call(V=0) == -1
    assert call(stride=4) == -1 and "row_stride" in _err(lib)
    assert call(T=-1.0) == -1 and "temperature" in _err(lib)
    assert call(T=math.nan) == -1
    assert call(T=math.inf) == -1
    assert call(step=1 << 32) == -1 and "step" in _err(lib)
    assert call(nsup=65) == -1
    assert call(nsup=1) == -1 and "suppress_ids" in _err(lib)
    ids = (ctypes.c_int32 * 3)(1, 9, 2)
    assert call(sup=ids, nsup=2) == -1 and "outside" in _err(lib)
    ids = (ctypes.c_int32 * 3)(3, 3, 2)
    assert call(sup=ids, nsup=2) == -1 and "twice" in _err(lib)
    ids = (ctypes.c_int32 * 8)(*range(8))
    assert call(sup=ids, nsup=8) == -1 and "every id" in _err(lib)
    assert call(nrules=3) == -1
    import commit_step_amd as dc
    rules = (dc._CRule * 2)()
    rules[0].kind = 9
    assert call(rules=rules, nrules=1) == -1 and "kind" in _err(lib)
    rules[0].kind = dc.RULE_THRESHOLD
    rules[0].mask = 16
    rules[0].out = 32
    rules[0].param = math.nan
    assert call(rules=rules, nrules=1) == -1 and "NaN" in _err(lib)
    rules[0].param = 0.5
    assert call(L=5000, V=8, rules=rules, nrules=1) == -5
    rules[0].score = 7
    assert call(rules=rules, nrules=1) == -1 and "score" in _err(lib)
    rules[0].score = dc.SCORE_MARGIN                  # ranks by margin, no margin output
    assert call(rules=rules, nrules=1) == -1 and "margin" in _err(lib)
    rules[0].kind = dc.RULE_ENTROPY_BOUND             # entropy_bound ranks by entropy only
    assert call(rules=rules, nrules=1) == -1 and "score" in _err(lib)
    rules[0].kind, rules[0].score = dc.RULE_THRESHOLD, 0
    # empty shapes: OK with nothing launched
    assert call(B=0) == 0 and call(L=0) == 0
    # more positions than one launch can hold
    assert call(B=4096, L=1025) == -5 and "launch limit" in _err(lib)


def test_commit_step_argument_errors(lib):
    import commit_step_amd as dc
    P = ctypes.c_void_p
    fake = P(16)   # never dereferenced: every call below fails validation first

    def call(canvas, rules=None, nrules=0, B=1, L=4, V=8):
        return lib.dllm_commit_step(fake, 1, B, L, V, V, 0.0, 0, 0, None, 0, fake, P(24), P(40),
                                    None, rules, nrules, canvas, fake, 1 << 20, None)

    assert call(None) == -1 and "canvas" in _err(lib)
    cv = dc._CCanvas()
    cv.tokens, cv.counts, cv.skip_rows = 64, 64, 1
    assert call(ctypes.byref(cv)) == -1 and "alias" in _err(lib)
    cv.counts = 24                                    # the prob array
    assert call(ctypes.byref(cv)) == -1 and "alias" in _err(lib)
    cv.counts = 80
    rules = (dc._CRule * 2)()
    for i, kind in enumerate((dc.RULE_THRESHOLD, dc.RULE_TOPK)):
        rules[i].kind, rules[i].mask, rules[i].out, rules[i].param = kind, 96 + i, 128 + i, 0.5
        rules[i].k = 160
    assert call(ctypes.byref(cv), rules, 2) == -1 and "ranking rule" in _err(lib)
    rules[1].kind, rules[1].tokens = dc.RULE_EDIT, 200   # an edit rule with other tokens
    assert call(ctypes.byref(cv), rules, 2) == -1 and "canvas" in _err(lib)
    cv.tokens = None
    rules[1].tokens = None                            # no tokens anywhere
    assert call(ctypes.byref(cv), rules, 2) == -1 and "tokens" in _err(lib)
    assert call(ctypes.byref(cv), B=0) == 0


def test_commit_step_static_host_checks(lib):
    """The allocation-free entry point checks its canvas and the static
    array's size on the host, before any device call."""
    import commit_step_amd as dc
    P = ctypes.c_void_p
    fake = P(16)
    cv = dc._CCanvas()

    def call(canvas, B, L, V):
        return lib.dllm_commit_step_static(fake, 1, B, L, V, V, 0.0, 0, 0, None, 0, fake, P(24),
                                           P(40), None, None, 0, canvas, None)

    assert call(None, 1, 4, 8) == -1 and "canvas" in _err(lib)
    B, L, V = 300000, 1, 64
    assert lib.dllm_token_stats_workspace_size(1, B, L, V) > (1 << 20)
    assert call(ctypes.byref(cv), B, L, V) == -5 and "static" in _err(lib)


def test_stage_timestamps_only_in_the_stage_build(lib):
    buf = (ctypes.c_uint64 * 8)()
    assert lib.dllm_stage_timestamps(buf, 8, 0) == -5 and "stage" in _err(lib)


def test_stage_timeline_metrics_from_records():
    """The stage timeline's arithmetic on hand-made records (ticks of 10 ns)."""
    import numpy as np
    from commit_step_amd import stage_timing as st
    ts = np.zeros((3, 16), dtype=np.int64)
    ts[0, [0, 1, 4, 5]] = [1000, 3000, 3100, 3200]                # a row that is not last
    ts[1, [0, 1, 4, 5, 6]] = [1010, 3500, 3600, 3700, 3900]       # the completing row
    ts[2, [0, 1, 4, 5]] = [1005, 2000, 2100, 2200]
    m = st.metrics(ts)
    want = {"workgroups": 3, "last_start": 0.1, "stream_max_wg": 24.9, "stream_median_wg": 20.0,
            "stream_end_last": 25.0, "stream_end_median": 20.0, "published_last": 26.0,
            "batch_done_last": 29.0, "completer_stream_end": 25.0, "completer_batch_counted": 27.0}
    for k, v in want.items():
        assert abs(m[k] - v) < 1e-9, (k, m[k], v)
    assert "slice_counted_last" not in m


def test_uniform_helpers_argument_errors(lib):
    import commit_step_amd as dc
    P = ctypes.c_void_p
    out = ctypes.c_double()
    assert lib.dllm_linear_temperature(3, 4, 0.4, 0.8, ctypes.byref(out)) == 0
    assert out.value == pytest.approx(0.4 + 0.4 * 3 / 4, rel=1e-15)
    assert dc.linear_temperature(48, 48) == 0.8
    assert lib.dllm_linear_temperature(5, 4, 0.4, 0.8, ctypes.byref(out)) == -1
    assert lib.dllm_linear_temperature(0, 0, 0.4, 0.8, ctypes.byref(out)) == -1
    assert lib.dllm_linear_temperature(1, 4, math.nan, 0.8, ctypes.byref(out)) == -1
    assert lib.dllm_linear_temperature(1, 4, 0.4, 0.8, None) == -1
    fake = P(16)
    assert lib.dllm_uniform_canvas(fake, 1, 4, 0, 1, 0, None) == -1 and "V" in _err(lib)
    assert lib.dllm_uniform_canvas(fake, 1, 4, 1 << 31, 1, 0, None) == -1
    assert lib.dllm_uniform_canvas(fake, 1, 4, 10, 1, 1 << 32, None) == -1 and "draw" in _err(lib)
    assert lib.dllm_uniform_canvas(None, 1, 4, 10, 1, 0, None) == -1
    assert lib.dllm_uniform_canvas(None, 0, 4, 10, 1, 0, None) == 0
    assert lib.dllm_renoise(fake, P(32), None, 2, 3, P(48), None) == -1
    assert lib.dllm_renoise(fake, P(32), P(40), 2, 3, P(32), None) == -1 and "alias" in _err(lib)
    stop = lib.dllm_stable_confident_stop
    assert stop(fake, P(24), 2, 3, -1, 0.1, 1, P(32), P(40), P(48), None) == -1
    assert stop(fake, P(24), 2, 3, 1, math.nan, 1, P(32), P(40), P(48), None) == -1
    assert stop(fake, P(24), 2, 3, 1, 0.1, 1, fake, P(40), P(48), None) == -1 and "alias" in _err(lib)
    assert stop(fake, P(24), 0, 3, 1, 0.1, 1, P(32), P(40), P(48), None) == 0


def test_read_probe_argument_errors(lib):
    P = ctypes.c_void_p
    probe = lib.dllm_read_probe
    assert probe(None, 64, 1, 256, P(64), None) == -1
    assert probe(P(16), 64, 1, 256, None, None) == -1
    assert probe(P(8), 64, 1, 256, P(64), None) == -1 and "aligned" in _err(lib)
    assert probe(P(16), 60, 1, 256, P(64), None) == -1
    assert probe(P(16), 0, 1, 256, P(64), None) == -1
    assert probe(P(16), 64, 0, 256, P(64), None) == -1 and "workgroups" in _err(lib)
    assert probe(P(16), 64, 1 << 31, 256, P(64), None) == -1
    assert probe(P(16), 64, 1, 128, P(64), None) == -1 and "threads" in _err(lib)


def test_decaying_threshold_host_parity(lib):
    import commit_step_amd as dc
    for t0, fl, d in product([0.95, 0.9, 1.0, 0.5], [0.95, 0.7, 0.0, -1.0], [0.0, 0.01, 0.05, 1e-9]):
        for s in [0, 1, 5, 31, 32, 1000, 1 << 40]:
            assert dc.decaying_threshold(t0, fl, d, s) == oracle.decaying_threshold(t0, fl, d, s)
    out = ctypes.c_double()
    assert lib.dllm_decaying_threshold(0.9, 0.5, 0.1, -1, ctypes.byref(out)) == -1
    assert lib.dllm_decaying_threshold(math.nan, 0.5, 0.1, 1, ctypes.byref(out)) == -1
    assert lib.dllm_decaying_threshold(0.9, 0.5, math.nan, 1, ctypes.byref(out)) == -1
    assert lib.dllm_decaying_threshold(0.9, 0.5, 0.1, 1, None) == -1


def test_per_row_threshold_argument_errors(lib):
    import commit_step_amd as dc
    P = ctypes.c_void_p
    fake = P(16)
    rows = lib.dllm_transfer_threshold_rows
    assert rows(fake, P(24), None, 2, 4, 0, P(32), None) == -1 and "taus" in _err(lib)
    assert rows(fake, P(24), P(32), 2, 4, 0, P(32), None) == -1 and "alias" in _err(lib)
    assert rows(fake, P(24), None, 0, 4, 0, P(32), None) == 0
    rules = (dc._CRule * 1)()
    rules[0].kind, rules[0].mask, rules[0].out, rules[0].k = dc.RULE_TOPK, 96, 128, 160
    rules[0].taus = 200                               # only threshold takes taus
    assert lib.dllm_token_stats(fake, 1, 1, 4, 8, 8, 0.0, 0, 0, None, 0, fake, P(24), P(40),
                                None, rules, 1, fake, 1 << 20, None) == -1
    assert "per-row" in _err(lib)
    with pytest.raises(ValueError):
        import torch
        dc.Rule(dc.RULE_FACTOR, None, torch.zeros(2, dtype=torch.float64))


def test_transfer_argument_errors(lib):
    fake = ctypes.c_void_p(16)
    assert lib.dllm_transfer_threshold(fake, fake, 1, 4, math.nan, 0, ctypes.c_void_p(32), None) == -1
    assert lib.dllm_transfer_threshold(None, fake, 1, 4, 0.5, 0, ctypes.c_void_p(32), None) == -1
    assert lib.dllm_transfer_threshold(fake, fake, 1, 4, 0.5, 0, fake, None) == -1   # out aliases conf
    assert lib.dllm_transfer_factor(fake, fake, -1, 4, 1.0, ctypes.c_void_p(32), None) == -1
    assert lib.dllm_transfer_entropy_bound(fake, fake, 1, 4097, 1.0, ctypes.c_void_p(32), None) == -5
    assert lib.dllm_transfer_topk(fake, fake, None, 1, 4, ctypes.c_void_p(32), None) == -1
    assert lib.dllm_transfer_edit(fake, fake, fake, fake, 1, 4, math.nan, ctypes.c_void_p(32), None) == -1
    assert lib.dllm_transfer_schedule(fake, 1, 0, fake, None) == -1
    assert lib.dllm_block_causal_mask(8, 0, fake, None) == -1
    assert lib.dllm_block_causal_mask(1 << 25, 32, fake, None) == -5      # beyond the launch limit
    assert lib.dllm_transfer_factor(fake, fake, 1 << 23, 4096, 1.0, ctypes.c_void_p(32), None) == -5
    assert lib.dllm_transfer_threshold(fake, fake, 1 << 27, 4, 0.5, 0, ctypes.c_void_p(32), None) == -5
    assert lib.dllm_block_ranges(0, 8, 0, 0, None, 0) == -1
    assert lib.dllm_block_ranges(-1, 8, 4, 0, None, 0) == -1
    for fn, args in [(lib.dllm_transfer_threshold, (fake, fake, 0, 4, 0.5, 0, fake, None)),
                     (lib.dllm_transfer_edit, (fake, fake, fake, fake, 3, 0, 0.5, fake, None)),
                     (lib.dllm_transfer_schedule, (fake, 0, 4, fake, None)),
                     (lib.dllm_block_causal_mask, (0, 4, fake, None))]:
        assert fn(*args) == 0          # empty: nothing launched


def test_binding_refuses_cpu_tensors(lib):
    import torch
    import commit_step_amd as dc
    with pytest.raises(ValueError):
        dc.token_stats(torch.zeros(1, 2, 8))
    with pytest.raises(ValueError):
        dc.threshold_transfer(torch.zeros(1, 2), torch.zeros(1, 2, dtype=torch.bool), 0.5)
