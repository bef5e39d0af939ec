"""Rows that are not 16-byte aligned, on the GPU against the oracle: odd
vocabularies (every row starts at another offset within 16 bytes), a base
pointer off by a few elements, padded row strides, split rows.  Each slice's
aligned body streams with 16-byte loads and its head and tail element by
element, so the cases place maxima, ties, suppressed ids, runners-up and NaN
in the head, the body and the tail.  A sampled body load starts 0 to 3
elements into a four-element generator group; the sampled cases cover each
offset and check the pick bit for bit against the same rows laid out
aligned."""
import json
from pathlib import Path

import numpy as np
import pytest
import torch

import commit_step_amd as dc
import oracle
from gpu_util import assert_sampled_x0, assert_stats, log, stats_np, to_dev
from workloads import bf16_bits

pytestmark = pytest.mark.gpu

FIELDS = ("prob", "entropy", "margin")


def _planted(rng, B, L, V, dtype):
    """Normal logits with ties of the row maximum at both ends and in the middle,
    and a runner-up near each end."""
    x = (rng.standard_normal((B, L, V)) * 2.0).astype(np.float32)
    for b in range(B):
        for l in range(L):
            r = (b * L + l) % 8
            if r % 3 == 0:
                x[b, l, [r, V // 2, V - 1 - r]] = 40.0          # first copy in the head
            elif r % 3 == 1:
                x[b, l, [V // 3, V - 1 - r]] = 40.0              # first in the body, one in the tail
                x[b, l, r] = 39.5                                # runner-up in the head
            else:
                x[b, l, V - 1 - r] = 40.0                        # maximum in the tail
                x[b, l, r] = 39.75
    return x if dtype == "f32" else bf16_bits(x)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,V", [(2, 8, 5003), (1, 16, 1001), (1, 3, 50257), (4, 64, 4099)])
def test_unaligned_rows_ties_and_runner_up(dtype, B, L, V):
    rng = np.random.default_rng(V + B)
    arr = _planted(rng, B, L, V, dtype)
    log(f"unaligned {dtype} B={B} L={L} V={V}")
    gpu = stats_np(dc.token_stats(to_dev(arr, dtype), margin=True))
    ref = oracle.token_stats(arr, dtype)
    assert_stats(gpu, ref, dtype, f"unaligned {dtype} {B}x{L}x{V}", fields=FIELDS)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_unaligned_suppressed_head_and_tail(dtype):
    B, L, V = 1, 8, 3001
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((B, L, V)) * 2.0).astype(np.float32)
    x[:, :, [0, 1, V - 1]] = 50.0                 # suppressed maxima at both ends
    x[:, :, 1500] = 20.0
    sup = (0, 1, 2, V - 2, V - 1)
    arr = x if dtype == "f32" else bf16_bits(x)
    gpu = stats_np(dc.token_stats(to_dev(arr, dtype), suppress_ids=sup, margin=True))
    ref = oracle.token_stats(arr, dtype, suppress_ids=sup)
    assert_stats(gpu, ref, dtype, f"suppressed ends {dtype}", fields=FIELDS)
    assert np.all(gpu[0] == 1500)


@pytest.mark.parametrize("dtype,off,pad", [("bf16", 1, 3), ("bf16", 3, 0), ("f32", 1, 1),
                                           ("f32", 2, 5)])
def test_unaligned_base_pointer_and_stride(dtype, off, pad):
    """logits start `off` elements into an allocation and rows are V + pad apart."""
    B, L, V = 2, 6, 4096
    rng = np.random.default_rng(off * 10 + pad)
    x = _planted(rng, B, L, V + pad + off, "f32")
    arr = x if dtype == "f32" else bf16_bits(x)
    full = to_dev(arr, dtype)                                    # (B, L, V + pad + off)
    flat = full.reshape(-1)[off:]
    rows = flat[: (B * L - 1) * (V + pad + off) + V]
    view = torch.as_strided(rows, (B, L, V), (L * (V + pad + off), V + pad + off, 1))
    log(f"base +{off} elements, stride V+{pad + off} {dtype}")
    gpu = stats_np(dc.token_stats(view, margin=True))
    host = np.lib.stride_tricks.as_strided(
        arr.reshape(-1)[off:], (B, L, V),
        (L * (V + pad + off) * arr.itemsize, (V + pad + off) * arr.itemsize, arr.itemsize))
    ref = oracle.token_stats(np.ascontiguousarray(host), dtype)
    assert_stats(gpu, ref, dtype, f"base+{off} {dtype}", fields=FIELDS)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_unaligned_nan_and_inf_in_head_and_tail(dtype):
    """Degenerate values at the ends send the row to the two-pass recomputation."""
    B, L, V = 1, 6, 2003
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((B, L, V)) * 2.0).astype(np.float32)
    x[0, 0, 0] = np.nan
    x[0, 1, V - 1] = np.nan
    x[0, 2, 1] = np.inf
    x[0, 3, [2, V - 2]] = np.inf
    x[0, 4, 0] = -np.inf
    arr = x if dtype == "f32" else bf16_bits(x)
    gpu = stats_np(dc.token_stats(to_dev(arr, dtype), margin=True))
    ref = oracle.token_stats(arr, dtype)
    assert_stats(gpu, ref, dtype, f"degenerate ends {dtype}", fields=FIELDS)


@pytest.mark.parametrize("kind", ["topk", "entropy_bound", "threshold"])
def test_unaligned_fused_rules(kind):
    """The fused rules on statistics from unaligned rows equal the oracle's rule on
    the same float32 statistics (rule isolation)."""
    B, L, V = 2, 40, 5001
    rng = np.random.default_rng(21)
    arr = _planted(rng, B, L, V, "bf16")
    cand = rng.random((B, L)) < 0.6
    cand_t = to_dev(cand)
    if kind == "topk":
        k = np.array([3, 7], dtype=np.int32)
        rule = dc.Rule.topk(cand_t, to_dev(k))
    elif kind == "entropy_bound":
        rule = dc.Rule.entropy_bound(cand_t, 1.0)
    else:
        rule = dc.Rule.threshold(cand_t, 0.5, False)
    st = dc.token_stats(to_dev(arr, "bf16"), rules=[rule])
    gpu = stats_np(st)
    ref = oracle.token_stats(arr, "bf16")
    assert_stats(gpu, ref, "bf16", f"unaligned fused {kind}")
    conf = gpu[2] if kind == "entropy_bound" else gpu[1]
    if kind == "topk":
        want = oracle.topk_transfer(conf, cand, k)
    elif kind == "entropy_bound":
        want = oracle.entropy_bound_transfer(conf, cand, 1.0)
    else:
        want = oracle.threshold_transfer(conf, cand, 0.5, False)
    assert np.array_equal(rule.out.cpu().numpy().astype(bool), np.asarray(want, bool))


def _offset_view(arr, dtype, off, pad):
    """(device view, host copy) of (B, L, V) rows starting `off` elements into
    an allocation, V + pad + off elements apart."""
    B, L, V = arr.shape
    S = V + pad + off
    big = np.zeros((B * L * S + off,), dtype=arr.dtype)
    host = np.lib.stride_tricks.as_strided(
        big[off:], (B, L, V), (L * S * big.itemsize, S * big.itemsize, big.itemsize))
    host[...] = arr
    full = to_dev(big, dtype)
    view = torch.as_strided(full[off:], (B, L, V), (L * S, S, 1))
    return view, host


@pytest.mark.parametrize("dtype,offs", [("bf16", (1, 2, 3, 4, 5, 6, 7)), ("f32", (1, 2, 3))])
@pytest.mark.parametrize("B,L,V", [(2, 8, 4096), (1, 3, 151936), (3, 40, 2056)])
def test_unaligned_sampled_matches_aligned(dtype, offs, B, L, V):
    """Sampled launches on rows 1..7 (bf16) or 1..3 (f32) elements off 16-byte
    alignment, with a padded stride so consecutive rows start at other offsets
    too: the pick equals the aligned layout's bit for bit (the same scores,
    first index on ties) and the oracle's up to near-ties; prob and entropy
    match the oracle."""
    rng = np.random.default_rng(V + 7 * B)
    x = (rng.standard_normal((B, L, V)) * 2.0).astype(np.float32)
    arr = x if dtype == "f32" else bf16_bits(x)
    T, seed, step = 0.9, 11, 2
    sup = (0, 5, V // 2 + 1, V - 3)
    aligned = stats_np(dc.token_stats(to_dev(arr, dtype), temperature=T, seed=seed, step=step,
                                      suppress_ids=sup, margin=True))
    ref = oracle.token_stats(arr, dtype, temperature=T, seed=seed, step=step, suppress_ids=sup)
    pos = [(b, l) for b in range(B) for l in range(L)]
    for off in offs:
        for pad in (0, 3):
            log(f"sampled {dtype} {B}x{L}x{V} base +{off} stride V+{pad + off}")
            view, host = _offset_view(arr, dtype, off, pad)
            gpu = stats_np(dc.token_stats(view, temperature=T, seed=seed, step=step,
                                          suppress_ids=sup, margin=True))
            bad = np.flatnonzero(gpu[0] != aligned[0])
            assert bad.size == 0, f"off {off} pad {pad}: pick differs from aligned at {bad[:10]}"
            assert_sampled_x0(gpu[0], ref.x0, arr, dtype, T, seed, step, sup, pos,
                              f"sampled base+{off}")
            assert_stats(gpu, ref, dtype, f"sampled base+{off} pad {pad}", x0_exact=False,
                         mask=(gpu[0] == ref.x0))


TIES = json.loads((Path(__file__).parent / "golden" / "sampled_ties.json").read_text())


@pytest.mark.parametrize("case", TIES["cases"], ids=lambda c: f"{c['dtype']}-{c['v1']}-{c['v2']}")
def test_unaligned_sampled_planted_ties(case):
    """Two ids that draw the same noise at this step (tests/golden/sampled_ties.json)
    carry the row's top logit, so their scores are exactly equal: the lower id
    wins, whether the two lie in the head, in one 16-byte span, in spans of
    other lanes or in the tail, on the offset layout and on the aligned one."""
    dtype, off, V, v1, v2, step = (case[k] for k in ("dtype", "off", "V", "v1", "v2", "step"))
    x = np.full((1, 1, V), -60.0, np.float32)
    x[0, 0, [v1, v2]] = 0.0
    arr = x if dtype == "f32" else bf16_bits(x)
    log(f"planted tie {dtype} base +{off} ids {v1}, {v2} step {step}")
    view, _ = _offset_view(arr, dtype, off, 0)
    for t, label in ((view, "offset"), (to_dev(arr, dtype), "aligned")):
        gpu = stats_np(dc.token_stats(t, temperature=0.8, seed=TIES["seed"], step=step))
        assert int(gpu[0][0, 0]) == v1, f"{label}: picked {int(gpu[0][0, 0])}, not {v1}"


def test_dream_shape_unaligned_matches_aligned():
    """The Dream-like workload at full size (4 x 256 x 151936 bf16, Gumbel-max
    T = 0.7, suppress list, fused factor) laid out with rows V + 1 elements
    apart, as `bench.py --workload dream_unaligned` times it: every position's
    pick equals the aligned layout's bit for bit, prob and entropy agree to
    summation order, and each launch's factor mask is the oracle's rule on
    that launch's own statistics (rule isolation).  (The aligned launch is
    checked against the oracle at every position in test_gpu_configs.)"""
    import workloads
    w = workloads.config3()
    B, L, V = w.shape
    T, seed, f = w.temperature, w.seed, w.params["f"]
    sup = tuple(w.suppress_ids)
    aligned = to_dev(w.logits, "bf16")
    padded = torch.empty((B, L, V + 1), dtype=torch.bfloat16, device="cuda")
    padded[..., :V].copy_(aligned)
    cand = to_dev(w.cand)
    res = []
    for t in (aligned, padded[..., :V]):
        log(f"dream shape, row stride {t.stride(1)}")
        rule = dc.Rule.factor(cand, f)
        st = dc.token_stats(t, temperature=T, seed=seed, step=0, suppress_ids=sup, rules=[rule])
        res.append(stats_np(st) + (rule.out.cpu().numpy(),))
    (ax, ap, ae, am), (ux, up, ue, um) = res
    bad = np.flatnonzero(ax != ux)
    assert bad.size == 0, f"picks differ at {bad[:10]}"
    c = w.cand.astype(bool)
    for label, p_, m_ in (("aligned", ap, am), ("unaligned", up, um)):
        want = np.asarray(oracle.factor_transfer(p_, c, f), bool)
        assert np.array_equal(m_.astype(bool), want), f"{label}: factor mask differs"
    for name, g, r in (("prob", up, ap), ("entropy", ue, ae)):
        rel = np.abs(g.astype(np.float64) - r) / np.maximum(np.abs(r), 1e-30)
        assert rel.max() <= 1e-5, f"{name} off by rel {rel.max():.2e}"
    log(f"  dream shape unaligned: prob max rel {np.max(np.abs(up - ap) / np.abs(ap)):.2e}")
