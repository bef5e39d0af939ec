"""The topk_margin confidence (p1 - p2) and the rules that rank by margin or
by Dream's negative entropy, on the GPU against the oracle."""
import numpy as np
import pytest
import torch

import commit_step_amd as dc
import oracle
from gpu_util import assert_stats, log, stats_np, to_dev
from workloads import bf16_bits, random_logits

pytestmark = pytest.mark.gpu

MARGIN = ("prob", "entropy", "margin")


@pytest.mark.parametrize("dtype,B,L,V,T,sup", [
    ("f32", 2, 3, 9, 0.0, ()),
    ("bf16", 2, 40, 30000, 0.0, (29999,)),       # split rows
    ("bf16", 1, 300, 65536, 0.0, (7,)),           # rotated sweeps
    ("f32", 2, 16, 20000, 0.8, ()),               # sampled x0: margin does not depend on it
    ("bf16", 1, 2, 262144, 0.0, ()),              # many slices
])
def test_margin_parity(dtype, B, L, V, T, sup):
    bits, _ = random_logits(200 + V % 89, B, L, V, dtype, 2.5, 0.5, 2.0, 9.0, sup)
    log(f"margin {dtype} B={B} L={L} V={V} T={T}")
    gpu = stats_np(dc.token_stats(to_dev(bits, dtype), temperature=T, seed=4 if T else None,
                                  suppress_ids=sup, margin=True))
    ref = oracle.token_stats(bits, dtype, temperature=T, seed=4 if T else None, suppress_ids=sup)
    assert_stats(gpu, ref, dtype, f"margin {dtype}", x0_exact=(T == 0.0),
                 mask=None if T == 0.0 else (gpu[0] == ref.x0), fields=MARGIN)
    if T > 0:
        assert_stats(gpu, ref, dtype, "margin sampled", x0_exact=False, fields=("margin",))


def test_margin_ties_near_ties_and_special_rows():
    rng = np.random.default_rng(12)
    V = 5000
    rows = []
    base = rng.standard_normal(V).astype(np.float32)
    a = base.copy(); a[[10, 4000]] = 9.0; rows.append(a)                 # tie: 0
    a = base.copy(); a[10] = 9.0; a[4000] = np.nextafter(np.float32(9.0), np.float32(0)); rows.append(a)
    a = base.copy(); a[4999] = 30.0; rows.append(a)                       # peaked
    a = np.full(V, -np.inf, np.float32); a[77] = 1.0; rows.append(a)      # one finite id: 1
    a = np.full(V, -np.inf, np.float32); rows.append(a)                    # uniform: 0
    a = base.copy(); a[3] = np.inf; rows.append(a)                         # one +inf: 1
    a = base.copy(); a[[3, 8]] = np.inf; rows.append(a)                    # two +inf: 0
    a = base.copy(); a[[5, 6]] = np.nan; a[100] = 12.0; rows.append(a)    # NaN counts as -inf
    a = base.copy() * 1e5; rows.append(a)                                  # far apart
    x = np.stack(rows)[None]
    for dtype, arr in (("f32", x), ("bf16", bf16_bits(x))):
        log(f"margin special rows {dtype}")
        gpu = stats_np(dc.token_stats(to_dev(arr, dtype), margin=True))
        ref = oracle.token_stats(arr, dtype)
        assert_stats(gpu, ref, dtype, f"margin special {dtype}", fields=MARGIN)
        assert gpu[3][0, 0] == 0.0 and gpu[3][0, 4] == 0.0 and gpu[3][0, 6] == 0.0
        assert gpu[3][0, 3] == 1.0 and gpu[3][0, 5] == 1.0


@pytest.mark.parametrize("kind,param,score", [
    ("threshold", 0.6, "margin"), ("topk", 7, "margin"), ("factor", 1.0, "margin"),
    ("threshold", -0.8, "neg_entropy"), ("topk", 5, "neg_entropy"), ("factor", 2.0, "neg_entropy"),
])
def test_rules_rank_by_margin_or_negative_entropy(kind, param, score):
    rng = np.random.default_rng(14)
    B, L, V = 3, 120, 12000
    bits, _ = random_logits(15, B, L, V, "bf16", 2.5, 0.5, 2.0, 9.0)
    cand = rng.random((B, L)) < 0.6
    cm = torch.from_numpy(cand).cuda()
    if kind == "threshold":
        r = dc.Rule.threshold(cm, param, score=score)
    elif kind == "topk":
        r = dc.Rule.topk(cm, param, score=score)
    else:
        r = dc.Rule.factor(cm, param, score=score)
    log(f"rule {kind} by {score}")
    st = dc.token_stats(to_dev(bits, "bf16"), rules=[r], margin=True)
    gx, gp, ge, gm = stats_np(st)
    conf = gm if score == "margin" else (-ge).astype(np.float32)
    want = oracle.rank_rule(kind, conf, ge, cand, param)
    assert np.array_equal(r.out.cpu().numpy(), want)
    # the standalone transfer on the same confidence array agrees
    conf_t = torch.from_numpy(np.ascontiguousarray(conf)).cuda()
    if kind == "threshold":
        alone = dc.threshold_transfer(conf_t, cm, param)
    elif kind == "topk":
        alone = dc.topk_transfer(conf_t, cm, param)
    else:
        alone = dc.factor_transfer(conf_t, cm, param)
    assert np.array_equal(alone.cpu().numpy(), want)
