"""Randomized end-to-end parity: many seeded small launches of the fused
statistics pass with one commit rule, over shapes the fixed tests do not pin
down (odd vocabularies that take the split path, vocabularies that split rows
across workgroups, single positions), fp32 and bf16 logits, greedy and
Gumbel-max, random suppress lists and random rule parameters.

For every case: x0 against the oracle (bit-exact when greedy, the near-tie
rule when sampled), prob and entropy within the dtype tolerance, and the fused
commit mask bit-exact against the oracle's rule applied to the launch's own
float32 statistics (rule isolation, so no near-bound carve-out is needed).
"""
import numpy as np
import pytest

import commit_step_amd as dc
import oracle
from gpu_util import assert_sampled_x0, assert_stats, log, stats_np, to_dev
from workloads import random_logits

pytestmark = pytest.mark.gpu

VOCABS = [1, 2, 7, 64, 1000, 1001, 4096, 5003, 8192, 12345, 33000, 70000]
N_CASES = 256


def _case(i):
    rng = np.random.default_rng(90000 + i)
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    V = int(rng.choice(VOCABS))
    B = int(rng.integers(1, 4))
    L = int(rng.choice([1, 2, 5, 16, 33, 40, 100, 257]))
    n_sup = int(rng.integers(0, min(6, V - 1) + 1)) if V > 1 else 0
    sup = tuple(sorted(set(int(v) for v in rng.choice(V, size=n_sup, replace=False)))) \
        if n_sup else ()
    T = 0.0 if rng.random() < 0.5 else float(np.float32(rng.uniform(0.4, 1.6)))
    sigma = float(rng.uniform(0.5, 4.0))
    kind = str(rng.choice(["threshold", "topk", "factor", "entropy_bound"]))
    cand = rng.random((B, L)) < rng.uniform(0.2, 1.0)
    return dict(rng=rng, dtype=dtype, V=V, B=B, L=L, sup=sup, T=T, sigma=sigma, kind=kind,
                cand=cand, seed=int(rng.integers(0, 2 ** 62)), step=int(rng.integers(0, 100)))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_fused_launch(i):
    c = _case(i)
    rng, dtype, B, L, V, sup, T, kind = (c["rng"], c["dtype"], c["B"], c["L"], c["V"], c["sup"],
                                         c["T"], c["kind"])
    log(f"case {i}: {dtype} B={B} L={L} V={V} T={T} suppress={len(sup)} rule={kind}")
    bits, _ = random_logits(1000 + i, B, L, V, dtype, c["sigma"], 0.4, 4.0, 14.0, sup)
    cand_t = to_dev(c["cand"])
    if kind == "threshold":
        tau, strict = float(rng.choice([0.3, 0.5, 0.9])), bool(rng.integers(2))
        rule = dc.Rule.threshold(cand_t, tau, strict)
    elif kind == "topk":
        k = rng.integers(-1, L + 2, size=B).astype(np.int32)
        rule = dc.Rule.topk(cand_t, to_dev(k))
    elif kind == "factor":
        f = float(rng.choice([0.2, 1.0, 3.0]))
        rule = dc.Rule.factor(cand_t, f)
    else:
        gamma = float(rng.choice([0.05, 0.5, 2.0]))
        rule = dc.Rule.entropy_bound(cand_t, gamma)
    st = dc.token_stats(to_dev(bits, dtype), temperature=T, seed=c["seed"] if T > 0 else None,
                        step=c["step"], suppress_ids=sup, rules=[rule])
    gpu = stats_np(st)
    mask = rule.out.cpu().numpy().astype(bool)
    ref = oracle.token_stats(bits, dtype, temperature=T, seed=c["seed"] if T > 0 else None,
                             step=c["step"], suppress_ids=sup)
    if T > 0:
        pos = [(b, l) for b in range(B) for l in range(L)]
        assert_sampled_x0(gpu[0], ref.x0, bits, dtype, T, c["seed"], c["step"], sup, pos,
                          f"case {i}")
        assert_stats(gpu, ref, dtype, f"case {i}", mask=(gpu[0] == ref.x0), x0_exact=False)
        assert_stats(gpu, ref, dtype, f"case {i} entropy", x0_exact=False, fields=("entropy",))
    else:
        assert_stats(gpu, ref, dtype, f"case {i}")
    assert not np.isin(gpu[0], sup).any(), f"case {i}: a suppressed id was proposed"
    if kind == "threshold":
        want = oracle.threshold_transfer(gpu[1], c["cand"], tau, strict)
    elif kind == "topk":
        want = oracle.topk_transfer(gpu[1], c["cand"], k)
    elif kind == "factor":
        want = oracle.factor_transfer(gpu[1], c["cand"], f)
    else:
        want = oracle.entropy_bound_transfer(gpu[2], c["cand"], gamma)
    assert np.array_equal(mask, want), f"case {i}: fused {kind} mask differs from the oracle's"


@pytest.mark.parametrize("i", range(120))
def test_random_margin_argmax_and_statistics_temperature(i):
    """Seeded random launches with the margin, the greedy argmax beside a
    sampled x0, and a statistics temperature: margin with prob and entropy
    within the dtype tolerance, argmax bit-exact."""
    rng = np.random.default_rng(50000 + i)
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    V = int(rng.choice([2, 7, 1000, 4096, 5003, 9000, 33000]))
    B, L = int(rng.integers(1, 4)), int(rng.choice([1, 5, 40, 100]))
    n_sup = int(rng.integers(0, min(4, V - 1) + 1))
    sup = tuple(sorted(set(int(v) for v in rng.choice(V, size=n_sup, replace=False)))) \
        if n_sup else ()
    T = 0.0 if rng.random() < 0.5 else float(np.float32(rng.uniform(0.5, 1.5)))
    Ts = float(np.float32(rng.choice([1.0, 0.5, 0.8, 1.7])))
    seed = int(rng.integers(0, 2 ** 40)) if T > 0 else None
    bits, _ = random_logits(60000 + i, B, L, V, dtype, float(rng.uniform(0.5, 4.0)), 0.4, 2.0,
                            12.0, sup)
    log(f"case {i}: {dtype} B={B} L={L} V={V} T={T} Ts={Ts} suppress={len(sup)}")
    st = dc.token_stats(to_dev(bits, dtype), temperature=T, seed=seed, step=3, suppress_ids=sup,
                        margin=True, argmax=True, stats_temperature=Ts)
    g = stats_np(st)
    am = st.argmax.cpu().numpy()
    ref = oracle.token_stats(bits, dtype, temperature=T, seed=seed, step=3, suppress_ids=sup,
                             stats_temperature=Ts)
    greedy = oracle.token_stats(bits, dtype, suppress_ids=sup, stats_temperature=Ts)
    assert np.array_equal(am, greedy.x0), f"case {i}: argmax"
    fields = ("prob", "entropy", "margin")
    if T > 0:
        pos = [(b, l) for b in range(B) for l in range(L)]
        assert_sampled_x0(g[0], ref.x0, bits, dtype, T, seed, 3, sup, pos, f"case {i}")
        assert_stats(g, ref, dtype, f"case {i}", mask=(g[0] == ref.x0), x0_exact=False,
                     fields=fields)
    else:
        assert_stats(g, ref, dtype, f"case {i}", fields=fields)
