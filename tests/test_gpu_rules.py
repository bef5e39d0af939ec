"""GPU parity of the commit rules, the schedule and the block helpers.

Rule isolation: the same float32 scores go to the HIP rules and to the oracle,
so every commit mask must match bit for bit (the comparisons and sums are exact
on both sides).  Inputs mix quantized scores (many exact ties), NaN and
+-inf scores, empty and full candidate sets, and rows up to DLLM_MAX_L.
"""
import math

import numpy as np
import pytest
import torch

import commit_step_amd as dc
import oracle
from gpu_util import log, to_dev
from workloads import random_logits

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1), (3, 7), (2, 64), (4, 256), (2, 513), (1, 1000), (1, 4096)]


def _scores(rng, B, L, kind, special=False):
    if kind == "conf":
        if rng.random() < 0.5:
            s = rng.choice(np.float32([0.0, 0.1, 0.5, 0.9, 0.95, 0.999, 1.0]), size=(B, L))
        else:
            s = rng.uniform(0, 1, size=(B, L)).astype(np.float32)
    else:
        if rng.random() < 0.5:
            s = rng.choice(np.float32([0.0, 0.01, 0.1, 0.25, 0.5, 2.0]), size=(B, L))
        else:
            s = rng.exponential(0.2, size=(B, L)).astype(np.float32)
    s = s.astype(np.float32)
    if special and L >= 4:
        flat = s.reshape(-1)
        idx = rng.choice(flat.size, size=min(flat.size, 6), replace=False)
        flat[idx[:2]] = np.nan
        flat[idx[2:3]] = np.inf
        flat[idx[3:4]] = -np.inf
        flat[idx[4:5]] = -0.0
    return s


def _cand(rng, B, L):
    mode = rng.integers(4)
    if mode == 0:
        return np.zeros((B, L), bool)
    if mode == 1:
        return np.ones((B, L), bool)
    return rng.random((B, L)) < rng.uniform(0.05, 0.95)


@pytest.mark.parametrize("B,L", SHAPES)
def test_rule_isolation_bit_exact(B, L):
    rng = np.random.default_rng(B * 10007 + L)
    trials = 12 if L <= 1000 else 4
    for trial in range(trials):
        special = trial % 3 == 2
        cand = _cand(rng, B, L)
        conf = _scores(rng, B, L, "conf", special)
        ent = _scores(rng, B, L, "ent", special)
        c_t, e_t, m_t = to_dev(conf), to_dev(ent), to_dev(cand)
        tau = float(rng.choice([0.0, 0.5, 0.9, 0.95, 1.0, 1.5]))
        strict = bool(rng.integers(2))
        got = dc.threshold_transfer(c_t, m_t, tau, strict).cpu().numpy()
        assert np.array_equal(got, oracle.threshold_transfer(conf, cand, tau, strict)), \
            f"threshold B={B} L={L} trial={trial}"
        k = rng.integers(-2, L + 3, size=B).astype(np.int32)
        got = dc.topk_transfer(c_t, m_t, to_dev(k)).cpu().numpy()
        assert np.array_equal(got, oracle.topk_transfer(conf, cand, k)), f"topk B={B} L={L}"
        f = float(rng.choice([0.0, 0.1, 0.5, 1.0, 2.0, 1e300, math.inf, -math.inf]))
        got = dc.factor_transfer(c_t, m_t, f).cpu().numpy()
        assert np.array_equal(got, oracle.factor_transfer(conf, cand, f)), \
            f"factor B={B} L={L} f={f} trial={trial}"
        g = float(rng.choice([0.0, 0.1, 0.35, 0.5, 1.0, 5.0, -1.0, 1e-40, 1e300, math.inf,
                              -math.inf]))
        got = dc.entropy_bound_transfer(e_t, m_t, g).cpu().numpy()
        assert np.array_equal(got, oracle.entropy_bound_transfer(ent, cand, g)), \
            f"entropy_bound B={B} L={L} gamma={g} trial={trial}"
        x0 = rng.integers(0, 3, size=(B, L)).astype(np.int32)
        tok = rng.integers(0, 3, size=(B, L)).astype(np.int32)
        te = float(rng.choice([0.0, 0.5, 0.9, 1.0]))
        got = dc.edit_transfer(to_dev(x0), c_t, to_dev(tok), m_t, te).cpu().numpy()
        assert np.array_equal(got, oracle.edit_transfer(x0, conf, tok, cand, te)), "edit"
    log(f"rule isolation B={B} L={L}: {trials} trials bit-exact")


def test_entropy_bound_exact_sum_at_the_boundary():
    """Sums that land exactly on gamma, and sums of tiny and huge terms."""
    h = np.array([[0.1, 0.2, 0.3, 0.4]], np.float32)
    cand = np.ones((1, 4), bool)
    s01 = float(np.float32(0.1)) + float(np.float32(0.2))
    for g in [0.0, s01, np.nextafter(s01, 0), np.nextafter(s01, 1), 0.3, 1.0]:
        got = dc.entropy_bound_transfer(to_dev(h), to_dev(cand), float(g)).cpu().numpy()
        assert np.array_equal(got, oracle.entropy_bound_transfer(h, cand, float(g))), g
    h = np.array([[1e-45, 3e38, 1e-30, 2.0, 1e-45]], np.float32)
    cand = np.ones((1, 5), bool)
    for g in [0.0, 1e-45, 2e-45, 1e-30, 2.0 + 1e-30, 3e38, 1e39]:
        got = dc.entropy_bound_transfer(to_dev(h), to_dev(cand), float(g)).cpu().numpy()
        assert np.array_equal(got, oracle.entropy_bound_transfer(h, cand, float(g))), g


def test_schedule_parity():
    rng = np.random.default_rng(3)
    for B, steps in [(1, 8), (5, 1), (64, 32), (7, 100), (1000, 3)]:
        n = rng.integers(-5, 700, size=B).astype(np.int32)
        got = dc.transfer_schedule(to_dev(n), steps).cpu().numpy()
        assert np.array_equal(got, oracle.transfer_schedule(n, steps)), (B, steps)
    got = dc.transfer_schedule(to_dev(np.array([32], np.int32)), 8).cpu().numpy()
    assert got.tolist() == [[4] * 8]


@pytest.mark.parametrize("L,bl", [(1, 1), (5, 1), (5, 2), (33, 7), (64, 64), (70, 200),
                                  (2048, 32), (1023, 32)])
def test_block_causal_mask_parity(L, bl):
    got = dc.block_causal_mask(L, bl).cpu().numpy()
    ref = oracle.block_causal_mask(L, bl)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (L, bl)


def test_empty_shapes_launch_nothing():
    z = torch.zeros((0, 5), dtype=torch.float32, device="cuda")
    m = torch.zeros((0, 5), dtype=torch.bool, device="cuda")
    assert dc.threshold_transfer(z, m, 0.5).shape == (0, 5)
    st = dc.token_stats(torch.zeros((2, 0, 8), dtype=torch.bfloat16, device="cuda"))
    assert st.x0.shape == (2, 0)
    assert dc.block_causal_mask(0, 4).shape == (0, 0)


@pytest.mark.parametrize("B,L,V,T", [(1, 256, 8192, 0.0), (3, 40, 30000, 0.0),
                                     (1, 6, 262144, 0.0), (2, 16, 5000, 0.9)])
def test_fused_rules_equal_standalone(B, L, V, T):
    """dllm_token_stats with fused rules gives the same masks as the standalone
    calls on its own outputs."""
    bits, rng = random_logits(21, B, L, V, "bf16", 2.0, 0.5, 4.0, 16.0)
    logits = to_dev(bits, "bf16")
    cand = rng.random((B, L)) < 0.6
    editable = ~cand
    tokens = rng.integers(0, V, size=(B, L)).astype(np.int32)
    m_t, e_t, tok_t = to_dev(cand), to_dev(editable), to_dev(tokens)
    k = rng.integers(0, L, size=B).astype(np.int32)
    combos = [
        [dc.Rule.threshold(m_t, 0.5)],
        [dc.Rule.threshold(m_t, 0.5, strict=True), dc.Rule.edit(e_t, tok_t, 0.3)],
        [dc.Rule.topk(m_t, to_dev(k))],
        [dc.Rule.factor(m_t, 1.0), dc.Rule.edit(e_t, tok_t, 0.9)],
        [dc.Rule.entropy_bound(m_t, 0.5), dc.Rule.edit(e_t, tok_t, 0.9)],
        [dc.Rule.entropy_bound(m_t, 3.0), dc.Rule.threshold(m_t, 0.2)],
    ]
    for rules in combos:
        st = dc.token_stats(logits, temperature=T, seed=4, rules=rules)
        for r in rules:
            if r.kind == dc.RULE_THRESHOLD:
                ref = dc.threshold_transfer(st.prob, r.mask, r.param, r.strict)
            elif r.kind == dc.RULE_TOPK:
                ref = dc.topk_transfer(st.prob, r.mask, r.k)
            elif r.kind == dc.RULE_FACTOR:
                ref = dc.factor_transfer(st.prob, r.mask, r.param)
            elif r.kind == dc.RULE_ENTROPY_BOUND:
                ref = dc.entropy_bound_transfer(st.entropy, r.mask, r.param)
            else:
                ref = dc.edit_transfer(st.x0, st.prob, r.tokens, r.mask, r.param)
            assert torch.equal(r.out, ref), f"fused kind {r.kind} differs"
            # and the oracle rule on the same (GPU) statistics agrees too
            conf = st.prob.cpu().numpy()
            c_np = r.mask.cpu().numpy()
            if r.kind == dc.RULE_ENTROPY_BOUND:
                o = oracle.entropy_bound_transfer(st.entropy.cpu().numpy(), c_np, r.param)
                assert np.array_equal(r.out.cpu().numpy(), o)
            elif r.kind == dc.RULE_FACTOR:
                assert np.array_equal(r.out.cpu().numpy(), oracle.factor_transfer(conf, c_np, r.param))
    log(f"fused == standalone for B={B} L={L} V={V} T={T}")
