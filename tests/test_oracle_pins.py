"""Pins of the oracle against what the pages and the mathematics fix (CPU only).

Each test checks the oracle against something other than itself: a closed form,
an invariant, a brute force over every prefix of tiny rows, a textbook special
case computed with a library routine, or a value the pages print
(tests/golden/, each file with its citation).
"""
import math
import os
from fractions import Fraction
from itertools import product

import numpy as np
import pytest

import oracle
from oracle.rules import block_ranges, block_causal_mask

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return [ln.split() for ln in fh if ln.strip() and not ln.startswith("#")]


def _stats4(row, T=0.0, seed=0, step=0, b=0, l=0, suppress=()):
    row = np.asarray(row, dtype=np.float64)
    V = row.shape[0]
    sup = np.zeros(V, dtype=bool)
    sup[list(suppress)] = True
    return oracle.token_stats_row(row, float(np.float32(T)), seed, step, b, l, sup)


def _stats1(row, **kw):
    return _stats4(row, **kw)[:3]


def _margin(row, **kw):
    return _stats4(row, **kw)[3]


# ----------------------------------------------------------------- token stats

@pytest.mark.parametrize("V,suppress", [(1, ()), (7, ()), (4096, (4095,)), (1000, (0, 5, 999))])
def test_uniform_row_closed_form(V, suppress):
    x0, p, H = _stats1(np.full(V, 0.37), suppress=suppress)
    n = V - len(suppress)
    assert p == pytest.approx(1.0 / n, rel=1e-14)
    assert H == pytest.approx(math.log(n), rel=1e-14, abs=1e-15)
    assert x0 == min(set(range(V)) - set(suppress))


def test_one_hot_row():
    row = np.zeros(5000)
    row[1234] = 1000.0
    x0, p, H = _stats1(row)
    assert (x0, p, H) == (1234, 1.0, 0.0)


# ----------------------------------------------------------------- margin
# mojo-dllm "The GPU path", row statistics paragraph: topk_margin is p minus the
# runner-up's probability, the runner-up being the largest logit at any other
# index.

@pytest.mark.parametrize("V,k,a,bv", [(10, 1, 2.0, -1.0), (100, 1, 0.5, 0.0), (4096, 1, 9.0, -3.0),
                                      (50, 2, 3.0, 0.0), (777, 5, 1.0, -1.0)])
def test_margin_two_level_closed_form(V, k, a, bv):
    rng = np.random.default_rng(V * 3 + k)
    row = np.full(V, bv)
    row[rng.choice(V, size=k, replace=False)] = a
    want = (math.exp(a) - math.exp(bv)) / (math.exp(a) + (V - 1) * math.exp(bv)) if k == 1 else 0.0
    assert _margin(row) == pytest.approx(want, rel=1e-13, abs=0)


def test_margin_three_level_closed_form():
    V, h1, h2 = 300, 7.0, 5.5
    row = np.zeros(V)
    row[42], row[17] = h1, h2
    want = (math.exp(h1) - math.exp(h2)) / (math.exp(h1) + math.exp(h2) + V - 2)
    assert _margin(row) == pytest.approx(want, rel=1e-13)


@pytest.mark.parametrize("delta", [1e-3, 1e-7, 1e-10])
def test_margin_near_tie_is_tanh(delta):
    # two ids, logits 0 and -delta: p1 - p2 = tanh(delta / 2), relatively exact
    # even where 1 - e^-delta would cancel
    assert _margin([0.0, -delta]) == pytest.approx(math.tanh(delta / 2), rel=1e-12, abs=0)


def test_margin_limits_and_degenerate_rows():
    assert _margin(np.full(9, 1.5)) == 0.0                          # uniform
    row = np.zeros(20); row[[3, 11]] = 4.0
    assert _margin(row) == 0.0                                      # tie at the maximum
    assert _margin(np.arange(6.0), suppress=(0, 1, 2, 3, 4)) == 1.0  # one id left
    row = np.zeros(8); row[5] = np.inf
    assert _margin(row) == 1.0                                      # one +inf id
    row[2] = np.inf
    assert _margin(row) == 0.0                                      # two +inf ids
    assert _margin(np.full(5, -np.inf)) == 0.0                      # uniform over 5
    assert _margin(np.full(5, np.nan), suppress=(0, 1, 2, 3)) == 1.0


def test_margin_brute_force_tiny_rows():
    rng = np.random.default_rng(17)
    for _ in range(300):
        V = int(rng.integers(1, 12))
        row = rng.standard_normal(V) * 3
        row[rng.random(V) < 0.15] = np.nan
        sup = tuple(v for v in range(V) if rng.random() < 0.2)
        if len(sup) == V:
            sup = sup[1:]
        allowed = [v for v in range(V) if v not in sup]
        vals = np.array([-np.inf if np.isnan(row[v]) else row[v] for v in allowed])
        if np.isneginf(vals).all():
            p = np.full(len(allowed), 1.0 / len(allowed))
        else:
            e = np.exp(vals - vals.max())
            p = e / e.sum()
        p = np.sort(p)[::-1]
        want = p[0] - (p[1] if len(p) > 1 else 0.0)
        assert _margin(row, suppress=sup) == pytest.approx(want, rel=1e-11, abs=1e-15)


def test_margin_does_not_depend_on_sampling():
    row = np.random.default_rng(3).standard_normal(500) * 2
    g = _margin(row)
    for T, seed in ((0.7, 5), (2.0, 99)):
        assert _margin(row, T=T, seed=seed) == g


@pytest.mark.parametrize("V,k,a,bv", [(10, 1, 2.0, -1.0), (100, 3, 0.5, 0.0), (4096, 7, 9.0, -3.0)])
def test_two_level_row_closed_form(V, k, a, bv):
    rng = np.random.default_rng(V + k)
    hi = np.sort(rng.choice(V, size=k, replace=False))
    row = np.full(V, bv)
    row[hi] = a
    pa = math.exp(a) / (k * math.exp(a) + (V - k) * math.exp(bv))
    pb = math.exp(bv) / (k * math.exp(a) + (V - k) * math.exp(bv))
    Hc = -k * pa * math.log(pa) - (V - k) * pb * math.log(pb)
    x0, p, H = _stats1(row)
    assert x0 == hi[0]
    assert p == pytest.approx(pa, rel=1e-13, abs=0)
    assert H == pytest.approx(Hc, rel=1e-12, abs=0)


@pytest.mark.parametrize("V,D", [(1000, 45.0), (50000, 60.0), (7, 300.0)])
def test_peaked_two_level_row_closed_form(V, D):
    """One entry D nats above V-1 equal ones: z- = (V-1) e^-D,
    H = log1p(z-) + D z- / (1 + z-), p = 1 / (1 + z-); exact relative accuracy
    is required even when z- is far below the float64 resolution of 1."""
    row = np.zeros(V)
    row[V // 3] = D
    zm = (V - 1) * math.exp(-D)
    x0, p, H = _stats1(row)
    assert x0 == V // 3
    assert p == pytest.approx(1.0 / (1.0 + zm), rel=1e-15, abs=0)
    assert H == pytest.approx(math.log1p(zm) + D * zm / (1.0 + zm), rel=1e-12, abs=0)


def test_moment_identities_on_random_rows():
    """H = log z - S2 / z and greedy p = 1 / z with z = sum e^(x-m),
    S2 = sum e^(x-m) (x-m) (mojo-dllm "The GPU path", row statistics paragraph)."""
    rng = np.random.default_rng(7)
    for V in (2, 17, 4096):
        for scale in (0.1, 3.0, 30.0):
            row = rng.standard_normal(V) * scale
            x0, p, H = _stats1(row)
            m = row.max()
            e = np.exp(row - m)
            z = math.fsum(e)
            s2 = math.fsum(e * (row - m))
            assert x0 == int(np.argmax(row))
            assert p == pytest.approx(1.0 / z, rel=1e-12)
            assert H == pytest.approx(math.log(z) - s2 / z, rel=1e-9, abs=0)


def test_suppress_equals_deleting_the_ids():
    """suppress_ids are removed before the softmax ("Deviations from the references")."""
    rng = np.random.default_rng(3)
    V = 300
    row = rng.standard_normal(V) * 2
    row[[4, 77]] += 9.0              # make a suppressed id the raw argmax
    sup = (4, 77, 299)
    keep = np.array([v for v in range(V) if v not in sup])
    x0, p, H = _stats1(row, suppress=sup)
    x0d, pd, Hd = _stats1(row[keep])
    assert x0 not in sup and x0 == keep[x0d]
    assert p == pytest.approx(pd, rel=1e-14)
    assert H == pytest.approx(Hd, rel=1e-14)


def test_nan_counts_as_minus_inf():
    rng = np.random.default_rng(11)
    row = rng.standard_normal(64)
    with_nan = row.copy()
    with_nan[[3, 10]] = np.nan
    with_inf = row.copy()
    with_inf[[3, 10]] = -np.inf
    assert _stats1(with_nan) == _stats1(with_inf)
    x0, p, H = _stats1(with_nan)
    assert np.isfinite(p) and np.isfinite(H) and x0 not in (3, 10)


def test_degenerate_rows_are_limits():
    V = 16
    # every unsuppressed entry -inf or NaN: uniform over the unsuppressed ids
    row = np.full(V, -np.inf)
    row[2] = np.nan
    x0, p, H = _stats1(row, suppress=(0,))
    assert (x0, p) == (1, 1.0 / 15) and H == pytest.approx(math.log(15))
    # limit check: a finite row with a huge common offset converges to the same
    x0f, pf, Hf = _stats1(np.full(V, -1e300), suppress=(0,))
    assert (x0f, pf) == (x0, p) and Hf == pytest.approx(H)
    # +inf entries: uniform over the +inf ids
    row = np.zeros(V)
    row[[5, 9, 12]] = np.inf
    row[7] = np.nan
    x0, p, H = _stats1(row, suppress=(9,))
    assert (x0, p) == (5, 0.5) and H == pytest.approx(math.log(2))
    # a finite row whose two top entries run away converges to that
    fin = np.zeros(V)
    fin[[5, 12]] = 1e6
    x0f, pf, Hf = _stats1(fin, suppress=(9,))
    assert (x0f, pf) == (x0, p) and Hf == pytest.approx(H)


def test_all_suppressed_is_an_error():
    with pytest.raises(ValueError):
        _stats1(np.zeros(3), suppress=(0, 1, 2))


def test_token_stats_batch_matches_rows_and_bf16_widening():
    rng = np.random.default_rng(5)
    x32 = (rng.standard_normal((2, 3, 50)) * 3).astype(np.float32)
    st = oracle.token_stats(x32, "f32", suppress_ids=(7,))
    for b, l in product(range(2), range(3)):
        assert (st.x0[b, l], st.prob[b, l], st.entropy[b, l]) == \
            _stats1(x32[b, l].astype(np.float64), suppress=(7,))
    # bf16 widening is exact: bits << 16
    bits = np.array([[[0x3F80, 0xC000, 0x7F80, 0x0001]]], dtype=np.uint16)
    w = oracle.widen_logits(bits, "bf16")
    assert w.tolist() == [[[1.0, -2.0, np.inf, 2.0 ** -133]]]


# ----------------------------------------------------------------- Philox / Gumbel

def test_philox_known_answer_vectors():
    for r in _golden_rows("philox4x32_10_kat.txt"):
        v = [int(t, 16) for t in r]
        out = oracle.philox4x32_10(tuple(v[0:4]), tuple(v[4:6]))
        assert [int(o) for o in out] == v[6:10]


def test_uniform_mapping_open_interval_and_exact_in_float32():
    u = oracle.uniform_from_word(np.array([0, 511, 512, 0xFFFFFFFF], dtype=np.uint64))
    assert u[0] == 2.0 ** -24 and u[1] == 2.0 ** -24
    assert u[2] == 3 * 2.0 ** -24
    assert u[3] == 1.0 - 2.0 ** -24
    assert np.all(u.astype(np.float32).astype(np.float64) == u)


def test_philox_uniform_ks_and_gumbel_moments():
    from scipy import stats
    u = oracle.uniform_from_word(oracle.philox_words(123, 4, 1, 2, 400000))
    assert stats.kstest(u, "uniform").pvalue > 1e-3
    g = oracle.gumbel_noise(99, 0, 3, 5, 1_000_000)
    assert abs(g.mean() - 0.5772156649) < 0.01
    assert abs(g.var() - math.pi ** 2 / 6) < 0.02


def test_noise_depends_on_every_counter_word():
    base = oracle.philox_words(5, 1, 2, 3, 64)
    for args in [(6, 1, 2, 3), (5, 2, 2, 3), (5, 1, 3, 3), (5, 1, 2, 4), (5 + (1 << 32), 1, 2, 3)]:
        assert not np.array_equal(base, oracle.philox_words(*args, 64))


@pytest.mark.parametrize("T", [0.5, 0.7, 1.0, 2.0])
def test_gumbel_max_frequencies_follow_tempered_softmax(T):
    """Gumbel-max: argmax(l / T + g) is distributed as softmax(l / T)."""
    from scipy import stats
    ell = np.array([0.0, 0.5, -1.0, 1.2, 0.3, -0.4, 0.9, 0.1])
    V, n = ell.shape[0], 6000
    counts = np.zeros(V)
    sup = np.zeros(V, dtype=bool)
    Tf = float(np.float32(T))
    for i in range(n):
        x0, _, _, _ = oracle.token_stats_row(ell, Tf, 2024, 0, i % 97, i // 97, sup)
        counts[x0] += 1
    p = np.exp(ell / Tf - (ell / Tf).max())
    p /= p.sum()
    assert stats.chisquare(counts, n * p).pvalue > 1e-3


def test_sampling_keeps_untempered_prob_and_zero_temperature_is_greedy():
    rng = np.random.default_rng(8)
    row = rng.standard_normal(256) * 2
    g0 = _stats1(row)
    for seed in (1, 2, 3):
        assert _stats1(row, T=0.0, seed=seed) == g0
    x0, p, H = _stats1(row, T=0.7, seed=1, step=3)
    m = row.max()
    z = np.exp(row - m).sum()
    assert p == pytest.approx(math.exp(row[x0] - m) / z, rel=1e-12)
    assert H == g0[2]


def test_every_position_gets_its_own_noise():
    row = np.zeros(512)            # flat row: the draw is decided by the noise alone
    draws = {_stats1(row, T=1.0, seed=77, b=b, l=l)[0] for b in range(3) for l in range(8)}
    assert len(draws) > 12
    steps = {_stats1(row, T=1.0, seed=77, step=s)[0] for s in range(8)}
    assert len(steps) > 4


# ----------------------------------------------------------------- rules

def _exact(x):
    return Fraction(*float(x).as_integer_ratio())


def test_threshold_force_one_and_bounds():
    rng = np.random.default_rng(1)
    for _ in range(200):
        L = int(rng.integers(1, 20))
        c = rng.uniform(0, 1, size=(1, L)).astype(np.float32)
        cand = rng.random((1, L)) < 0.6
        tau = float(rng.uniform(0, 1.2))
        out = oracle.threshold_transfer(c, cand, tau)
        assert not np.any(out & ~cand)
        n_pass = int(np.sum(cand & (c.astype(np.float64) >= tau)))
        if cand.any():
            assert out.sum() == max(n_pass, 1)
            if n_pass == 0:
                cc = np.where(cand, c, -1.0)
                assert out[0, int(np.argmax(cc))]
        else:
            assert not out.any()
    c = np.array([[0.2, 0.7, 0.7, 0.1]], dtype=np.float32)
    cand = np.ones((1, 4), dtype=bool)
    assert oracle.threshold_transfer(c, cand, 0.0).all()
    assert oracle.threshold_transfer(c, cand, 1.5).tolist() == [[False, True, False, False]]


def test_threshold_strict_differs_only_at_equality():
    c = np.array([[0.5, 0.25, 0.75, 0.5]], dtype=np.float32)
    cand = np.ones((1, 4), dtype=bool)
    assert oracle.threshold_transfer(c, cand, 0.5).tolist() == [[True, False, True, True]]
    assert oracle.threshold_transfer(c, cand, 0.5, strict=True).tolist() == [[False, False, True, False]]


def test_topk_exact_count_and_stable_ties():
    rng = np.random.default_rng(2)
    for _ in range(300):
        L = int(rng.integers(1, 16))
        c = rng.choice([0.1, 0.5, 0.9], size=(2, L)).astype(np.float32)
        cand = rng.random((2, L)) < 0.7
        k = rng.integers(-2, L + 3, size=2)
        out = oracle.topk_transfer(c, cand, k)
        for b in range(2):
            C = np.flatnonzero(cand[b])
            assert out[b].sum() == min(max(int(k[b]), 0), len(C))
            assert not np.any(out[b] & ~cand[b])
            # every committed beats every uncommitted candidate, ties by position
            for i in np.flatnonzero(out[b]):
                for j in C:
                    if not out[b, j]:
                        assert c[b, i] > c[b, j] or (c[b, i] == c[b, j] and i < j)


def _brute_factor(c_sorted, f):
    best = 0
    for n in range(len(c_sorted) + 1):
        if all((i + 1) * (1 - _exact(c_sorted[i])) <= _exact(f) for i in range(n)):
            best = n
    return max(best, 1) if c_sorted else 0


def test_factor_brute_force_every_prefix():
    rng = np.random.default_rng(4)
    levels = np.array([1.0, 0.999, 0.9, 0.75, 0.5, 0.3, 0.0], dtype=np.float32)
    for _ in range(1500):
        L = int(rng.integers(1, 9))
        c = rng.choice(levels, size=(1, L)).astype(np.float32) if rng.random() < 0.5 \
            else rng.uniform(0, 1, size=(1, L)).astype(np.float32)
        cand = rng.random((1, L)) < 0.8
        f = float(rng.choice([0.0, 0.1, 0.5, 1.0, 2.0, 3.5]))
        out = oracle.factor_transfer(c, cand, f)
        C = [l for l in range(L) if cand[0, l]]
        cs = sorted((float(c[0, l]) for l in C), reverse=True)
        assert out.sum() == _brute_factor(cs, f)
        # the committed set is a top prefix of the confidence order
        if out.any():
            assert c[0][out[0]].min() >= c[0][cand[0] & ~out[0]].max(initial=-1.0)


def test_factor_no_off_by_one():
    """Only the last sorted candidate fails: it stays uncommitted ("Deviations")."""
    c = np.array([[0.9, 0.95, 0.2]], dtype=np.float32)
    cand = np.ones((1, 3), dtype=bool)
    # i=0: 1 * 0.05 ok; i=1: 2 * 0.1 = 0.2 ok; i=2: 3 * 0.8 = 2.4 > 1
    assert oracle.factor_transfer(c, cand, 1.0).tolist() == [[True, True, False]]
    assert oracle.factor_transfer(c, cand, 3.0).all()            # f >= |C| commits all
    assert oracle.factor_transfer(c, cand, 0.0).sum() == 1       # at least one


def _brute_entropy(h_sorted, gamma):
    best = 0
    for n in range(len(h_sorted) + 1):
        if all(sum((_exact(h) for h in h_sorted[:i]), Fraction(0)) <= _exact(gamma)
               for i in range(n)):
            best = n
    return max(best, 1) if h_sorted else 0


def test_entropy_bound_brute_force_every_prefix():
    rng = np.random.default_rng(6)
    for _ in range(1500):
        L = int(rng.integers(1, 9))
        h = (rng.choice([0.0, 0.1, 0.25, 0.5, 1.0], size=(1, L)) if rng.random() < 0.5
             else rng.exponential(0.3, size=(1, L))).astype(np.float32)
        cand = rng.random((1, L)) < 0.8
        gamma = float(rng.choice([0.0, 0.1, 0.35, 0.5, 1.0, 5.0]))
        out = oracle.entropy_bound_transfer(h, cand, gamma)
        C = [l for l in range(L) if cand[0, l]]
        hs = sorted(float(h[0, l]) for l in C)
        assert out.sum() == _brute_entropy(hs, gamma)
        if out.any():
            assert h[0][out[0]].max() <= h[0][cand[0] & ~out[0]].min(initial=np.inf)


def test_entropy_bound_exclusive_sum_and_gamma_zero():
    h = np.array([[0.3, 0.0, 0.0, 0.2, 0.0]], dtype=np.float32)
    cand = np.ones((1, 5), dtype=bool)
    # gamma = 0: the leading zero-entropy candidates plus one more
    assert oracle.entropy_bound_transfer(h, cand, 0.0).tolist() == [[False, True, True, True, True]]
    # exclusive: S_3 = 0 + 0 + 0 = 0 <= 0.2 admits 0.2; S_4 = 0.2 <= 0.25 admits 0.3
    assert oracle.entropy_bound_transfer(h, cand, 0.25).all()
    assert oracle.entropy_bound_transfer(h, cand, -1.0).sum() == 1   # at least one


def test_rules_nan_scores_rank_last():
    c = np.array([[np.nan, 0.4, 0.6]], dtype=np.float32)
    cand = np.ones((1, 3), dtype=bool)
    assert oracle.topk_transfer(c, cand, [2]).tolist() == [[False, True, True]]
    assert oracle.threshold_transfer(c, cand, 0.99).tolist() == [[False, False, True]]
    h = np.array([[np.nan, 0.4, 0.1]], dtype=np.float32)
    assert oracle.entropy_bound_transfer(h, cand, 1.0).tolist() == [[True, True, True]]
    assert oracle.entropy_bound_transfer(h, cand, 0.45).tolist() == [[False, True, True]]


def test_edit_rule_invariants():
    rng = np.random.default_rng(9)
    x0 = rng.integers(0, 4, size=(3, 40)).astype(np.int32)
    tok = rng.integers(0, 4, size=(3, 40)).astype(np.int32)
    p = rng.uniform(0, 1, size=(3, 40)).astype(np.float32)
    ed = rng.random((3, 40)) < 0.5
    out = oracle.edit_transfer(x0, p, tok, ed, 0.5)
    assert not np.any(out & ~ed) and not np.any(out & (x0 == tok))
    assert np.array_equal(out, ed & (x0 != tok) & (p.astype(np.float64) > 0.5))
    assert not oracle.edit_transfer(x0, p, tok, ed, 1.0).any()
    # strict: p == tau is not edited
    assert not oracle.edit_transfer(np.array([[1]]), np.array([[0.5]], np.float32),
                                    np.array([[0]]), np.array([[True]]), 0.5).any()


# ----------------------------------------------------------------- schedule / blocks

def test_schedule_printed_examples():
    for r in _golden_rows("schedule_examples.txt"):
        n, steps, quotas = int(r[0]), int(r[1]), [int(t) for t in r[2:]]
        assert oracle.transfer_schedule([n], steps)[0].tolist() == quotas


def test_schedule_invariants():
    rng = np.random.default_rng(10)
    n = rng.integers(0, 600, size=64)
    for steps in (1, 3, 8, 32, 64, 100):
        q = oracle.transfer_schedule(n, steps)
        assert q.shape == (64, steps) and q.dtype == np.int32
        assert np.array_equal(q.sum(axis=1), n)
        assert np.all(q.max(axis=1) - q.min(axis=1) <= 1)
        assert np.all(np.diff(q, axis=1) <= 0)
    assert oracle.transfer_schedule([32], 32)[0].tolist() == [1] * 32   # LLaDA-2 block 32, 32 steps
    assert oracle.transfer_schedule([37], 8)[0].tolist() == [5, 5, 5, 5, 5, 4, 4, 4]
    assert oracle.transfer_schedule([-3, 0], 4).tolist() == [[0] * 4, [0] * 4]


def test_block_ranges_printed_example_and_invariants():
    for r in _golden_rows("block_examples.txt"):
        G, bl, n = map(int, r)
        for P in (0, 5, 77):
            assert len(block_ranges(P, G, bl)) == n
    for P, G, bl in product([0, 1, 31, 32, 77, 100], [0, 1, 31, 32, 33, 435], [1, 7, 32]):
        for align in (False, True):
            rs = block_ranges(P, G, bl, align)
            if G == 0:
                assert rs == []
                continue
            lo = (P // bl) * bl if align else P
            assert rs[0][0] == lo and rs[-1][1] == P + G
            assert all(s < e for s, e in rs)
            assert all(rs[i][1] == rs[i + 1][0] for i in range(len(rs) - 1))
            assert all(e - s == bl for s, e in rs[:-1])
            if align:
                assert all(s % bl == 0 for s, _ in rs)
                assert len(rs) == -(-(P + G) // bl) - P // bl
            else:
                assert len(rs) == -(-G // bl)
    rs = block_ranges(77, 435, 32, align=True)
    assert len(rs) == 14 and rs[0] == (64, 96) and rs[-1] == (480, 512)
    with pytest.raises(ValueError):
        block_ranges(0, 10, 0)


def test_block_causal_mask_special_cases():
    for L in (1, 5, 33):
        causal = np.where(np.triu(np.ones((L, L), dtype=bool), k=1), -np.inf, 0.0)
        assert np.array_equal(block_causal_mask(L, 1), causal.astype(np.float32))
        assert np.array_equal(block_causal_mask(L, L), np.zeros((L, L), np.float32))
        assert np.array_equal(block_causal_mask(L, L + 10), np.zeros((L, L), np.float32))
    M = block_causal_mask(70, 16)
    assert M.dtype == np.float32 and set(np.unique(M).tolist()) == {0.0, -np.inf}
    for q in range(70):
        assert np.array_equal(M[q], M[(q // 16) * 16])          # rows of a block agree
        keep = M[q] == 0                                         # keep-mask form
        assert keep[: (q // 16 + 1) * 16].all() and not keep[(q // 16 + 1) * 16:].any()
    assert block_causal_mask(0, 4).shape == (0, 0)


# ----------------------------------------------------------------- threshold schedules
# mlxcel "Block Diffusion", "LLaDA-2 Block Unmasking": an initial / floor
# confidence threshold (0.95 by default) and a linearly decaying threshold.

def test_decaying_threshold_endpoints_slope_and_floor():
    assert oracle.decaying_threshold(0.95, 0.95, 0.0, 31) == 0.95        # the default: constant
    assert oracle.decaying_threshold(0.95, 0.7, 0.01, 0) == 0.95
    assert oracle.decaying_threshold(0.95, 0.7, 0.01, 10) == pytest.approx(0.85, abs=1e-15)
    assert oracle.decaying_threshold(0.95, 0.7, 0.01, 25) == 0.7          # reaches the floor
    assert oracle.decaying_threshold(0.95, 0.7, 0.01, 1000) == 0.7        # and stays there
    vals = [oracle.decaying_threshold(0.9, 0.5, 0.03, s) for s in range(12)]
    assert all(a >= b for a, b in zip(vals, vals[1:]))
    with pytest.raises(ValueError):
        oracle.decaying_threshold(0.9, 0.5, 0.03, -1)


def test_per_row_thresholds_act_row_by_row():
    rng = np.random.default_rng(41)
    B, L = 5, 30
    conf = rng.random((B, L)).astype(np.float32)
    cand = rng.random((B, L)) < 0.6
    taus = np.array([0.2, 0.5, 0.99, 0.0, 0.7])
    for strict in (False, True):
        got = oracle.threshold_transfer(conf, cand, taus, strict)
        for b in range(B):
            one = oracle.threshold_transfer(conf[b:b + 1], cand[b:b + 1], float(taus[b]), strict)
            assert np.array_equal(got[b:b + 1], one)
        # a row whose threshold no candidate reaches commits exactly one
        assert got[2].sum() == (1 if cand[2].any() else 0)
    with pytest.raises(ValueError):
        oracle.threshold_transfer(conf, cand, np.array([0.5, np.nan, 0.5, 0.5, 0.5]))
