"""Pins of the uniform-noise decoding helpers and of the statistics
temperature (oracle/uniform.py, oracle/stats.py) -- CPU only."""
import math

import numpy as np
import pytest
from scipy import stats as sps

import oracle
from oracle.philox import philox4x32_10


# ----------------------------------------------------------------- statistics temperature

@pytest.mark.parametrize("Ts", [2.0, 0.5, 4.0, 0.125])
def test_stats_temperature_is_dividing_the_logits(Ts):
    # a power-of-two Ts divides every logit exactly, so scaling inside must
    # equal passing the divided logits
    rng = np.random.default_rng(int(Ts * 8))
    x = (rng.standard_normal((2, 3, 300)) * 4).astype(np.float32)
    x[0, 1, 5] = np.nan
    x[1, 2, :] = -np.inf
    x[1, 2, 7] = np.inf
    a = oracle.token_stats(x, "f32", stats_temperature=Ts, suppress_ids=(3,))
    b = oracle.token_stats((x / np.float32(Ts)).astype(np.float32), "f32", suppress_ids=(3,))
    for f in ("x0", "prob", "entropy", "margin"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


def test_stats_temperature_limits():
    rng = np.random.default_rng(2)
    row = rng.standard_normal((1, 1, 500)) * 3
    hot = oracle.token_stats(row.astype(np.float32), "f32", stats_temperature=1e7)
    assert hot.entropy[0, 0] == pytest.approx(math.log(500), abs=1e-5)
    cold = oracle.token_stats(row.astype(np.float32), "f32", stats_temperature=1e-6)
    assert cold.prob[0, 0] == pytest.approx(1.0, abs=1e-12) and cold.entropy[0, 0] < 1e-12
    greedy = oracle.token_stats(row.astype(np.float32), "f32")
    assert hot.x0[0, 0] == cold.x0[0, 0] == greedy.x0[0, 0]


def test_sampled_x0_does_not_depend_on_the_statistics_temperature():
    x = (np.random.default_rng(3).standard_normal((1, 4, 200)) * 2).astype(np.float32)
    a = oracle.token_stats(x, "f32", temperature=0.7, seed=5, step=2)
    b = oracle.token_stats(x, "f32", temperature=0.7, seed=5, step=2, stats_temperature=0.6)
    assert np.array_equal(a.x0, b.x0)


# ----------------------------------------------------------------- schedule, canvas, renoise

def test_linear_temperature_endpoints_and_linearity():
    N = 48
    ts = [oracle.linear_temperature(r, N, 0.4, 0.8) for r in range(N, -1, -1)]
    assert ts[0] == 0.8 and ts[-1] == pytest.approx(0.4, abs=1e-15)
    d = np.diff(ts)
    assert np.allclose(d, -(0.8 - 0.4) / N, rtol=1e-12)
    with pytest.raises(ValueError):
        oracle.linear_temperature(N + 1, N, 0.4, 0.8)


def test_uniform_canvas_range_uniformity_and_independence():
    V = 97
    c = oracle.uniform_canvas(64, 512, V, 11, 0)
    assert c.dtype == np.int32 and c.min() >= 0 and c.max() < V
    counts = np.bincount(c.ravel(), minlength=V)
    assert sps.chisquare(counts).pvalue > 1e-3
    d = oracle.uniform_canvas(64, 512, V, 11, 1)
    assert (c != d).mean() > 0.95                        # another draw, another canvas
    assert np.array_equal(c, oracle.uniform_canvas(64, 512, V, 11, 0))   # deterministic
    assert (oracle.uniform_canvas(3, 7, 1, 5, 2) == 0).all()


@pytest.mark.parametrize("k", [1, 8, 20, 30])
def test_uniform_canvas_power_of_two_vocab_takes_the_top_bits(k):
    # V = 2^k: floor(x * 2^k / 2^64) is the top k bits of the 64-bit word
    seed, draw = 123456789012345, 7
    c = oracle.uniform_canvas(2, 6, 1 << k, seed, draw)
    for b in range(2):
        for l in range(6):
            w = philox4x32_10((l, b, 0xFFFFFFFF, draw), (seed & 0xFFFFFFFF, seed >> 32))
            top = int(w[1]) >> (32 - k) if k <= 32 else None
            assert c[b, l] == top


def test_renoise_is_a_where():
    s = np.arange(10, dtype=np.int32).reshape(2, 5)
    n = -np.ones((2, 5), dtype=np.int32)
    acc = np.array([[1, 0, 1, 0, 0], [0, 0, 0, 0, 1]], dtype=bool)
    assert oracle.renoise(s, acc, n).tolist() == [[0, -1, 2, -1, -1], [-1, -1, -1, -1, 9]]


# ----------------------------------------------------------------- stopping

def test_stable_confident_stopping_counts_and_exact_mean():
    stop = oracle.StableConfidentStopping(1, 0.25)
    a = np.array([[1, 2], [3, 4]], dtype=np.int32)
    h = np.array([[0.25, 0.25], [0.0, 0.75]], dtype=np.float32)
    assert stop(a, h).tolist() == [False, False]          # nothing to compare with yet
    assert stop(a, h).tolist() == [True, False]           # stable; mean 0.25 <= 0.25; mean 0.375
    b = a.copy(); b[0, 0] = 9
    assert stop(b, h).tolist() == [False, False]          # changed: the count restarts
    h2 = np.array([[0.25, np.nextafter(np.float32(0.25), np.float32(1))], [0.0, 0.0]], np.float32)
    assert stop(b, h2).tolist() == [False, True]          # a hair above the mean bound
    zero = oracle.StableConfidentStopping(0, 0.1)
    assert zero(a, np.zeros((2, 2), np.float32)).tolist() == [True, True]
    h3 = np.array([[np.inf, 0.0], [np.nan, 0.0]], np.float32)
    assert zero(a, h3).tolist() == [False, False]         # +inf > c L; NaN compares false


def _confident(c, row):
    """One stable row through the oracle's rule (k = 0), as a bool."""
    stop = oracle.StableConfidentStopping(0, c)
    row = np.asarray(row, dtype=np.float32)
    return bool(stop(np.zeros((1, len(row)), np.int32), row[None, :])[0])


def test_stable_confident_stopping_extended_reals():
    """The mean bound sum(H) <= c L taken in the extended reals, as IEEE
    arithmetic evaluates it: sum and compare in float64 wherever float64 is
    exact for the values used."""
    inf, nan = np.inf, np.nan
    cases = [
        (0.1, [-inf, 5.0], True),          # -inf sum is below every bound
        (-inf, [-inf, 5.0], True),         # -inf <= -inf
        (0.1, [-inf, inf], False),         # -inf + inf is undefined
        (inf, [-inf, inf], False),         # ... also against an infinite bound
        (0.1, [-inf, nan], False),
        (0.1, [inf, 0.0], False),          # +inf above a finite bound
        (inf, [inf, 0.0], True),           # +inf <= +inf
        (inf, [1e30, 3e38], True),         # a finite sum below +inf
        (-inf, [-1e30, -3e38], False),     # a finite sum above -inf
        (inf, [nan, 0.0], False),
        (-0.5, [-0.5, -0.5], True),        # a negative bound met exactly
        (-0.5, [-0.5, np.nextafter(np.float32(-0.5), np.float32(0))], False),
    ]
    for c, row, want in cases:
        with np.errstate(invalid="ignore"):
            s = float(np.sum(np.asarray(row, dtype=np.float64)))
        assert (s <= c * len(row)) == want, (c, row)      # the IEEE evaluation agrees
        assert _confident(c, row) == want, (c, row)


def test_stable_confident_stopping_large_bound_is_exact():
    """A bound c L of 2^141 to 2^160 still compares exactly: 16384 entropies
    of 3.4e38 sum to ~5.6e42 (2^142.0), above c L = 1.5e38 x 16384 (2^141.2)
    and below 4e38 x 16384; float64 holds both sides well apart."""
    row = np.full(16384, 3.4e38, dtype=np.float32)
    total = float(np.sum(row.astype(np.float64)))
    assert total > 1.5e38 * 16384 and total < 4e38 * 16384
    assert _confident(1.5e38, row) is False
    assert _confident(4e38, row) is True
    assert _confident(float(np.float32(3.4e38)), row) is True      # the mean exactly at c


def test_uniform_loop_converges_to_the_models_canvas_and_freezes_rows():
    B, L, V, N = 3, 12, 50, 16
    target = np.random.default_rng(4).integers(0, V, size=(B, L))

    def model(canvas, step):
        # sharper and sharper around a fixed target; row 2 stays unsure
        x = np.zeros((B, L, V), dtype=np.float32)
        for b in range(B):
            for l in range(L):
                x[b, l, target[b, l]] = 3.0 + 2.0 * step if b < 2 else 0.5
        return x

    argmax, steps = oracle.decode_uniform(model, B, L, V, seed=9, num_steps=N,
                                          entropy_bound=0.5, stability_threshold=1,
                                          confidence_threshold=0.005)
    assert np.array_equal(argmax[:2], target[:2])
    assert steps == N                                    # row 2 never gets confident
    assert np.array_equal(argmax[2], target[2])          # but its argmax is the target


def test_uniform_loop_stops_early_when_every_row_is_confident():
    B, L, V = 2, 8, 30
    target = np.arange(B * L).reshape(B, L) % V

    def model(canvas, step):
        x = np.zeros((B, L, V), dtype=np.float32)
        for b in range(B):
            for l in range(L):
                x[b, l, target[b, l]] = 40.0
        return x

    argmax, steps = oracle.decode_uniform(model, B, L, V, seed=1, num_steps=48,
                                          stability_threshold=1, confidence_threshold=0.005)
    assert steps == 2 and np.array_equal(argmax, target)


def test_uniform_loop_freezes_finished_rows():
    """A row that has stopped keeps its canvas while the others go on: the
    canvas the model sees for it no longer changes, even once the model turns
    unsure about it."""
    B, L, V, N = 2, 10, 40, 12
    target = np.random.default_rng(6).integers(0, V, size=(B, L))
    seen = []

    def model(canvas, step):
        seen.append(canvas.copy())
        x = np.zeros((B, L, V), dtype=np.float32)
        for l in range(L):
            if step <= 3:
                x[0, l, target[0, l]] = 40.0      # row 0: sure, then flat after step 3
            x[1, l, target[1, l]] = 1.0           # row 1: never confident
        return x

    argmax, steps = oracle.decode_uniform(model, B, L, V, seed=2, num_steps=N,
                                          stability_threshold=1, confidence_threshold=0.005)
    assert steps == N
    assert np.array_equal(argmax[0], target[0])
    frozen = seen[3][0]
    for c in seen[3:]:
        assert np.array_equal(c[0], frozen)       # row 0 stopped at step 2
    assert any(not np.array_equal(seen[i][1], seen[i + 1][1]) for i in range(3, N - 1))
