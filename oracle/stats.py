"""Oracle: per-position token statistics (test infrastructure).

What is computed (mlx-arsenal "dLLM block decoding", "What mlx-arsenal ships",
token_stats row of the function table): for every position, the proposed token
x0, its probability and the entropy of the position's distribution, NaN-safe,
greedy or Gumbel-max sampling with an explicit key, with ``suppress_ids``.

Readings of the pages taken here:
  * suppressed ids are removed before the softmax, so prob and entropy are over
    the remaining vocabulary ("Deviations from the references", suppress_ids item);
  * prob and entropy are those of softmax(logits) as passed; temperature only
    changes how x0 is drawn (mojo-dllm "The loop LLaDA uses": noise goes on the
    logits before the argmax and the token keeps its softmax probability; the
    DiffusionGemma loop divides by the temperature before calling token_stats
    when it wants tempered entropy);
  * greedy x0 is the first index of the maximum (mojo-dllm "The GPU path", row
    statistics paragraph: a tie goes to the smaller index; "Deviations": the
    first maximal one);
  * sampled x0 is the first index of the maximum of logit / T + g, with g the
    Gumbel noise of oracle.philox (Gumbel-max trick);
  * margin is the topk_margin confidence of mojo-dllm "The GPU path" (row
    statistics paragraph: p minus the runner-up's probability, the runner-up
    being the largest logit at any index other than the argmax): p_(1) - p_(2)
    of softmax(logits) over the unsuppressed ids, whatever x0 is; a tie at the
    maximum gives 0, a single unsuppressed id gives 1;
  * with a statistics temperature Ts (the DiffusionGemma loop of "Uniform-noise
    decoding (DiffusionGemma)" measures entropy on the temperature-scaled
    logits z = logits / T), prob, entropy and margin are those of
    softmax(logits / Ts); x0 does not depend on Ts;
  * "NaN-safe": a NaN logit counts as -inf; a row whose unsuppressed logits are
    all -inf (or NaN) is uniform over the unsuppressed ids; a row with +inf
    logits is uniform over its +inf ids.  These are the limits of finite rows,
    and no output is ever NaN.

Everything is float64, row by row, from the exact input values (bf16 and fp32
widen to float64 without rounding).  Entropy is the textbook
H = -sum_v p_v log p_v (terms with p_v = 0 dropped), not a moment formula; its
log z is evaluated as log1p of the non-maximal mass so that it stays accurate
in float64 when that mass is tiny.
"""
from collections import namedtuple

import numpy as np

from .philox import gumbel_noise

Stats = namedtuple("Stats", ["x0", "prob", "entropy", "margin"])


def widen_logits(logits, dtype):
    """Exact float64 copy of the logits.

    dtype "f32": a float32 array.  dtype "bf16": a uint16 array of bfloat16 bit
    patterns (bf16 is the high half of a float32, so bits << 16 is exact).
    """
    a = np.asarray(logits)
    if dtype == "f32":
        if a.dtype != np.float32:
            raise TypeError("f32 logits must be a float32 array")
        return a.astype(np.float64)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 logits must be a uint16 array of bit patterns")
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError("dtype must be 'f32' or 'bf16'")


def _first_argmax(values, allowed):
    """Lowest index v with allowed[v] attaining the maximum of values over allowed."""
    idx = np.flatnonzero(allowed)
    vals = values[idx]
    best = vals.max()
    return int(idx[np.flatnonzero(vals == best)[0]])


def token_stats_row(ell, temperature, seed, step, b, l, suppressed, stats_temperature=1.0):
    """Statistics of one position.

    ell: float64 (V,) logits; temperature: the float32 value as float;
    suppressed: bool (V,) mask of suppressed ids (not all True);
    stats_temperature: Ts > 0 (a float32 value as float), prob / entropy /
    margin are those of softmax(ell / Ts).
    Returns (x0, prob, entropy, margin) as (int, float, float, float).
    """
    V = ell.shape[0]
    allowed = ~suppressed
    n_allowed = int(allowed.sum())
    if n_allowed == 0:
        raise ValueError("every id is suppressed")
    lp = np.where(np.isnan(ell), -np.inf, ell)          # NaN counts as -inf
    sampling = temperature > 0.0
    g = gumbel_noise(seed, step, b, l, V) if sampling else None

    ls = lp / stats_temperature                          # the logits the softmax sees
    m = ls[allowed].max()
    if np.isfinite(m):
        with np.errstate(invalid="ignore", over="ignore"):
            w = np.where(allowed, np.exp(ls - m), 0.0)   # exp(-inf) = 0
        # z = 1 + z_minus, z_minus = the mass of every entry but one maximal one;
        # log z = log1p(z_minus) keeps its accuracy when z_minus is below the
        # float64 resolution of 1 (a top logit some 40+ nats above the rest).
        top = _first_argmax(ls, allowed)
        z_minus = np.sum(np.delete(w, top))
        z = 1.0 + z_minus
        log_z = np.log1p(z_minus)
        p = w / z
        keep = allowed & (p > 0.0)
        H = -np.sum(p[keep] * ((ls[keep] - m) - log_z))
        # runner-up: the largest logit at any allowed index but the top one
        others = allowed.copy()
        others[top] = False
        r = ls[others].max() if others.any() else -np.inf
        margin = -np.expm1(r - m) / z                    # (1 - e^(r - m)) / z
        if sampling:
            with np.errstate(invalid="ignore"):
                s = lp / temperature + g
            x0 = _first_argmax(s, allowed)
        else:
            x0 = _first_argmax(lp, allowed)
        return x0, float(p[x0]), float(H), float(margin)

    # Degenerate rows: the limit of finite rows.
    if m == -np.inf:
        support = allowed                       # uniform over the unsuppressed ids
    else:
        support = allowed & (ell == np.inf)     # uniform over the +inf ids
    n = int(support.sum())
    x0 = _first_argmax(g, support) if sampling else int(np.flatnonzero(support)[0])
    return x0, 1.0 / n, float(np.log(n)), (1.0 if n == 1 else 0.0)


def token_stats(logits, dtype="f32", temperature=0.0, seed=None, step=0,
                suppress_ids=(), positions=None, stats_temperature=1.0):
    """Per-position (x0, prob, entropy, margin) of (B, L, V) logits.

    temperature: 0 = greedy; > 0 = Gumbel-max with key ``seed`` at ``step``
    (``seed`` is required then, as the pages require an explicit key).  The
    temperature is taken as the float32 value a C caller would pass.
    stats_temperature Ts > 0: prob, entropy and margin are those of
    softmax(logits / Ts), Ts taken as a float32 value too.
    positions: optional iterable of (b, l); then only those are computed and the
    other outputs are left at x0 = -1, prob = entropy = margin = NaN.
    """
    a = np.asarray(logits)
    if a.ndim != 3:
        raise ValueError("logits must be (B, L, V)")
    B, L, V = a.shape
    T = float(np.float32(temperature))
    if not (T >= 0.0):
        raise ValueError("temperature must be >= 0")
    if T > 0.0 and seed is None:
        raise ValueError("sampling needs an explicit seed")
    Ts = float(np.float32(stats_temperature))
    if not (Ts > 0.0 and np.isfinite(Ts)):
        raise ValueError("stats_temperature must be finite and > 0")
    suppressed = np.zeros(V, dtype=bool)
    for s in suppress_ids:
        if not 0 <= int(s) < V:
            raise ValueError("suppress id out of range")
        suppressed[int(s)] = True
    x0 = np.full((B, L), -1, dtype=np.int32)
    prob = np.full((B, L), np.nan)
    ent = np.full((B, L), np.nan)
    mar = np.full((B, L), np.nan)
    todo = positions if positions is not None else ((b, l) for b in range(B) for l in range(L))
    for b, l in todo:
        row = widen_logits(a[b, l], dtype)
        x0[b, l], prob[b, l], ent[b, l], mar[b, l] = token_stats_row(
            row, T, seed if seed is not None else 0, step, b, l, suppressed, Ts)
    return Stats(x0, prob, ent, mar)
