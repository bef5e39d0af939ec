"""Oracle: uniform-noise decoding helpers (test infrastructure).

Source: mlx-arsenal research note "dLLM block decoding": the function table row
of linear_temperature / uniform_canvas / renoise / StableConfidentStopping
(temperature schedule, random canvas, re-noising, stable-and-confident stop),
and the loop of "Uniform-noise decoding (DiffusionGemma)": a canvas starts as
uniformly random tokens; each step scales the logits by a temperature that
decays linearly with the remaining steps, measures entropy on the scaled
logits, draws a categorical sample, accepts the lowest-entropy predictions
under an entropy budget over all positions, re-noises every other position,
freezes rows that have stopped, and stops a row once its argmax canvas is
stable and confident.  mlxcel "Block Diffusion", "DiffusionGemma Canvas
Denoising": stop when the canvas is stable and confident for the configured
stability window.

Readings taken where the pages give only names and defaults:
  * linear_temperature(r, N, t_min, t_max) = t_min + (t_max - t_min) * r / N,
    so the first step (r = N) runs at t_max and the temperature falls
    linearly towards t_min;
  * uniform_canvas: each token uniform on [0, V), from Philox4x32-10 (the
    sampling generator) at counter (l, b, 0xFFFFFFFF, draw) under the same
    key; with x = w0 + 2^32 w1 the token is floor(x * V / 2^64);
  * renoise(sample, accepted, noise) = where(accepted, sample, noise);
  * the categorical sample of softmax(z), z = logits / T, is the Gumbel-max
    draw of token_stats at temperature T (same Philox noise);
  * StableConfidentStopping(k, c): a row counts the consecutive steps whose
    argmax canvas equals the previous step's; it stops when that count
    reaches k and its mean entropy is at most c (exact rational comparison);
    a row holding a non-finite entropy is not confident.
"""
from fractions import Fraction

import numpy as np

from .philox import philox4x32_10
from .rules import entropy_bound_transfer
from .stats import token_stats

CANVAS_STREAM = 0xFFFFFFFF


def linear_temperature(remaining, num_steps, t_min, t_max):
    """t_min + (t_max - t_min) * remaining / num_steps (float64)."""
    if num_steps < 1 or not 0 <= remaining <= num_steps:
        raise ValueError("need 0 <= remaining <= num_steps, num_steps >= 1")
    return t_min + (t_max - t_min) * remaining / num_steps


def uniform_canvas(B, L, V, seed, draw):
    """(B, L) int32 tokens uniform on [0, V); draw selects an independent canvas."""
    if not 1 <= V <= 0x7FFFFFFF:
        raise ValueError("V must be in [1, 2^31)")
    seed = int(seed)
    key = (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    out = np.zeros((B, L), dtype=np.int32)
    for b in range(B):
        for l in range(L):
            w = philox4x32_10((l, b, CANVAS_STREAM, int(draw)), key)
            x = int(w[0]) | (int(w[1]) << 32)
            out[b, l] = (x * int(V)) >> 64
    return out


def renoise(sample, accepted, noise):
    """where(accepted, sample, noise)."""
    sample, noise = np.asarray(sample), np.asarray(noise)
    accepted = np.asarray(accepted, dtype=bool)
    out = noise.copy()
    for idx in zip(*np.nonzero(accepted)):
        out[idx] = sample[idx]
    return out


class StableConfidentStopping:
    """Per-row stop: k consecutive unchanged argmax canvases and mean entropy <= c."""

    def __init__(self, stability_threshold, confidence_threshold):
        self.k = int(stability_threshold)
        self.c = float(confidence_threshold)
        self.prev = None
        self.count = None

    def __call__(self, argmax, entropy):
        argmax = np.asarray(argmax)
        B, L = argmax.shape
        if self.count is None:
            self.count = np.zeros(B, dtype=np.int64)
        done = np.zeros(B, dtype=bool)
        for b in range(B):
            same = self.prev is not None and bool(np.array_equal(argmax[b], self.prev[b]))
            self.count[b] = self.count[b] + 1 if same else 0
            hs = np.asarray(entropy, dtype=np.float32)[b]
            done[b] = self.count[b] >= self.k and self._confident(hs)
        self.prev = argmax.copy()
        return done

    def _confident(self, hs):
        """mean(hs) <= c, i.e. sum(hs) <= c L, in the extended reals: the sum
        is undefined (never confident) with a NaN or with both infinities, +inf
        with a +inf term, -inf with a -inf term, else the exact rational sum.
        An empty row sums to 0 and compares with 0 (its c L)."""
        L = len(hs)
        c = self.c
        if L == 0:
            return True
        nan, pinf, ninf = bool(np.isnan(hs).any()), bool((hs == np.inf).any()), \
            bool((hs == -np.inf).any())
        if nan or (pinf and ninf):
            return False
        if pinf:
            return c == np.inf                     # +inf <= c L only for c L = +inf
        if ninf:
            return True                            # -inf <= every c L
        if np.isinf(c):
            return c > 0                           # a finite sum against +-inf
        total = sum((Fraction(float(h)) for h in hs), Fraction(0))
        return total <= Fraction(c) * L


def decode_uniform(model, B, L, V, seed, num_steps=48, entropy_bound=0.1, t_min=0.4, t_max=0.8,
                   stability_threshold=1, confidence_threshold=0.005, stats_fn=None):
    """The DiffusionGemma loop.  model(canvas, step) -> (B, L, V) float32 logits.
    stats_fn(logits, T, step) -> (argmax, sample, entropy float32) may replace
    the oracle's own statistics (a test passes the GPU's, so both sides take
    the same decisions).  Returns (argmax, steps)."""
    canvas = uniform_canvas(B, L, V, seed, 0)
    stop = StableConfidentStopping(stability_threshold, confidence_threshold)
    everywhere = np.ones((B, L), dtype=bool)
    done = np.zeros(B, dtype=bool)
    argmax = canvas
    steps = 0
    for remaining in range(num_steps, 0, -1):
        steps += 1
        T = float(np.float32(linear_temperature(remaining, num_steps, t_min, t_max)))
        logits = model(canvas, steps)
        if stats_fn is None:
            greedy = token_stats(logits, "f32", stats_temperature=T)
            sampled = token_stats(logits, "f32", temperature=T, seed=seed, step=steps)
            am, sample, ent = greedy.x0, sampled.x0, greedy.entropy.astype(np.float32)
        else:
            am, sample, ent = stats_fn(logits, T, steps)
        accepted = entropy_bound_transfer(ent, everywhere, entropy_bound)
        new_canvas = renoise(sample, accepted, uniform_canvas(B, L, V, seed, steps))
        argmax = np.where(done[:, None], argmax, am)
        canvas = np.where(done[:, None], canvas, new_canvas)
        done = done | stop(argmax, ent)
        if done.all():
            break
    return argmax, steps
