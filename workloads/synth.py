"""Seeded synthetic workloads shaped like the pages' decoding settings.

The pages measure this step on no dataset; every input here is synthetic.
Shapes follow the models the pages discuss: LLaDA-8B (vocabulary 126,464, mask
id 126,336; mojo-dllm "Development plan", model facts), a Dream-like canvas
(vocabulary 151,936), DiffusionGemma (canvas 256; mlxcel "Block Diffusion"
CLI reference) and LLaDA-2 block decoding (block 32).

Conventions (fixed once, so every consumer sees the same bits):
  * numpy PCG64 generators; workload n uses seed 1000 + n, except per-step or
    per-batch-row draws, which use [1000 + n, index];
  * draw order: logits -> peak positions -> peak tokens / strengths ->
    candidate / committed sets -> tokens;
  * "x % of positions" is exactly round(x * L) positions per batch row, chosen
    with a permutation;
  * N(0, s) means standard deviation s; normals are drawn in float32;
  * peak tokens are uniform over the ids that are not suppressed;
  * bf16 logits are made from the float32 values by round-to-nearest-even and
    are returned as uint16 bit patterns.
"""
from dataclasses import dataclass, field

import numpy as np


def bf16_bits(x):
    """float32 array -> uint16 bfloat16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def _draw_allowed(rng, V, suppressed, size):
    """Uniform draws from [0, V) minus the (sorted, unique) suppressed ids."""
    r = rng.integers(0, V - len(suppressed), size=size)
    for s in sorted(suppressed):
        r = np.where(r >= s, r + 1, r)
    return r


@dataclass
class Workload:
    """One batch of inputs and the parameters the workload runs the rules with."""
    name: str
    logits: np.ndarray            # (B, L, V): float32, or uint16 bf16 bits
    dtype: str                    # "f32" | "bf16"
    suppress_ids: tuple = ()
    temperature: float = 0.0
    seed: int = 0
    step: int = 0
    cand: np.ndarray = None       # (B, L) bool candidates of the ranking rule
    editable: np.ndarray = None   # (B, L) bool positions the edit rule may revise
    tokens: np.ndarray = None     # (B, L) int32 current canvas
    params: dict = field(default_factory=dict)

    @property
    def shape(self):
        return self.logits.shape


def random_logits(seed, B, L, V, dtype="bf16", sigma=2.0, peak_frac=0.0,
                  peak_lo=0.0, peak_hi=0.0, suppress_ids=()):
    """N(0, sigma) logits with one raised token on round(peak_frac * L) positions
    of every batch row (strength uniform in [peak_lo, peak_hi])."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, L, V), dtype=np.float32) * np.float32(sigma)
    npk = int(round(peak_frac * L))
    if npk:
        pos = np.stack([rng.permutation(L)[:npk] for _ in range(B)])
        tok = _draw_allowed(rng, V, tuple(suppress_ids), (B, npk))
        strength = rng.uniform(peak_lo, peak_hi, size=(B, npk)).astype(np.float32)
        for b in range(B):
            x[b, pos[b], tok[b]] += strength[b]
    return (bf16_bits(x) if dtype == "bf16" else x), rng


# Parameters of the five workloads (numbers only; the generators below draw them).
CONFIG_PARAMS = {
    1: dict(name="tiny", B=1, L=64, V=4096, dtype="f32", sigma=2.0,
            rule="threshold", tau=0.9, strict=False),
    2: dict(name="llada_block", B=1, L=32, V=126464, dtype="bf16", sigma=3.0,
            rule="topk", steps=32, mask_id=126336),
    3: dict(name="dream_canvas", B=4, L=256, V=151936, dtype="bf16", sigma=2.5,
            rule="factor", f=1.0, temperature=0.7, seed=1003, steps=4),
    4: dict(name="diffusiongemma_canvas", B=1, L=256, V=262144, dtype="bf16",
            sigma=2.0, rule="entropy_bound+edit", gamma=0.5, tau_edit=0.9),
    5: dict(name="batched", B=32, L=512, V=126464, dtype="bf16", sigma=3.0,
            rule="threshold", tau=0.95, strict=True, prompt_len=77, gen_len=435,
            block_len=32, mask_L=2048),
}


def config1():
    """Tiny: (1, 64, 4096) fp32 ~ N(0, 2); +12 on one token at 30 % of positions;
    mask id V-1 suppressed; half the positions are candidates; threshold 0.9."""
    p = CONFIG_PARAMS[1]
    B, L, V = p["B"], p["L"], p["V"]
    sup = (V - 1,)
    x, rng = random_logits(1001, B, L, V, "f32", p["sigma"], 0.3, 12.0, 12.0, sup)
    cand = np.zeros((B, L), dtype=bool)
    for b in range(B):
        cand[b, rng.permutation(L)[:L // 2]] = True
    return Workload("cfg1_tiny", x, "f32", suppress_ids=sup, cand=cand,
                    params=dict(tau=p["tau"], strict=p["strict"]))


def config2_step(step):
    """LLaDA-like block step: (1, 32, 126464) bf16 ~ N(0, 3) with a +U(8, 16)
    peak at 40 % of positions, regenerated from [1002, step]; the LLaDA mask id
    is suppressed.  Candidates come from the caller's trajectory (all 32 are
    masked at step 0)."""
    p = CONFIG_PARAMS[2]
    B, L, V = p["B"], p["L"], p["V"]
    sup = (p["mask_id"],)
    x, _ = random_logits([1002, int(step)], B, L, V, "bf16", p["sigma"], 0.4,
                         8.0, 16.0, sup)
    return Workload(f"cfg2_llada_step{step}", x, "bf16", suppress_ids=sup,
                    step=int(step), params=dict(steps=p["steps"]))


def config3():
    """Dream-like canvas: (4, 256, 151936) bf16 ~ N(0, 2.5) with a +U(6, 14)
    peak at 35 % of positions; mask id V-1 suppressed; Gumbel-max at T = 0.7
    with seed 1003; 60 % of positions are candidates; factor f = 1.0."""
    p = CONFIG_PARAMS[3]
    B, L, V = p["B"], p["L"], p["V"]
    sup = (V - 1,)
    x, rng = random_logits(1003, B, L, V, "bf16", p["sigma"], 0.35, 6.0, 14.0, sup)
    cand = np.zeros((B, L), dtype=bool)
    for b in range(B):
        cand[b, rng.permutation(L)[:int(round(0.6 * L))]] = True
    return Workload("cfg3_dream", x, "bf16", suppress_ids=sup,
                    temperature=p["temperature"], seed=p["seed"], cand=cand,
                    params=dict(f=p["f"], steps=p["steps"]))


def config4():
    """DiffusionGemma-like canvas: (1, 256, 262144) bf16 ~ N(0, 2).  Every
    position gets a peak mix: strength s ~ U(8, 24), k ~ U{1..8} distinct tokens,
    weights w ~ Dirichlet(0.3), and s + max(ln w_j, -30) is added to token j.
    40 % of positions are committed (editable); their tokens are, for a seeded
    half, the planted token of largest weight and otherwise uniform.  The other
    60 % are the candidates.  entropy_bound gamma = 0.5, edit tau = 0.9."""
    p = CONFIG_PARAMS[4]
    B, L, V = p["B"], p["L"], p["V"]
    rng = np.random.default_rng(1004)
    x = rng.standard_normal((B, L, V), dtype=np.float32) * np.float32(p["sigma"])
    strength = rng.uniform(8.0, 24.0, size=(B, L))
    kmix = rng.integers(1, 9, size=(B, L))
    top_token = np.zeros((B, L), dtype=np.int64)
    for b in range(B):
        for l in range(L):
            toks = rng.integers(0, V, size=int(kmix[b, l]))
            while np.unique(toks).size != toks.size:       # distinct tokens: redraw
                toks = rng.integers(0, V, size=int(kmix[b, l]))
            w = rng.dirichlet(np.full(int(kmix[b, l]), 0.3))
            logw = np.maximum(np.log(np.maximum(w, 1e-300)), -30.0)
            x[b, l, toks] += (strength[b, l] + logw).astype(np.float32)
            top_token[b, l] = toks[int(np.argmax(w))]
    n_comm = int(round(0.4 * L))
    editable = np.zeros((B, L), dtype=bool)
    tokens = np.zeros((B, L), dtype=np.int32)
    for b in range(B):
        committed = rng.permutation(L)[:n_comm]
        editable[b, committed] = True
        planted = rng.permutation(committed)[:n_comm // 2]
        tokens[b] = rng.integers(0, V, size=L)
        tokens[b, planted] = top_token[b, planted]
    cand = ~editable
    return Workload("cfg4_diffusiongemma", bf16_bits(x), "bf16", cand=cand,
                    editable=editable, tokens=tokens,
                    params=dict(gamma=p["gamma"], tau_edit=p["tau_edit"]))


def config5_batch_row(b):
    """One batch row of the batched workload: (1, 512, 126464) bf16 ~ N(0, 3)
    with +10 on one token at 50 % of positions, drawn from [1005, b]; every
    position is a candidate; threshold 0.95 strict."""
    p = CONFIG_PARAMS[5]
    L, V = p["L"], p["V"]
    x, _ = random_logits([1005, int(b)], 1, L, V, "bf16", p["sigma"], 0.5,
                         10.0, 10.0)
    return Workload(f"cfg5_batched_row{b}", x, "bf16",
                    cand=np.ones((1, L), dtype=bool),
                    params=dict(tau=p["tau"], strict=p["strict"]))
