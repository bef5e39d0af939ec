"""Oracle for the dLLM commit step -- TEST INFRASTRUCTURE, not part of the product.

A plain, slow CPU implementation (numpy float64, Python loops, exact rational
arithmetic where a rule compares a sum) of what the commit step computes:
per-position token statistics over (B, L, V) logits and the commit rules that
decide which masked positions take their proposed token.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never calls it and shares
no code, table or constant generator with it; the only thing both sides share is
the seeded input generator in ``workloads/``, which holds none of the method's
arithmetic.

Sources (the pages this follows):
  * mlx-arsenal research note "dLLM block decoding": the function table in
    "What mlx-arsenal ships", the loops in "Reference loop" / "Token editing
    (LLaDA2.1)" / "Uniform-noise decoding (DiffusionGemma)", and the list in
    "Deviations from the references".
  * mojo-dllm book: "The loop LLaDA uses" and the "Row statistics on the device"
    paragraph of "The GPU path".
  * mlxcel manual "Block Diffusion": "LLaDA-2 Block Unmasking" and "Samplers and
    Reveal Policies".

Every function is pinned by tests/test_oracle_pins.py against closed forms,
invariants, brute force on tiny inputs and printed values (tests/golden/).
"""
from .philox import philox4x32_10, philox_words, uniform_from_word, gumbel_noise
from .stats import token_stats, token_stats_row, widen_logits, Stats
from .rules import (threshold_transfer, topk_transfer, factor_transfer,
                    entropy_bound_transfer, edit_transfer, transfer_schedule,
                    block_ranges, block_causal_mask, decaying_threshold)
from .step import commit_step, apply_step, counts, rank_rule, StepResult
from .uniform import (linear_temperature, uniform_canvas, renoise, StableConfidentStopping,
                      decode_uniform)

__all__ = [
    "philox4x32_10", "philox_words", "uniform_from_word", "gumbel_noise",
    "token_stats", "token_stats_row", "widen_logits", "Stats",
    "threshold_transfer", "topk_transfer", "factor_transfer",
    "entropy_bound_transfer", "edit_transfer", "transfer_schedule",
    "block_ranges", "block_causal_mask", "decaying_threshold",
    "commit_step", "apply_step", "counts", "rank_rule", "StepResult",
    "linear_temperature", "uniform_canvas", "renoise", "StableConfidentStopping",
    "decode_uniform",
]
