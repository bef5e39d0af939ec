"""Seeded synthetic inputs for the commit step (shared by tests, smoke and bench).

This package only draws inputs: logits, masks, tokens and the parameters of each
workload.  It holds none of the commit step's arithmetic, and it imports
neither the oracle nor the HIP library.
"""
from .synth import (Workload, bf16_bits, random_logits, config1, config2_step,
                    config3, config4, config5_batch_row, CONFIG_PARAMS)

__all__ = ["Workload", "bf16_bits", "random_logits", "config1", "config2_step",
           "config3", "config4", "config5_batch_row", "CONFIG_PARAMS"]
