"""The planted sampling ties of tests/golden/sampled_ties.json, checked with the
oracle: each pair of ids draws noise words equal in the 23 bits the uniform
takes, and with equal top logits the oracle picks the lower id."""
import json
from pathlib import Path

import numpy as np
import pytest

import oracle
from oracle.philox import philox_words

TIES = json.loads((Path(__file__).parent / "golden" / "sampled_ties.json").read_text())


@pytest.mark.parametrize("case", TIES["cases"], ids=lambda c: f"{c['dtype']}-{c['v1']}-{c['v2']}")
def test_planted_tie(case):
    V, v1, v2, step = case["V"], case["v1"], case["v2"], case["step"]
    w = philox_words(TIES["seed"], step, 0, 0, V) >> np.uint64(9)
    assert v1 < v2 and w[v1] == w[v2]
    g = oracle.gumbel_noise(TIES["seed"], step, 0, 0, V)
    assert g[v1] == g[v2]
    x = np.full((1, 1, V), -60.0, np.float32)
    x[0, 0, [v1, v2]] = 0.0
    ref = oracle.token_stats(x, "f32", temperature=0.8, seed=TIES["seed"], step=step)
    assert int(ref.x0[0, 0]) == v1
