"""Plant plausible mistakes in a copy of the oracle and check the pins catch them.

Each case copies ``oracle/`` into a temporary directory, applies one textual
mutation (a dropped term, a wrong sign, a wrong index or comparison), and runs
the pin tests that should notice it against the mutated copy, in a child
process.  The mutation passes only if that run fails.  CPU only; the real
oracle is never modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PIN_FILES = ["test_oracle_pins.py", "test_oracle_step.py", "test_oracle_uniform.py"]

MUTATIONS = [
    # (file, original text, mutated text, -k selection of pin tests)
    ("stats.py", "((ls[keep] - m) - log_z)", "(ls[keep] - m)",
     "moment or two_level or uniform"),
    ("stats.py", "log_z = np.log1p(z_minus)", "log_z = np.log(z)", "peaked"),
    ("stats.py", "H = -np.sum(", "H = np.sum(", "two_level or moment"),
    ("stats.py", "vals == best)[0]", "vals == best)[-1]", "two_level or uniform"),
    ("stats.py", "s = lp / temperature + g", "s = lp * temperature + g",
     "frequencies"),
    ("stats.py", "support = allowed & (ell == np.inf)", "support = allowed",
     "degenerate"),
    ("stats.py", "np.where(np.isnan(ell), -np.inf, ell)", "np.where(np.isnan(ell), 0.0, ell)",
     "nan"),
    ("philox.py", "c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1,",
     "c0, c1, c2, c3 = (hi1 ^ c3 ^ np.uint64(k0), lo1,", "known_answer"),
    ("philox.py", "k1 = (k1 + PHILOX_W1) & 0xFFFFFFFF", "k1 = k1", "known_answer"),
    ("philox.py", "+ 0.5) * 2.0 ** -23", ") * 2.0 ** -23", "uniform_mapping"),
    ("rules.py", "prefix.add(_ent(ent[b, l]))\n",
     "prefix.add(_ent(ent[b, l]))\n            if not prefix.at_most(gamma):\n"
     "                n = i\n                break\n", "entropy_bound"),
    ("rules.py", "out[b, order[:max(n, 1)]] = True\n    return out\n\n\nclass",
     "out[b, order[:n if n < len(order) - 1 else len(order)]] = True\n    return out\n\n\nclass",
     "factor"),
    ("rules.py", "(_conf(conf[b, l]) > tau if strict else _conf(conf[b, l]) >= tau)",
     "(_conf(conf[b, l]) >= tau)", "strict"),
    ("rules.py", "key=lambda l: (-_conf(conf_row[l]), l))",
     "key=lambda l: (-_conf(conf_row[l]), -l))", "topk"),
    ("rules.py", "nb // steps + (1 if s < nb % steps else 0)",
     "nb // steps + (1 if s >= steps - nb % steps else 0)", "schedule"),
    ("rules.py", "np.where(key_block <= q // bl, 0.0, -np.inf)",
     "np.where(key_block < q // bl, 0.0, -np.inf)", "causal_mask"),
    ("rules.py", "start = (P // bl) * bl if align else P", "start = P", "block_ranges"),
    ("rules.py", "and _conf(prob[b, l]) > tau_edit", "and _conf(prob[b, l]) >= tau_edit",
     "edit"),
    ("stats.py", "others[top] = False", "others[top] = allowed[top]", "margin"),
    ("stats.py", "margin = -np.expm1(r - m) / z", "margin = (1.0 - np.exp(r - m)) / z", "margin"),
    ("stats.py", "(1.0 if n == 1 else 0.0)", "0.0", "margin"),
    ("stats.py", "ls = lp / stats_temperature", "ls = lp", "stats_temperature"),
    ("uniform.py", "return t_min + (t_max - t_min) * remaining / num_steps",
     "return t_max + (t_min - t_max) * remaining / num_steps", "linear_temperature"),
    ("uniform.py", "out[b, l] = (x * int(V)) >> 64", "out[b, l] = x % int(V)", "uniform_canvas"),
    ("uniform.py", "self.count[b] = self.count[b] + 1 if same else 0",
     "self.count[b] = self.count[b] + 1", "stopping"),
    ("uniform.py", "return total <= Fraction(c) * L", "return total <= Fraction(c)", "stopping"),
    ("uniform.py", "return True                            # -inf <= every c L",
     "return False                           # -inf <= every c L", "extended_reals"),
    ("uniform.py", "if nan or (pinf and ninf):", "if nan:", "extended_reals"),
    ("uniform.py", "canvas = np.where(done[:, None], canvas, new_canvas)", "canvas = new_canvas",
     "freezes_finished"),
    ("step.py", "take = (commit is not None and commit[b, l]) or (edit is not None and edit[b, l])",
     "take = commit is not None and commit[b, l]", "hand_worked"),
    ("step.py", "if cand[b, l] and not commit[b, l])", "if cand[b, l])", "hand_worked or block_loop"),
    ("step.py", "c[b, 1] = sum(1 for l in range(edit.shape[1]) if edit[b, l])",
     "c[b, 1] = 0", "hand_worked or editing_loop"),
    ("step.py", "em = edit_transfer(st.x0, prob32, tokens, editable, tau_edit)",
     "em = edit_transfer(st.x0, prob32, tokens, editable | cand, tau_edit)", "editing_loop"),
    ("rules.py", "float(tau_initial) - float(decay) * int(step))",
     "float(tau_initial) - float(decay) * (int(step) + 1))", "decaying"),
    ("rules.py", "return max(float(tau_floor),", "return min(float(tau_floor),", "decaying"),
    ("rules.py", "        tau = float(taus[b])\n", "        tau = float(taus[0])\n", "per_row"),
]


@pytest.mark.parametrize("case", range(len(MUTATIONS)))
def test_planted_mistake_is_caught(case, tmp_path):
    fname, old, new, select = MUTATIONS[case]
    dst = tmp_path / "oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), dst,
                    ignore=shutil.ignore_patterns("__pycache__"))
    src = (dst / fname).read_text()
    assert old in src, f"mutation {case} no longer applies to {fname}"
    (dst / fname).write_text(src.replace(old, new, 1))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "golden")
    for pins in PIN_FILES:
        shutil.copy(os.path.join(ROOT, "tests", pins), tmp_path)
    env = dict(os.environ, PYTHONPATH=str(tmp_path), PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-k", select] + [str(tmp_path / pins) for pins in PIN_FILES],
                       cwd=tmp_path, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 1, (f"mutation {case} ({fname}) was not caught:\n"
                               + r.stdout[-2000:] + r.stderr[-2000:])
