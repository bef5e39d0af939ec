"""The stage-timing tool's host logic, on synthetic records: times from the
first workgroup's start, the gap to an earlier launch's newer records, the
stream statistics and the chain of the workgroup that completes the batch row."""
import numpy as np
import pytest

st = pytest.importorskip("commit_step_amd.stage_timing")


def _records():
    ts = np.zeros((3, len(st.STAGES)), dtype=np.int64)
    S = {n: i for i, n in enumerate(st.STAGES)}
    ts[0, [S["start"], S["stream_end"], S["published"], S["batch_counted"]]] = [1000, 1500, 1600, 1700]
    ts[1, [S["start"], S["stream_end"], S["finalized"], S["published"], S["stores_drained"],
           S["batch_counted"], S["rule_loaded"], S["rule_ranked"], S["batch_done"]]] = \
        [1010, 1800, 1830, 1850, 1860, 1900, 1950, 2050, 2100]
    ts[2, [S["start"], S["stream_end"]]] = [990, 1400]
    ts[2, S["rule_loaded"]] = 900          # left over from an earlier launch
    return ts


def test_metrics_of_synthetic_records():
    m = st.metrics(_records())
    tick_us = st.TICK_NS * 1e-3
    assert m["workgroups"] == 3
    assert m["last_start"] == pytest.approx(20 * tick_us)
    assert m["gap_from_previous_launch"] == pytest.approx(90 * tick_us)
    assert m["stream_median_wg"] == pytest.approx(500 * tick_us)
    assert m["stream_max_wg"] == pytest.approx(790 * tick_us)
    assert m["stream_end_last"] == pytest.approx(810 * tick_us)
    # the completing workgroup is the one with a batch-done record
    assert m["completer_batch_done"] == pytest.approx(1110 * tick_us)
    assert m["completer_rule_loaded"] == pytest.approx(960 * tick_us)
    assert m["completer_start"] == pytest.approx(20 * tick_us)
    # the stale record of the earlier launch is not this launch's rule_loaded
    assert m["rule_loaded_last"] == pytest.approx(960 * tick_us)
    chain = [m["completer_" + n] for n in st.CHAIN if "completer_" + n in m]
    assert chain == sorted(chain)
