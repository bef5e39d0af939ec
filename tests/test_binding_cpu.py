"""Host logic of the Python binding that runs without a GPU: the default
workspace is one buffer per (device, stream), grown on demand and never
created or grown during graph capture."""
import pytest
import torch

import commit_step_amd as cs


@pytest.fixture(autouse=True)
def fresh_workspaces():
    saved = dict(cs._workspaces)
    cs._workspaces.clear()
    yield
    cs._workspaces.clear()
    cs._workspaces.update(saved)


CPU = torch.device("cpu")


def test_workspace_is_kept_per_stream():
    a = cs._workspace(CPU, 11, 1000)
    assert a.numel() >= 1000 and a.dtype == torch.uint8 and int(a.count_nonzero()) == 0
    assert cs._workspace(CPU, 11, 1000) is a           # same stream: same buffer
    assert cs._workspace(CPU, 11, 10) is a             # smaller request: same buffer
    b = cs._workspace(CPU, 12, 1000)                   # another stream: its own buffer
    assert b is not a and b.data_ptr() != a.data_ptr()
    assert cs._workspace(CPU, 11, 1000) is a and cs._workspace(CPU, 12, 1000) is b


def test_workspace_key_includes_the_device():
    a = cs._workspace(torch.device("cpu", 0), 5, 64)
    b = cs._workspace(torch.device("cpu", 1), 5, 64)
    assert a is not b


def test_workspace_grows_zero_filled():
    a = cs._workspace(CPU, 3, 300)
    a.fill_(7)                                         # a stale buffer is not reused
    g = cs._workspace(CPU, 3, 5000)
    assert g is not a and g.numel() >= 5000 and int(g.count_nonzero()) == 0
    assert cs._workspace(CPU, 3, 300) is g


def test_workspace_minimum_size():
    assert cs._workspace(CPU, 4, 0).numel() == 256


def test_workspace_refuses_creation_or_growth_during_capture(monkeypatch):
    a = cs._workspace(CPU, 9, 4096)
    monkeypatch.setattr(cs, "_capturing", lambda device: True)
    assert cs._workspace(CPU, 9, 4096) is a            # large enough: reused under capture
    with pytest.raises(RuntimeError, match="graph capture"):
        cs._workspace(CPU, 9, 8192)                    # growth under capture
    with pytest.raises(RuntimeError, match="graph capture"):
        cs._workspace(CPU, 10, 16)                     # a new stream under capture
