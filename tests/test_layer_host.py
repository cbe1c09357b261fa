"""Host-side ownership rules of MoeLayer's workspace (no GPU): it grows only
when a call needs more, it is reused otherwise, and a buffer that a graph
capture used is kept alive when a later call grows a new one."""
import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "mixture_experts_layer_13_amd", "libmoe.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmoe.so not built")


def test_workspace_grows_and_is_reused():
    from mixture_experts_layer_13_amd.layer import Workspace
    ws = Workspace("cpu")
    a = ws.get(1000)
    assert a.numel() >= 1000 and a.dtype == torch.uint8
    assert ws.get(500) is a and ws.get(1000) is a
    b = ws.get(5000)
    assert b is not a and b.numel() >= 5000
    assert ws.retained == []          # nothing captured: the old buffer may be freed
    assert ws.get(16).numel() >= 256  # never below the minimum size


def test_captured_workspace_outlives_growth():
    from mixture_experts_layer_13_amd.layer import Workspace
    ws = Workspace("cpu")
    a = ws.get(1000, capturing=True)
    assert ws.captured
    assert ws.get(800) is a and ws.captured          # eager reuse keeps the captured mark
    b = ws.get(10_000)
    assert b is not a and ws.retained == [a]         # a graph may still hold a's address
    assert not ws.captured
    c = ws.get(20_000)
    assert ws.retained == [a] and c is not b         # b was never captured: not retained
    d = ws.get(30_000, capturing=True)
    e = ws.get(40_000)
    assert ws.retained == [a, d] and e is not d
