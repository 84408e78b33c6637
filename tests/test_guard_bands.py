"""The guard-band checker used by the GPU tests (kivi_testlib.Guard), exercised on host
memory: writes inside a buffer pass, a write one element before or past it is reported, and
freed buffers drop out."""
import pytest
import torch

from kivi_testlib import Guard


def test_writes_inside_pass():
    g = Guard()
    a = g.zeros((3, 5), torch.float16, "cpu")
    b = g.empty(7, torch.float32, "cpu")
    assert a.is_contiguous() and a.data_ptr() - a.untyped_storage().data_ptr() == Guard.MARGIN
    assert (a == 0).all()
    a.fill_(1.0)
    b.fill_(-2.0)
    g.check("fill")


@pytest.mark.parametrize("side", ["before", "after"])
def test_overrun_is_reported(side):
    g = Guard()
    a = g.zeros((4, 8), torch.int16, "cpu")
    raw = torch.empty(0, dtype=torch.int16).set_(a.untyped_storage())
    first = Guard.MARGIN // 2
    raw[first - 1 if side == "before" else first + a.numel()] = 7
    with pytest.raises(AssertionError, match="before" if side == "before" else "past the end"):
        g.check("planted")


def test_freed_buffers_drop_out():
    g = Guard()
    a = g.zeros(16, torch.uint8, "cpu")
    del a
    g.check("free")
    assert g.items == []
