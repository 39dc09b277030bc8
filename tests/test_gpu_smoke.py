"""The build's smoke entry point (one small routed-expert MoE forward on
cuda:0 checked against the oracle end to end), run as part of the GPU suite
so that a break in it shows up with the other parity tests."""
import pytest

import __graft_entry__

pytestmark = pytest.mark.gpu


def test_smoke_entry_point():
    __graft_entry__.smoke()
