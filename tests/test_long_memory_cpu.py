"""The long-memory GPU cases carry state across chunks: checked on the CPU.

The GPU cases in test_long_memory_gpu.py are meant to fail if a chunk path
mishandles what one chunk hands to the next. That needs memory that
survives a chunk boundary at a size the bar can see. Here the oracle shows
it: restarting the recurrence from a zero state at the second chunk (or at
a later segment start) moves those outputs far past the bf16 bar, for both
gate recipes. With the usual prefill gates the same restart changes
nothing visible, which is why these cases were added.
"""
import numpy as np
import pytest

import oracle
from gated_deltanet_recurrence_amd import inputs
from parity import TOL_BF16, o_err


def _restart_gap(c, t0, t1, per_channel=False, skip=16):
    """Outputs of tokens t0 + skip .. t1 when the recurrence restarts from a
    zero state at t0, against the uninterrupted run: the part of what was
    carried into t0 that is still visible ``skip`` tokens later."""
    f = oracle.gdn_recurrent_channel if per_channel else oracle.gdn_recurrent
    o_ref, _ = f(c.q[:, :t1], c.k[:, :t1], c.v[:, :t1], c.g[:, :t1], c.beta[:, :t1], c.s0, None,
                 c.scale)
    o_cut, _ = f(c.q[:, t0:t1], c.k[:, t0:t1], c.v[:, t0:t1], c.g[:, t0:t1], c.beta[:, t0:t1],
                 None, None, c.scale)
    return float(o_err(o_cut[:, skip:], o_ref[:, t0 + skip:t1]))


@pytest.mark.parametrize("gate", ["zero", "near_one"])
def test_memory_crosses_a_chunk_boundary(gate):
    c = inputs.make_long_memory(seed=7, B=2, T=256, H=2, gate=gate)
    assert _restart_gap(c, 64, 128) > 5 * TOL_BF16
    assert _restart_gap(c, 192, 256) > 5 * TOL_BF16


def test_memory_crosses_a_chunk_boundary_per_channel():
    c = inputs.make_long_memory(seed=8, B=2, T=192, H=2, gate="near_one", per_channel=True)
    assert _restart_gap(c, 64, 128, per_channel=True) > 5 * TOL_BF16


def test_usual_prefill_gates_forget_within_a_chunk():
    """With the prefill workload's gates the same restart is invisible at
    the bar 16 tokens past the boundary: why the cases above exist."""
    c = inputs.make_prefill(seed=9, B=2, T=192, H=2)
    assert _restart_gap(c, 64, 128) < 1e-3
