"""Host-side sanitizer runs and non-finite propagation (CPU only).

* The fp64 oracle is built with AddressSanitizer and UndefinedBehavior-
  Sanitizer (gcc) together with a C driver that calls every oracle entry
  point on small, awkward layouts (tests/sanitize/oracle_checks.c); any
  out-of-bounds access or undefined operation aborts it.
* NaN and Inf inputs must propagate through the oracle's recurrence into
  every later output and the final state of their own (sequence, head)
  chain, and into nothing else: a check that silently masked them (a
  clamp, a max with zero, an isfinite filter) would hide broken inputs.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from gated_deltanet_recurrence_amd import inputs

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(HERE, "sanitize", "oracle_checks.c"),
           os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stderr[-4000:]
    assert "ok" in res.stdout


@pytest.mark.parametrize("field,value", [("v", np.nan), ("k", np.inf), ("q", np.nan),
                                         ("g", np.nan), ("beta", np.inf)])
def test_non_finite_inputs_propagate(field, value):
    """A non-finite value at token 5 of head 1 in packed sequence 1 reaches
    that chain's later outputs (the query's only from its own token on) and
    its final state, and no other chain."""
    c = inputs.make_varlen(seed=61, H=3, d=16, dtype="f32", lengths=[9, 12, 7])
    arr = getattr(c, field).clone()
    t_bad = 9 + 5
    arr[0, t_bad, 1] = value
    c2 = c.__class__(**{**c.__dict__, field: arr})
    o, s1 = oracle.gdn_recurrent(c2.q, c2.k, c2.v, c2.g, c2.beta, c2.s0, c2.cu_seqlens, c2.scale)
    o_ok, s_ok = oracle.gdn_recurrent(c.q, c.k, c.v, c.g, c.beta, c.s0, c.cu_seqlens, c.scale)
    bad = ~np.isfinite(o)
    last = 21                      # end of sequence 1
    if field == "q":
        # a query only reads the state: just its own token's output is hit
        assert bad[0, t_bad, 1].all()
        assert np.isfinite(o[0, t_bad + 1:last, 1]).all()
        assert np.array_equal(s1[1, 1], s_ok[1, 1])
        hit = (slice(t_bad, t_bad + 1),)
    else:
        # the chain (sequence 1, head 1): non-finite from the bad token on
        assert bad[0, t_bad:last, 1].all()
        assert not np.isfinite(s1[1, 1]).all()
        hit = (slice(t_bad, last),)
    # every other chain is untouched, bit for bit
    mask = np.ones(o.shape[:3], dtype=bool)
    mask[0, hit[0], 1] = False
    assert np.array_equal(o[mask], o_ok[mask])
    for n in range(3):
        for h in range(3):
            if (n, h) != (1, 1):
                assert np.array_equal(s1[n, h], s_ok[n, h])
