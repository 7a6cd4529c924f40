"""Non-finite inputs on the GPU paths: a NaN in one input entry poisons what
the recurrence makes depend on it, and nothing else ("Overwrite and Forget",
section 4: the state is the only carrier between tokens of one (sequence,
head); heads and sequences never mix). Nothing is masked: the poisoned
outputs and state entries come out NaN.

* v[b, t, h, c] NaN: only d_v column c of that (sequence, head) depends on it
  (the delta rule acts on each state row on its own), from token t on, and
  state row c. The chunkwise paths form a chunk's outputs together
  (0 * NaN = NaN in the products that mask later tokens), so there column c
  is NaN from the start of t's chunk; the token-serial paths match the
  oracle's token t.
* k[b, t, hk] NaN: every d_v of the value heads reading that key head, from
  t's chunk (chunkwise) or token t on, and their whole state.

Everything else must be finite and match the oracle at the usual bar.
"""
import numpy as np
import pytest
import torch

import oracle
import gated_deltanet_recurrence_amd as gdn
from gated_deltanet_recurrence_amd import inputs
from parity import TOL_BF16, TOL_F32, dev, host64, o_err, s_err

pytestmark = pytest.mark.gpu

B, T, H, D = 2, 300, 3, 128
BAD_B, BAD_T, BAD_H, BAD_C = 1, 150, 2, 37       # token 150 lies in chunk 2 (128..191)
CHUNK0 = BAD_T // 64 * 64


def _case(dtype):
    return inputs.make_prefill(seed=960, B=B, T=T, H=H, d=D, dtype=dtype, with_state=True)


def _check(o, fin, c, field, first_bad, tol):
    """o, fin from the GPU, field 'v' or 'k' poisoned at (BAD_B, BAD_T, BAD_H);
    first_bad: the first token whose outputs may be poisoned."""
    o, fin = host64(o.cpu()), host64(fin.cpu())
    o_ref, s_ref = oracle.gdn_recurrent(c.q, c.k, c.v, c.g, c.beta, c.s0, scale=c.scale)
    cols = [BAD_C] if field == "v" else list(range(D))
    good_o = np.ones(o.shape, dtype=bool)
    good_o[BAD_B, first_bad:, BAD_H, cols] = False
    good_s = np.ones(fin.shape, dtype=bool)
    good_s[BAD_B, BAD_H, cols, :] = False
    # poisoned entries are NaN, the rest finite
    assert np.isnan(o[~good_o]).all() and np.isnan(fin[~good_s]).all()
    assert np.isfinite(o[good_o]).all() and np.isfinite(fin[good_s]).all()
    # the untouched pairs and the untouched part of the poisoned pair match the oracle
    for b in range(B):
        for h in range(H):
            if (b, h) == (BAD_B, BAD_H):
                continue
            assert o_err(o[b:b + 1, :, h:h + 1], o_ref[b:b + 1, :, h:h + 1]) <= tol
            assert s_err(fin[b:b + 1, h:h + 1], s_ref[b:b + 1, h:h + 1]) <= tol
    head = o[BAD_B, :first_bad, BAD_H]
    ref = o_ref[BAD_B, :first_bad, BAD_H]
    assert np.abs(head - ref).max() <= tol * max(np.abs(ref).max(), 1e-30)
    if field == "v":
        keep = [c2 for c2 in range(D) if c2 != BAD_C]
        x, r = o[BAD_B, :, BAD_H][:, keep], o_ref[BAD_B, :, BAD_H][:, keep]
        assert np.abs(x - r).max() <= tol * np.abs(r).max()


def _poison(c, field):
    x = getattr(c, field).clone()
    if field == "v":
        x[BAD_B, BAD_T, BAD_H, BAD_C] = float("nan")
    else:
        x[BAD_B, BAD_T, BAD_H] = float("nan")
    setattr(c, field, x)


@pytest.mark.parametrize("field", ["v", "k"])
@pytest.mark.parametrize("path", ["two_pass", "one_pass", "recurrent_f32"])
def test_nan_poisons_only_its_dependents(field, path):
    c = _case("f32" if path == "recurrent_f32" else "bf16")
    _poison(c, field)
    fin = torch.empty((B, H, D, D), dtype=torch.float32, device="cuda:0")
    if path == "recurrent_f32":
        o, _ = gdn.gdn_prefill_recurrent(dev(c.q), dev(c.k), dev(c.v), dev(c.g), dev(c.beta),
                                         dev(c.s0), fin, scale=c.scale)
        first_bad, tol = BAD_T, TOL_F32
    else:
        o, _ = gdn.gdn_prefill(dev(c.q), dev(c.k), dev(c.v), dev(c.g), dev(c.beta), dev(c.s0),
                               fin, scale=c.scale,
                               workspace="auto" if path == "two_pass" else None)
        first_bad, tol = CHUNK0, TOL_BF16
    torch.cuda.synchronize()
    _check(o, fin, c, field, first_bad, tol)


@pytest.mark.parametrize("field", ["v", "k"])
def test_nan_in_decode_step(field):
    """One decode step: the poisoned (sequence, head) only; for v only its
    state row and output entry c."""
    c = inputs.make_decode(seed=961, B=4, H=3, d=D)
    x = getattr(c, field).clone()
    if field == "v":
        x[BAD_B, 0, BAD_H, BAD_C] = float("nan")
    else:
        x[BAD_B, 0, BAD_H] = float("nan")
    setattr(c, field, x)
    st = dev(c.s0)
    o = gdn.gdn_decode_step(dev(c.q[:, 0]), dev(c.k[:, 0]), dev(c.v[:, 0]), dev(c.g[:, 0]),
                            dev(c.beta[:, 0]), st, scale=c.scale)
    torch.cuda.synchronize()
    o, st = host64(o.cpu()), host64(st.cpu())
    o_ref, s_ref = oracle.gdn_recurrent(c.q, c.k, c.v, c.g, c.beta, c.s0, scale=c.scale)
    cols = [BAD_C] if field == "v" else list(range(D))
    bad_o = np.zeros(o.shape, dtype=bool)
    bad_o[BAD_B, BAD_H, cols] = True
    bad_s = np.zeros(st.shape, dtype=bool)
    bad_s[BAD_B, BAD_H, cols, :] = True
    assert np.isnan(o[bad_o]).all() and np.isnan(st[bad_s]).all()
    assert np.isfinite(o[~bad_o]).all() and np.isfinite(st[~bad_s]).all()
    ok = ~bad_o
    assert np.abs(o[ok] - o_ref[:, 0][ok]).max() <= TOL_BF16 * np.abs(o_ref[:, 0][ok]).max()
    ok = ~bad_s
    assert np.abs(st[ok] - s_ref[ok]).max() <= TOL_BF16 * np.abs(s_ref[ok]).max()
