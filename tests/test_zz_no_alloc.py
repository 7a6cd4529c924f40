"""gdn_prefill_noalloc (the entry point that allocates nothing) against
gdn_prefill with a caller workspace, through the C ABI.

Two calls in a row on the static scratch, the second with a smaller, packed
input, so that the second runs over what the first left in the buffer; each
must give gdn_prefill's result bit for bit (same kernels), hence within the
bf16 bar of the oracle. Sizes above the scratch are rejected before anything
is enqueued, and paths that use no scratch run as in gdn_prefill.
"""
import pytest
import torch

import oracle
import gated_deltanet_recurrence_amd as gdn
from gated_deltanet_recurrence_amd import inputs
from parity import TOL_BF16, TOL_F32, dev, o_err, o_err_packed, report, s_err

pytestmark = pytest.mark.gpu

GDN_ERR_SCRATCH = -7


def _both(c):
    s0 = dev(c.s0)
    shape = (c.N, c.H, c.d_v, c.d_k)
    f_ws = torch.empty(shape, dtype=torch.float32, device="cuda:0")
    f_na = torch.empty(shape, dtype=torch.float32, device="cuda:0")
    o_na = torch.empty(tuple(c.v.shape), dtype=c.v.dtype, device="cuda:0")
    args = (dev(c.q), dev(c.k), dev(c.v), dev(c.g), dev(c.beta))
    cu = dev(c.cu_seqlens)
    o_ws, _ = gdn.gdn_prefill(*args, s0, f_ws, cu_seqlens=cu, scale=c.scale, workspace="auto")
    gdn.gdn_prefill_noalloc(*args, s0, f_na, o_na, cu_seqlens=cu, scale=c.scale)
    torch.cuda.synchronize()
    return o_ws, f_ws, o_na, f_na


def test_noalloc_matches_the_workspace_path_twice():
    big = inputs.make_prefill(seed=170, B=2, T=700, H=3, d=128, with_state=True)
    small = inputs.make_varlen(seed=171, H=2, d=128, lengths=[5, 0, 130, 64])
    for c in (big, small):
        o_ws, f_ws, o_na, f_na = _both(c)
        assert torch.equal(o_na, o_ws) and torch.equal(f_na, f_ws)
        o_ref, s_ref = oracle.gdn_recurrent(c.q, c.k, c.v, c.g, c.beta, c.s0, c.cu_seqlens,
                                            c.scale)
        if c.cu_seqlens is None:
            eo = o_err(o_na, o_ref)
        else:
            eo = o_err_packed(o_na, o_ref, [int(x) for x in c.cu_seqlens.tolist()])
        es = s_err(f_na, s_ref)
        report(f"noalloc {c.name} B={c.B} T={c.T} H={c.H}", o=eo, state=es)
        assert eo <= TOL_BF16 and es <= TOL_BF16


def test_noalloc_rejects_sizes_beyond_the_scratch():
    from gated_deltanet_recurrence_amd import _binding
    # B=4, T=8192, H=16: (512 + 5) slots x 16 heads x 6 KiB > 32 MiB
    q = torch.zeros((4, 8192, 16, 128), dtype=torch.bfloat16, device="cuda:0")
    g = torch.zeros((4, 8192, 16), dtype=torch.float32, device="cuda:0")
    o = torch.empty_like(q)
    with pytest.raises(_binding.GDNError, match=str(GDN_ERR_SCRATCH)):
        gdn.gdn_prefill_noalloc(q, q, q, g, g, None, None, o)
    torch.cuda.synchronize()


def test_noalloc_fp32_path_needs_no_scratch():
    c = inputs.make_prefill(seed=172, B=1, T=90, H=2, d=64, dtype="f32", with_state=True)
    o_ws, f_ws, o_na, f_na = _both(c)
    assert torch.equal(o_na, o_ws) and torch.equal(f_na, f_ws)
    o_ref, s_ref = oracle.gdn_recurrent(c.q, c.k, c.v, c.g, c.beta, c.s0, None, c.scale)
    assert o_err(o_na, o_ref) <= TOL_F32 and s_err(f_na, s_ref) <= TOL_F32
