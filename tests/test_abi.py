"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/gdn.h, and rejects bad arguments with the documented status
codes before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

GDN_OK, GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_DTYPE, GDN_ERR_UNSUPPORTED = 0, -1, -2, -3, -4
GDN_ERR_WORKSPACE = -6
GDN_ERR_SCRATCH = -7


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|const char \*)\s*(gdn_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    from gated_deltanet_recurrence_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        from gated_deltanet_recurrence_amd import build
        build.build()
    return _binding.load()


def test_header_and_binding_agree(lib):
    from gated_deltanet_recurrence_amd import _binding
    decl = declared_functions()
    assert len(decl) >= 8
    assert sorted(_binding.EXPORTED) == decl


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.gdn_version() == 3
    for st in (GDN_OK, GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_DTYPE, GDN_ERR_UNSUPPORTED, -5,
               GDN_ERR_WORKSPACE, GDN_ERR_SCRATCH, 99):
        s = lib.gdn_status_string(st)
        assert isinstance(s, bytes) and len(s) > 0


P = ctypes.c_void_p(16)      # a non-null dummy pointer; never dereferenced on rejection


def _prefill(lib, *, null=None, B=1, T=8, H=1, Hk=None, dk=128, dv=128, N=1, dtype=1, cu=None,
             ws=None, ws_bytes=0):
    ptrs = [P] * 8
    if null is not None:
        ptrs[null] = None
    q, k, v, g, beta, s0, s1, o = ptrs
    Hk = H if Hk is None else Hk
    return lib.gdn_prefill(q, k, v, g, beta, s0, s1, o, cu, B, T, H, Hk, dk, dv, N, 1.0, dtype,
                           ws, ws_bytes, None)


def _ws_size(lib, B=1, T=8, H=1, dk=128, dv=128, N=1, varlen=0, dtype=1):
    out = ctypes.c_size_t(12345)
    st = lib.gdn_prefill_workspace_size(B, T, H, dk, dv, N, varlen, dtype, ctypes.byref(out))
    return st, out.value


def test_workspace_size(lib):
    # 6 KiB of bf16 T diag(beta) (its lower 64 x 64 part: 32 x 32 + 32 x 64)
    # per (chunk slot, head); (tokens / 64 + N + 1) slots
    item = (32 * 32 + 32 * 64) * 2
    assert item == 6144
    assert _ws_size(lib, B=4, T=4096, H=16, N=4) == (GDN_OK, (4 * 4096 // 64 + 5) * 16 * item)
    assert _ws_size(lib, B=1, T=1000, H=3, N=7, varlen=1) == (GDN_OK, (1000 // 64 + 8) * 3 * item)
    assert _ws_size(lib, B=2, T=0, H=2, N=2) == (GDN_OK, 3 * 2 * item)
    # paths that use no workspace
    assert _ws_size(lib, dtype=0) == (GDN_OK, 0)
    assert _ws_size(lib, dk=64, dv=64) == (GDN_OK, 0)
    # the errors gdn_prefill would return
    assert _ws_size(lib, dk=48)[0] == GDN_ERR_UNSUPPORTED
    assert _ws_size(lib, B=2, N=1)[0] == GDN_ERR_SHAPE
    assert _ws_size(lib, dtype=9)[0] == GDN_ERR_DTYPE
    assert lib.gdn_prefill_workspace_size(1, 8, 1, 128, 128, 1, 0, 1, None) == GDN_ERR_NULL


def test_prefill_workspace_rejected(lib):
    need = _ws_size(lib, T=100)[1]
    aligned = ctypes.c_void_p(1 << 20)      # never dereferenced: rejected before launch
    assert _prefill(lib, T=100, ws=aligned, ws_bytes=need - 1) == GDN_ERR_WORKSPACE
    assert _prefill(lib, T=100, ws=ctypes.c_void_p((1 << 20) + 64), ws_bytes=need) == GDN_ERR_WORKSPACE


@pytest.mark.parametrize("which", [0, 1, 2, 3, 4, 7])
def test_prefill_null_pointers(lib, which):
    assert _prefill(lib, null=which) == GDN_ERR_NULL


def test_prefill_null_allowed_without_tokens(lib):
    # T = 0 with NULL activations passes validation (nothing is read); it is not
    # launched here, so only a rejection for another reason would show up
    assert _prefill(lib, null=0, T=0, dk=48) == GDN_ERR_UNSUPPORTED


def test_prefill_validation(lib):
    assert _prefill(lib, dtype=7) == GDN_ERR_DTYPE
    assert _prefill(lib, B=0) == GDN_ERR_SHAPE
    assert _prefill(lib, T=-1) == GDN_ERR_SHAPE
    assert _prefill(lib, H=0) == GDN_ERR_SHAPE
    assert _prefill(lib, B=2, N=1) == GDN_ERR_SHAPE          # N must equal B without offsets
    assert _prefill(lib, B=2, N=2, cu=P) == GDN_ERR_SHAPE    # packed sequences need B == 1
    assert _prefill(lib, dk=48) == GDN_ERR_UNSUPPORTED
    assert _prefill(lib, dv=256) == GDN_ERR_UNSUPPORTED
    assert _prefill(lib, B=1 << 16, N=1 << 16, T=1 << 16) == GDN_ERR_SHAPE
    # grouped heads: H_k must divide H
    assert _prefill(lib, H=4, Hk=0) == GDN_ERR_SHAPE
    assert _prefill(lib, H=4, Hk=3) == GDN_ERR_SHAPE
    assert _prefill(lib, H=4, Hk=8) == GDN_ERR_SHAPE


def test_decode_validation(lib):
    f = lib.gdn_decode_step
    assert f(P, P, P, P, P, None, P, 1, 1, 1, 128, 128, 1.0, 1, None) == GDN_ERR_NULL
    assert f(P, P, P, P, P, P, P, 1, 1, 1, 128, 128, 1.0, 2, None) == GDN_ERR_DTYPE
    assert f(P, P, P, P, P, P, P, 0, 1, 1, 128, 128, 1.0, 1, None) == GDN_ERR_SHAPE
    assert f(P, P, P, P, P, P, P, 1, 6, 4, 128, 128, 1.0, 1, None) == GDN_ERR_SHAPE
    assert f(P, P, P, P, P, P, P, 1, 1, 1, 100, 128, 1.0, 1, None) == GDN_ERR_UNSUPPORTED


def test_mixer_validation(lib):
    pro = lib.gdn_mixer_prologue
    args = [P] * 7 + [None, None] + [P] * 5
    bad = list(args)
    bad[0] = None
    assert pro(*bad, 1, 4, 1, 1, 128, 128, 1, 1, None) == GDN_ERR_NULL
    assert pro(*args, 1, 4, 1, 1, 128, 128, 1, 5, None) == GDN_ERR_DTYPE
    assert pro(*args, 1, 4, 1, 1, 96, 128, 1, 1, None) == GDN_ERR_UNSUPPORTED
    assert pro(*args, 2, 4, 1, 1, 128, 128, 1, 1, None) == GDN_ERR_SHAPE
    assert pro(*args, 1, 4, 2, 4, 128, 128, 1, 1, None) == GDN_ERR_SHAPE
    epi = lib.gdn_mixer_epilogue
    assert epi(None, P, None, P, 4, 1, 128, 1e-6, 1, None) == GDN_ERR_NULL
    assert epi(P, P, None, P, 4, 1, 100, 1e-6, 1, None) == GDN_ERR_UNSUPPORTED
    assert epi(P, P, None, P, -1, 1, 128, 1e-6, 1, None) == GDN_ERR_SHAPE


def test_check_cu_seqlens(lib):
    arr = lambda xs: (ctypes.c_int32 * len(xs))(*xs)
    f = lib.gdn_check_cu_seqlens
    assert f(arr([0, 5, 5, 12]), 3, 12) == GDN_OK
    assert f(arr([0, 5, 4, 12]), 3, 12) == GDN_ERR_SHAPE
    assert f(arr([1, 5, 12]), 2, 12) == GDN_ERR_SHAPE
    assert f(arr([0, 5, 11]), 2, 12) == GDN_ERR_SHAPE
    assert f(None, 2, 12) == GDN_ERR_NULL


def test_prepare_apply_validation(lib):
    need = _ws_size(lib, T=100)[1]
    ws = ctypes.c_void_p(1 << 20)            # never dereferenced: rejected before launch
    prep, app = lib.gdn_prefill_prepare, lib.gdn_prefill_apply
    # only the MFMA chunk path has two passes
    assert prep(P, P, P, P, None, 1, 100, 1, 1, 64, 64, 1, 1, ws, need, None) == GDN_ERR_UNSUPPORTED
    assert prep(P, P, P, P, None, 1, 100, 1, 1, 128, 128, 1, 0, ws, need, None) == GDN_ERR_UNSUPPORTED
    # the workspace is required and checked
    assert prep(P, P, P, P, None, 1, 100, 1, 1, 128, 128, 1, 1, None, 0, None) == GDN_ERR_NULL
    assert prep(P, P, P, P, None, 1, 100, 1, 1, 128, 128, 1, 1, ws, need - 1, None) == GDN_ERR_WORKSPACE
    assert prep(None, P, P, P, None, 1, 100, 1, 1, 128, 128, 1, 1, ws, need, None) == GDN_ERR_NULL
    assert prep(P, None, P, P, None, 1, 100, 1, 1, 128, 128, 1, 1, ws, need, None) == GDN_ERR_NULL
    assert prep(P, P, P, P, None, 2, 100, 1, 1, 128, 128, 1, 1, ws, need, None) == GDN_ERR_SHAPE
    a = [P] * 3 + [P, None, None, P, None]
    assert app(*a, 1, 100, 1, 1, 128, 128, 1, 1.0, 1, None, 0, None) == GDN_ERR_NULL
    assert app(*a, 1, 100, 1, 1, 128, 128, 1, 1.0, 1, ws, need - 1, None) == GDN_ERR_WORKSPACE
    assert app(*a, 1, 100, 1, 1, 16, 16, 1, 1.0, 1, ws, need, None) == GDN_ERR_UNSUPPORTED
    b = list(a)
    b[6] = None                              # o
    assert app(*b, 1, 100, 1, 1, 128, 128, 1, 1.0, 1, ws, need, None) == GDN_ERR_NULL
    # more (64-token slot, head) items than 32-bit indices reach: rejected
    # before the workspace is looked at
    big = (1, 2**31 - 1, 64, 64, 128, 128, 1)   # B, T, H, H_k, d_k, d_v, N
    assert prep(P, P, P, P, None, *big, 1, ws, 1 << 62, None) == GDN_ERR_UNSUPPORTED
    assert app(*a, *big, 1.0, 1, ws, 1 << 62, None) == GDN_ERR_UNSUPPORTED
    assert lib.gdn_prefill(P, P, P, P, P, None, None, P, None, *big, 1.0, 1, ws, 1 << 62,
                           None) == GDN_ERR_UNSUPPORTED
    out = ctypes.c_size_t(0)
    assert lib.gdn_prefill_workspace_size(1, 2**31 - 1, 64, 128, 128, 1, 0, 1,
                                          ctypes.byref(out)) == GDN_ERR_UNSUPPORTED
    # one head fewer fits
    assert lib.gdn_prefill_workspace_size(1, 2**31 - 1, 63, 128, 128, 1, 0, 1,
                                          ctypes.byref(out)) == GDN_OK and out.value > 0


def test_channel_gated_validation(lib):
    f = lib.gdn_prefill_channel_gated
    a = [P] * 5 + [None, None, P, None]
    bad = list(a)
    bad[3] = None                            # g
    assert f(*bad, 1, 8, 2, 2, 128, 128, 1, 1.0, 1, None, 0, None) == GDN_ERR_NULL
    assert f(*a, 1, 8, 4, 3, 128, 128, 1, 1.0, 1, None, 0, None) == GDN_ERR_SHAPE
    assert f(*a, 1, 8, 2, 2, 48, 128, 1, 1.0, 1, None, 0, None) == GDN_ERR_UNSUPPORTED
    # the chunkwise path's workspace: sized per item, checked before any launch
    out = ctypes.c_size_t(0)
    ws_size = lib.gdn_prefill_channel_workspace_size
    assert ws_size(1, 100, 2, 128, 128, 1, 0, 1, ctypes.byref(out)) == GDN_OK
    need = out.value
    scalar = ctypes.c_size_t(0)
    assert lib.gdn_prefill_workspace_size(1, 100, 2, 128, 128, 1, 0, 1, ctypes.byref(scalar)) == GDN_OK
    assert need > scalar.value > 0
    assert ws_size(1, 100, 2, 64, 64, 1, 0, 1, ctypes.byref(out)) == GDN_OK and out.value == 0
    assert ws_size(1, 100, 2, 128, 128, 1, 0, 1, None) == GDN_ERR_NULL
    ws = 256 * 1024                          # aligned stand-in address, never dereferenced
    assert f(*a, 1, 100, 2, 2, 128, 128, 1, 1.0, 1, ws, need - 1, None) == GDN_ERR_WORKSPACE
    assert f(*a, 1, 100, 2, 2, 128, 128, 1, 1.0, 1, ws + 16, need, None) == GDN_ERR_WORKSPACE
    d = lib.gdn_decode_step_channel_gated
    assert d(P, P, P, None, P, P, P, 1, 2, 2, 128, 128, 1.0, 1, None) == GDN_ERR_NULL
    assert d(P, P, P, P, P, P, P, 1, 2, 2, 128, 128, 1.0, 3, None) == GDN_ERR_DTYPE
    assert d(P, P, P, P, P, P, P, 1, 6, 4, 128, 128, 1.0, 1, None) == GDN_ERR_SHAPE


def test_seqpar_validation(lib):
    out = ctypes.c_size_t(0)
    f = lib.gdn_prefill_seqpar_workspace_size
    # B, T, H, d_k, d_v, N, varlen, segments, dtype
    assert f(1, 4096, 16, 128, 128, 1, 0, 8, 1, ctypes.byref(out)) == GDN_OK and out.value > 0
    one = out.value
    assert f(1, 4096, 16, 128, 128, 8, 1, 8, 1, ctypes.byref(out)) == GDN_OK
    assert out.value > one                   # packed: 8 sequences of up to 8 segments
    assert f(1, 4096, 16, 64, 64, 1, 0, 8, 1, ctypes.byref(out)) == GDN_ERR_UNSUPPORTED
    assert f(1, 4096, 16, 128, 128, 1, 0, 0, 1, ctypes.byref(out)) == GDN_ERR_SHAPE
    assert f(1, 4096, 16, 128, 128, 1, 0, 8, 0, ctypes.byref(out)) == GDN_ERR_UNSUPPORTED
    assert f(1, 4096, 16, 128, 128, 1, 0, 8, 1, None) == GDN_ERR_NULL
    assert f(2, 4096, 16, 128, 128, 2, 1, 8, 1, ctypes.byref(out)) == GDN_ERR_SHAPE  # packed: B = 1
    assert f(1, 4096, 16, 128, 128, 4096, 1, 16, 1, ctypes.byref(out)) == GDN_ERR_UNSUPPORTED
    assert f(1, 2**31 - 1, 64, 128, 128, 1, 0, 1, 1, ctypes.byref(out)) == GDN_ERR_UNSUPPORTED
    sp = lib.gdn_prefill_seqpar
    ws = ctypes.c_void_p(1 << 20)            # never dereferenced: rejected before launch
    a = [P] * 5 + [None, None, P, None]
    dims = [1, 4096, 16, 16, 128, 128, 1, 8]  # B, T, H, H_k, d_k, d_v, N, segments
    assert sp(*a, *dims, 1.0, 1, None, 0, None) == GDN_ERR_NULL
    assert sp(*a, *dims, 1.0, 1, ws, 10, None) == GDN_ERR_WORKSPACE
    bad = list(dims)
    bad[3] = 5                               # H_k does not divide H
    assert sp(*a, *bad, 1.0, 1, ws, 1 << 40, None) == GDN_ERR_SHAPE
    bad = list(dims)
    bad[6] = 3                               # N != B without offsets
    assert sp(*a, *bad, 1.0, 1, ws, 1 << 40, None) == GDN_ERR_SHAPE
    b = list(a)
    b[7] = None                              # o
    assert sp(*b, *dims, 1.0, 1, ws, 1 << 40, None) == GDN_ERR_NULL


def test_noalloc_validation(lib):
    f = lib.gdn_prefill_noalloc

    def call(null=None, B=1, T=8, H=1, dk=128, dv=128, N=1, dtype=1):
        ptrs = [P] * 8
        if null is not None:
            ptrs[null] = None
        return f(*ptrs, None, B, T, H, H, dk, dv, N, 1.0, dtype, None)
    assert call(null=0) == GDN_ERR_NULL
    assert call(dtype=3) == GDN_ERR_DTYPE
    assert call(dk=48) == GDN_ERR_UNSUPPORTED
    # beyond the static scratch (32 MiB = 5461 items of 6 KiB): rejected before launch
    assert call(B=4, T=8192, H=16, N=4) == GDN_ERR_SCRATCH
    assert call(B=1, T=64 * 5461, H=1) == GDN_ERR_SCRATCH


def test_binding_rejects_host_tensors(lib):
    import torch
    from gated_deltanet_recurrence_amd import _binding
    q = torch.zeros(1, 4, 1, 128, dtype=torch.bfloat16)
    g = torch.zeros(1, 4, 1, dtype=torch.float32)
    with pytest.raises(_binding.GDNError, match="GPU tensor"):
        _binding.gdn_prefill(q, q, q, g, g, workspace=None)
    with pytest.raises(_binding.GDNError, match="GPU tensor"):
        _binding.gdn_decode_step(q[:, 0], q[:, 0], q[:, 0], g[:, 0], g[:, 0],
                                 torch.zeros(1, 1, 128, 128))


def test_binding_requires_one_device_per_call(lib):
    # inside a call every tensor must sit on the call's device (checked before
    # the library runs; the meta device stands in for a second GPU)
    import torch
    from gated_deltanet_recurrence_amd import _binding
    _binding._ctx.device = torch.device("cuda", 0)
    try:
        with pytest.raises(_binding.GDNError, match="is on meta"):
            _binding._same_device(torch.empty(0, device="meta"), "v")
    finally:
        _binding._ctx.device = None
    _binding._same_device(torch.empty(0, device="meta"), "v")   # no call running: no check
