"""ctypes binding of libgdn.so: argument marshalling only.

Each wrapper checks that the torch tensors it is given are on the GPU,
contiguous, of the expected dtype and shape, passes their device pointers and
the current HIP stream to the C entry point of the same name, and raises on a
non-zero status. No arithmetic of the method runs here; torch only supplies
device memory and streams. If libgdn.so is missing the first call raises
(build it with ``python -m gated_deltanet_recurrence_amd.build``): there is
no fallback path.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_DTYPE_F32 = 0
GDN_DTYPE_BF16 = 1
_DTYPES = {torch.float32: GDN_DTYPE_F32, torch.bfloat16: GDN_DTYPE_BF16}

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

# name -> argtypes (restype int for all)
_SIGS = {
    "gdn_version": [],
    "gdn_status_string": [_i],
    "gdn_check_cu_seqlens": [_vp, _i, _i],
    "gdn_prefill": [_vp] * 9 + [_i] * 7 + [_f, _i, _vp, _sz, _vp],
    "gdn_prefill_noalloc": [_vp] * 9 + [_i] * 7 + [_f, _i, _vp],
    "gdn_prefill_workspace_size": [_i] * 8 + [_vp],
    "gdn_prefill_prepare": [_vp] * 5 + [_i] * 8 + [_vp, _sz, _vp],
    "gdn_prefill_apply": [_vp] * 8 + [_i] * 7 + [_f, _i, _vp, _sz, _vp],
    "gdn_prefill_recurrent": [_vp] * 9 + [_i] * 7 + [_f, _i, _vp],
    "gdn_decode_step": [_vp] * 7 + [_i] * 5 + [_f, _i, _vp],
    "gdn_mixer_prologue": [_vp] * 14 + [_i] * 8 + [_vp],
    "gdn_mixer_epilogue": [_vp] * 4 + [_i] * 3 + [_f, _i, _vp],
    "gdn_prefill_seqpar": [_vp] * 9 + [_i] * 8 + [_f, _i, _vp, _sz, _vp],
    "gdn_prefill_seqpar_workspace_size": [_i] * 9 + [_vp],
    "gdn_prefill_channel_gated": [_vp] * 9 + [_i] * 7 + [_f, _i, _vp, _sz, _vp],
    "gdn_prefill_channel_workspace_size": [_i] * 8 + [_vp],
    "gdn_decode_step_channel_gated": [_vp] * 7 + [_i] * 5 + [_f, _i, _vp],
    "gdn_decode_mixer_step": [_vp] * 11 + [_f, _vp, _vp] + [_i] * 5 + [_f, _i, _vp],
}
EXPORTED = tuple(_SIGS)

_lib = None


class GDNError(RuntimeError):
    pass


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libgdn.so (once) and declare the entry points' signatures."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise GDNError(f"{p} is missing: build it with "
                       "`python -m gated_deltanet_recurrence_amd.build`")
    lib = ctypes.CDLL(p)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "gdn_status_string" else ctypes.c_int
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = load().gdn_status_string(status).decode()
        raise GDNError(f"libgdn status {status}: {msg}")


# The device a call runs on (that of its first tensor): every tensor of the
# call must live there, and it is the current device while the library runs
# (its per-device launch settings are looked up for the current device).
_ctx = threading.local()


@contextlib.contextmanager
def _on(device):
    if device.type != "cuda":                 # the tensor checks reject the call
        yield
        return
    prev = getattr(_ctx, "device", None)
    _ctx.device = device
    try:
        with torch.cuda.device(device):
            yield
    finally:
        _ctx.device = prev


def _same_device(t: torch.Tensor, name: str):
    want = getattr(_ctx, "device", None)
    if want is not None and t.device != want:
        raise GDNError(f"{name} is on {t.device}, the call's other tensors on {want}")


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, shape=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise GDNError(f"{name} must be a GPU tensor")
    _same_device(t, name)
    if not t.is_contiguous():
        raise GDNError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise GDNError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise GDNError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise GDNError(f"unsupported dtype {t.dtype}")
    return _DTYPES[t.dtype]


def gdn_prefill_workspace_size(B, T, H, d_k, d_v, N, varlen, dtype) -> int:
    """Bytes of workspace gdn_prefill uses for these sizes (0: none)."""
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    out = ctypes.c_size_t(0)
    _check(load().gdn_prefill_workspace_size(B, T, H, d_k, d_v, N, int(bool(varlen)), code,
                                             ctypes.byref(out)))
    return out.value


def gdn_prefill_channel_workspace_size(B, T, H, d_k, d_v, N, varlen, dtype) -> int:
    """Bytes of workspace gdn_prefill_channel_gated uses for these sizes (0: none)."""
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    out = ctypes.c_size_t(0)
    _check(load().gdn_prefill_channel_workspace_size(B, T, H, d_k, d_v, N, int(bool(varlen)),
                                                     code, ctypes.byref(out)))
    return out.value


def _prefill(entry, q, k, v, g, beta, initial_state=None, final_state=None, o=None,
             cu_seqlens=None, scale=None, workspace=None):
    B, T, Hk, dk = q.shape
    H, dv = v.shape[2], v.shape[3]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    dt = q.dtype
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=q.device)
    if scale is None:
        scale = dk ** -0.5
    with _on(q.device):
        args = [
            _dev(q, "q", dt), _dev(k, "k", dt, q.shape), _dev(v, "v", dt, (B, T, H, dv)),
            _dev(g, "g", torch.float32,
                 (B, T, H, dk) if entry == "gdn_prefill_channel_gated" else (B, T, H)),
            _dev(beta, "beta", torch.float32, (B, T, H)),
            _dev(initial_state, "initial_state", torch.float32, (N, H, dv, dk)),
            _dev(final_state, "final_state", torch.float32, (N, H, dv, dk)),
            _dev(o, "o", dt, (B, T, H, dv)),
            _dev(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,)),
        ]
        tail = [float(scale), _dtype_code(q)]
        if entry in ("gdn_prefill", "gdn_prefill_channel_gated"):
            if isinstance(workspace, str):
                if workspace != "auto":
                    raise GDNError("workspace must be None, 'auto' or a tensor, "
                                   f"got {workspace!r}")
                size = (gdn_prefill_workspace_size if entry == "gdn_prefill"
                        else gdn_prefill_channel_workspace_size)
                nbytes = size(B, T, H, dk, dv, N, cu_seqlens is not None, _dtype_code(q))
                workspace = (torch.empty(nbytes, dtype=torch.uint8, device=q.device)
                             if nbytes else None)
            tail += list(_ws(workspace))
        _check(getattr(load(), entry)(*args, B, T, H, Hk, dk, dv, N, *tail, _stream(q.device)))
    return o, final_state


def gdn_prefill(q, k, v, g, beta, initial_state=None, final_state=None, o=None,
                cu_seqlens=None, scale=None, workspace="auto"):
    """Chunkwise forward (see include/gdn.h). Returns (o, final_state).

    workspace: "auto" allocates the scratch memory of the two-pass path with
    torch (size from gdn_prefill_workspace_size), a uint8 GPU tensor is used
    as given, None selects the single-pass path that needs none."""
    return _prefill("gdn_prefill", q, k, v, g, beta, initial_state, final_state, o,
                    cu_seqlens, scale, workspace)


def gdn_prefill_noalloc(q, k, v, g, beta, initial_state=None, final_state=None, o=None,
                        cu_seqlens=None, scale=None):
    """gdn_prefill with the library's static scratch instead of a workspace
    (see include/gdn.h): the C call allocates nothing. Pass ``o`` (and the
    states) to allocate nothing here either. Returns (o, final_state)."""
    return _prefill("gdn_prefill_noalloc", q, k, v, g, beta, initial_state, final_state, o,
                    cu_seqlens, scale)


def _ws(workspace):
    if workspace is None:
        return None, 0
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise GDNError("workspace must be a contiguous GPU tensor")
    _same_device(workspace, "workspace")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def gdn_prefill_prepare(q, k, g, beta, workspace, cu_seqlens=None, d_v=None):
    """First pass of the workspace path (see include/gdn.h): T diag(beta) of
    every 64-token chunk and head into `workspace` (T the inverse of the
    chunk's unit-lower-triangular key Gram system). The value heads H are
    those of g and beta."""
    B, T, Hk, dk = k.shape
    H = g.shape[2]
    dv = dk if d_v is None else d_v
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    if q.shape != k.shape or q.dtype != k.dtype:
        raise GDNError("q must match k in shape and dtype")
    with _on(k.device):
        _check(load().gdn_prefill_prepare(
            _dev(q, "q"), _dev(k, "k"), _dev(g, "g", torch.float32, (B, T, H)),
            _dev(beta, "beta", torch.float32, (B, T, H)),
            _dev(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,)),
            B, T, H, Hk, dk, dv, N, _dtype_code(k), *_ws(workspace), _stream(k.device)))


def gdn_prefill_apply(q, k, v, g, workspace, initial_state=None, final_state=None, o=None,
                      cu_seqlens=None, scale=None):
    """Second pass of the workspace path: the state recurrence over chunks.
    Returns (o, final_state)."""
    B, T, Hk, dk = q.shape
    H, dv = v.shape[2], v.shape[3]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    dt = q.dtype
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=q.device)
    if scale is None:
        scale = dk ** -0.5
    with _on(q.device):
        _check(load().gdn_prefill_apply(
            _dev(q, "q", dt), _dev(k, "k", dt, q.shape), _dev(v, "v", dt, (B, T, H, dv)),
            _dev(g, "g", torch.float32, (B, T, H)),
            _dev(initial_state, "initial_state", torch.float32, (N, H, dv, dk)),
            _dev(final_state, "final_state", torch.float32, (N, H, dv, dk)),
            _dev(o, "o", dt, (B, T, H, dv)), _dev(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,)),
            B, T, H, Hk, dk, dv, N, float(scale), _dtype_code(q), *_ws(workspace),
            _stream(q.device)))
    return o, final_state


def gdn_prefill_recurrent(q, k, v, g, beta, initial_state=None, final_state=None, o=None,
                          cu_seqlens=None, scale=None):
    """Token-serial fp32 forward (see include/gdn.h). Returns (o, final_state)."""
    return _prefill("gdn_prefill_recurrent", q, k, v, g, beta, initial_state, final_state, o,
                    cu_seqlens, scale)


def gdn_prefill_seqpar_workspace_size(B, T, H, d_k, d_v, N, varlen, segments, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    out = ctypes.c_size_t(0)
    _check(load().gdn_prefill_seqpar_workspace_size(B, T, H, d_k, d_v, N, int(bool(varlen)),
                                                    segments, code, ctypes.byref(out)))
    return out.value


def gdn_prefill_seqpar(q, k, v, g, beta, segments, initial_state=None, final_state=None, o=None,
                       cu_seqlens=None, scale=None, workspace=None):
    """Sequence-parallel chunked forward (see include/gdn.h): the longest
    sequence is cut into `segments` runs of whole chunks, the others into runs
    of the same length, and the runs' chains go side by side. Packed sequences
    as for gdn_prefill (B = 1, cu_seqlens). Returns (o, final_state).
    workspace: a uint8 GPU tensor, or None to allocate one with torch."""
    B, T, Hk, dk = q.shape
    H, dv = v.shape[2], v.shape[3]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    dt = q.dtype
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=dt, device=q.device)
    if scale is None:
        scale = dk ** -0.5
    if workspace is None:
        workspace = torch.empty(
            gdn_prefill_seqpar_workspace_size(B, T, H, dk, dv, N, cu_seqlens is not None,
                                              segments, dt),
            dtype=torch.uint8, device=q.device)
    with _on(q.device):
        _check(load().gdn_prefill_seqpar(
            _dev(q, "q", dt), _dev(k, "k", dt, q.shape), _dev(v, "v", dt, (B, T, H, dv)),
            _dev(g, "g", torch.float32, (B, T, H)), _dev(beta, "beta", torch.float32, (B, T, H)),
            _dev(initial_state, "initial_state", torch.float32, (N, H, dv, dk)),
            _dev(final_state, "final_state", torch.float32, (N, H, dv, dk)),
            _dev(o, "o", dt, (B, T, H, dv)),
            _dev(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,)),
            B, T, H, Hk, dk, dv, N, int(segments), float(scale), _dtype_code(q), *_ws(workspace),
            _stream(q.device)))
    return o, final_state


def gdn_prefill_channel_gated(q, k, v, g, beta, initial_state=None, final_state=None, o=None,
                              cu_seqlens=None, scale=None, workspace="auto"):
    """Forward pass with one decay rate per key channel: g [B,T,H,d_k] fp32
    (see include/gdn.h). Returns (o, final_state). workspace: "auto" allocates
    the scratch memory of the chunkwise path (bf16, d_k = d_v = 128) with
    torch, a uint8 GPU tensor is used as given, None selects the token-serial
    path."""
    return _prefill("gdn_prefill_channel_gated", q, k, v, g, beta, initial_state, final_state, o,
                    cu_seqlens, scale, workspace)


def gdn_decode_step_channel_gated(q, k, v, g, beta, state, o=None, scale=None):
    """One in-place step with one decay rate per key channel: g [B,H,d_k] fp32."""
    return _decode("gdn_decode_step_channel_gated", q, k, v, g, beta, state, o, scale)


def gdn_decode_step(q, k, v, g, beta, state, o=None, scale=None):
    """One in-place recurrent step. q,k: [B,H_k,d_k]; v: [B,H,d_v]; g,beta: [B,H];
    state: [B,H,d_v,d_k] fp32 (updated). Returns o [B,H,d_v]."""
    return _decode("gdn_decode_step", q, k, v, g, beta, state, o, scale)


def _decode(entry, q, k, v, g, beta, state, o, scale):
    B, Hk, dk = q.shape
    H, dv = v.shape[1], v.shape[2]
    dt = q.dtype
    if o is None:
        o = torch.empty((B, H, dv), dtype=dt, device=q.device)
    if scale is None:
        scale = dk ** -0.5
    with _on(q.device):
        _check(getattr(load(), entry)(
            _dev(q, "q", dt), _dev(k, "k", dt, q.shape), _dev(v, "v", dt, (B, H, dv)),
            _dev(g, "g", torch.float32, (B, H, dk) if entry.endswith("channel_gated") else (B, H)),
            _dev(beta, "beta", torch.float32, (B, H)),
            _dev(state, "state", torch.float32, (B, H, dv, dk)), _dev(o, "o", dt, (B, H, dv)),
            B, H, Hk, dk, dv, float(scale), _dtype_code(q), _stream(q.device)))
    return o


def gdn_mixer_prologue(q_raw, k_raw, v_raw, conv_w, a, b, A, dt_bias=None, cu_seqlens=None,
                       out=None):
    """Conv+SiLU, L2-norm of q,k, gates. q_raw, k_raw: [B,T,H_k,d_k]; v_raw:
    [B,T,H,d_v]; a, b: [B,T,H]. Returns (q, k, v, g, beta)."""
    B, T, Hk, dk = q_raw.shape
    H, dv = v_raw.shape[2], v_raw.shape[3]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    dt = q_raw.dtype
    if out is None:
        out = (torch.empty_like(q_raw), torch.empty_like(k_raw), torch.empty_like(v_raw),
               torch.empty((B, T, H), dtype=torch.float32, device=q_raw.device),
               torch.empty((B, T, H), dtype=torch.float32, device=q_raw.device))
    q, k, v, g, beta = out
    with _on(q_raw.device):
        _check(load().gdn_mixer_prologue(
            _dev(q_raw, "q_raw", dt), _dev(k_raw, "k_raw", dt, q_raw.shape),
            _dev(v_raw, "v_raw", dt, (B, T, H, dv)),
            _dev(conv_w, "conv_w", dt, (2 * Hk * dk + H * dv, 4)),
            _dev(a, "a", dt, (B, T, H)), _dev(b, "b", dt, (B, T, H)),
            _dev(A, "A", torch.float32, (H,)), _dev(dt_bias, "dt_bias", torch.float32, (H,)),
            _dev(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,)),
            _dev(q, "q", dt, q_raw.shape), _dev(k, "k", dt, q_raw.shape),
            _dev(v, "v", dt, (B, T, H, dv)), _dev(g, "g", torch.float32, (B, T, H)),
            _dev(beta, "beta", torch.float32, (B, T, H)),
            B, T, H, Hk, dk, dv, N, _dtype_code(q_raw), _stream(q_raw.device)))
    return q, k, v, g, beta


def gdn_mixer_epilogue(y, z, norm_w=None, out=None, eps=1e-6):
    """Gated RMSNorm over the last axis of y [B,T,H,d_v] with gate z."""
    B, T, H, dv = y.shape
    dt = y.dtype
    if out is None:
        out = torch.empty_like(y)
    with _on(y.device):
        _check(load().gdn_mixer_epilogue(
            _dev(y, "y", dt), _dev(z, "z", dt, y.shape),
            _dev(norm_w, "norm_w", torch.float32, (dv,)),
            _dev(out, "out", dt, y.shape), B * T, H, dv, float(eps), _dtype_code(y),
            _stream(y.device)))
    return out


def gdn_decode_mixer_step(q_raw, k_raw, v_raw, conv_w, conv_state, a, b, A, z, state,
                          dt_bias=None, norm_w=None, out=None, scale=None, eps=1e-6):
    """One token of the whole mixer (see include/gdn.h). q_raw, k_raw: [B,H_k,d_k];
    v_raw, z: [B,H,d_v]; a, b: [B,H]; conv_state: [B,3,2*H_k*d_k + H*d_v] and
    state: [B,H,d_v,d_k] fp32 are updated in place. Returns out [B,H,d_v]."""
    B, Hk, dk = q_raw.shape
    H, dv = v_raw.shape[1], v_raw.shape[2]
    dt = q_raw.dtype
    C = 2 * Hk * dk + H * dv
    if out is None:
        out = torch.empty((B, H, dv), dtype=dt, device=q_raw.device)
    if scale is None:
        scale = dk ** -0.5
    with _on(q_raw.device):
        _check(load().gdn_decode_mixer_step(
            _dev(q_raw, "q_raw", dt), _dev(k_raw, "k_raw", dt, q_raw.shape),
            _dev(v_raw, "v_raw", dt, (B, H, dv)), _dev(conv_w, "conv_w", dt, (C, 4)),
            _dev(conv_state, "conv_state", dt, (B, 3, C)),
            _dev(a, "a", dt, (B, H)), _dev(b, "b", dt, (B, H)), _dev(A, "A", torch.float32, (H,)),
            _dev(dt_bias, "dt_bias", torch.float32, (H,)), _dev(z, "z", dt, (B, H, dv)),
            _dev(norm_w, "norm_w", torch.float32, (dv,)), float(eps),
            _dev(state, "state", torch.float32, (B, H, dv, dk)), _dev(out, "out", dt, (B, H, dv)),
            B, H, Hk, dk, dv, float(scale), _dtype_code(q_raw), _stream(q_raw.device)))
    return out
