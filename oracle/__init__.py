"""fp64 CPU oracle of the Gated Delta Rule token mixer - TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the HIP path
(``gated_deltanet_recurrence_amd``) and neither side imports the other. The
arithmetic lives in ``gdn_oracle.c`` (plain C, double precision, token by
token, see the citations there); this module only converts arrays to float64,
slices out the (sequence, head) pairs a caller asks for, and calls the C code.

Pinned by ``tests/test_oracle_pins.py`` against the worked example of the
"Linear Attention" chapter (chunk section), the invariant S_t k_t = v_t for
unit keys and beta = 1, the gate special cases, a closed form for mutually
orthogonal keys (also with grouped query/key heads and with per-channel
decay), the unrolled product form (also per channel), and brute-force checks
of the convolution, norms and gates.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c into oracle/liboracle.so with gcc (-O3, OpenMP).

    No -ffast-math and no -march: the result must be plain IEEE double
    arithmetic and must run on any x86-64 host the library is copied to.
    """
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O3", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.oracle_gdn_recurrent.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _i64p,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_double, ctypes.c_int]
        lib.oracle_gdn_recurrent.restype = ctypes.c_int
        lib.oracle_gdn_recurrent_channel.argtypes = lib.oracle_gdn_recurrent.argtypes
        lib.oracle_gdn_recurrent_channel.restype = ctypes.c_int
        lib.oracle_causal_conv_silu.argtypes = [_dp, _dp, _dp, _i64p, ctypes.c_int,
                                                ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.oracle_causal_conv_silu.restype = ctypes.c_int
        lib.oracle_l2norm_rows.argtypes = [_dp, ctypes.c_int64, ctypes.c_int, ctypes.c_double]
        lib.oracle_l2norm_rows.restype = ctypes.c_int
        lib.oracle_gates.argtypes = [_dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_int64, ctypes.c_int]
        lib.oracle_gates.restype = ctypes.c_int
        lib.oracle_gated_rmsnorm.argtypes = [_dp, _dp, _dp, _dp, ctypes.c_int64,
                                             ctypes.c_int, ctypes.c_double]
        lib.oracle_gated_rmsnorm.restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _f64(x) -> np.ndarray:
    """Any array-like (numpy or a CPU torch tensor of any float dtype) as a
    C-contiguous float64 numpy array."""
    if hasattr(x, "detach"):                      # torch tensor, kept import-free
        x = x.detach().cpu()
        if str(x.dtype) in ("torch.bfloat16", "torch.float16"):
            x = x.float()
        x = x.numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_dp)


def _cu64(cu, n_tokens: int, n_seq: int) -> np.ndarray:
    if cu is None:
        raise ValueError("cu_seqlens required")
    c = np.ascontiguousarray(np.asarray(cu.tolist() if hasattr(cu, "tolist") else cu,
                                        dtype=np.int64))
    if c.shape != (n_seq + 1,) or c[0] != 0 or c[-1] != n_tokens or np.any(np.diff(c) < 0):
        raise ValueError("bad cu_seqlens")
    return c


def expand_heads(x, H: int) -> np.ndarray:
    """The KV head expansion of the "Gated DeltaNet body" layer code ("5. Linear
    Attention" chapter): when there are fewer query/key heads than value heads,
    q and k are repeated along the head axis (axis 2) with repeat_interleave,
    each head H / H_k times in a row, so value head h reads query/key head
    h // (H / H_k)."""
    x = _f64(x)
    Hk = x.shape[2]
    if H % Hk != 0:
        raise ValueError("value heads must be a multiple of query/key heads")
    return x if Hk == H else np.ascontiguousarray(np.repeat(x, H // Hk, axis=2))


def gdn_recurrent(q, k, v, g, beta, s0=None, cu_seqlens=None, scale: float = 1.0,
                  nthreads: int = 0):
    """Gated delta rule over token-major inputs.

    q, k: [B, T, H_k, d_k]; v: [B, T, H, d_v]; g (= log alpha), beta: [B, T, H];
    s0: [N, H, d_v, d_k] or None. With fewer query/key heads than value heads
    (H_k dividing H) q and k are first expanded by ``expand_heads``. With
    ``cu_seqlens`` (N+1 offsets) B must be 1 and the T axis holds N packed
    sequences; otherwise N = B.
    Returns (o [B, T, H, d_v], s_final [N, H, d_v, d_k]) as float64.
    """
    v, g, beta = (_f64(x) for x in (v, g, beta))
    H = v.shape[2]
    q, k = expand_heads(q, H), expand_heads(k, H)
    B, T, _, dk = q.shape
    dv = v.shape[3]
    if k.shape != q.shape or v.shape[:3] != (B, T, H) or g.shape != (B, T, H) \
            or beta.shape != (B, T, H):
        raise ValueError("shape mismatch")
    if cu_seqlens is None:
        N = B
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("cu_seqlens requires B == 1")
        N = len(cu_seqlens) - 1
        cu = _cu64(cu_seqlens, T, N)
    s0a = None if s0 is None else _f64(s0)
    if s0a is not None and s0a.shape != (N, H, dv, dk):
        raise ValueError("bad initial state shape")
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    s1 = np.zeros((N, H, dv, dk), dtype=np.float64)
    rc = _load().oracle_gdn_recurrent(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(s0a), _ptr(s1), _ptr(o), cu.ctypes.data_as(_i64p),
                                      N, H, dk, dv, float(scale), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_gdn_recurrent rejected its arguments")
    return o, s1


def gdn_recurrent_channel(q, k, v, g, beta, s0=None, cu_seqlens=None, scale: float = 1.0,
                          nthreads: int = 0):
    """The gated delta rule with one decay rate per key channel ("6.6 Gated
    DeltaNet" section 6.6.7, the Kimi Linear gate): g = log(alpha) is
    [B, T, H, d_k] and column j of the d_v x d_k state decays by alpha[j]
    before the retrieval. Other arguments and the result as for
    ``gdn_recurrent`` (grouped query/key heads included)."""
    v, g, beta = (_f64(x) for x in (v, g, beta))
    H = v.shape[2]
    q, k = expand_heads(q, H), expand_heads(k, H)
    B, T, _, dk = q.shape
    dv = v.shape[3]
    if k.shape != q.shape or v.shape[:3] != (B, T, H) or g.shape != (B, T, H, dk) \
            or beta.shape != (B, T, H):
        raise ValueError("shape mismatch")
    if cu_seqlens is None:
        N = B
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("cu_seqlens requires B == 1")
        N = len(cu_seqlens) - 1
        cu = _cu64(cu_seqlens, T, N)
    s0a = None if s0 is None else _f64(s0)
    if s0a is not None and s0a.shape != (N, H, dv, dk):
        raise ValueError("bad initial state shape")
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    s1 = np.zeros((N, H, dv, dk), dtype=np.float64)
    rc = _load().oracle_gdn_recurrent_channel(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                              _ptr(s0a), _ptr(s1), _ptr(o),
                                              cu.ctypes.data_as(_i64p), N, H, dk, dv,
                                              float(scale), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_gdn_recurrent_channel rejected its arguments")
    return o, s1


def gdn_recurrent_heads(q, k, v, g, beta, heads: Sequence[int], s0=None, cu_seqlens=None,
                        scale: float = 1.0, seqs: Optional[Sequence[int]] = None,
                        nthreads: int = 0):
    """The recurrence for a subset of heads (and, for unpacked batches, of
    batch rows ``seqs``). Returns (o [b', T, h', d_v], s_final [n', h', d_v, d_k])
    for the selected rows/sequences and heads, in the order given."""
    heads = list(heads)
    grp = v.shape[2] // q.shape[2]            # value heads per query/key head
    kheads = [h // grp for h in heads]         # the query/key head of each, as expanded
    if cu_seqlens is None:
        rows = list(range(q.shape[0])) if seqs is None else list(seqs)
        sl = lambda x: x[rows][:, :, heads]
        slk = lambda x: x[rows][:, :, kheads]
        s0s = None if s0 is None else s0[rows][:, heads]
        return gdn_recurrent(slk(q), slk(k), sl(v), sl(g), sl(beta), s0s, None, scale, nthreads)
    cu = [int(c) for c in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
    seq_ids = list(range(len(cu) - 1)) if seqs is None else list(seqs)
    outs, states = [], []
    for n in seq_ids:
        a, b = cu[n], cu[n + 1]
        sl = lambda x: x[:, a:b][:, :, heads]
        slk = lambda x: x[:, a:b][:, :, kheads]
        s0n = None if s0 is None else s0[n:n + 1][:, heads]
        o, s1 = gdn_recurrent(slk(q), slk(k), sl(v), sl(g), sl(beta), s0n, None, scale, nthreads)
        outs.append(o)
        states.append(s1)
    return outs, np.concatenate(states, axis=0)


def causal_conv_silu(x, w, cu_seqlens=None):
    """Depthwise causal conv (zero left history per sequence) + SiLU.
    x: [B, T, C]; w: [C, K]. With cu_seqlens, B must be 1."""
    x, w = _f64(x), _f64(w)
    B, T, C = x.shape
    K = w.shape[1]
    if cu_seqlens is None:
        N, cu = B, np.arange(B + 1, dtype=np.int64) * T
    else:
        N = len(cu_seqlens) - 1
        cu = _cu64(cu_seqlens, T, N)
    y = np.zeros_like(x)
    rc = _load().oracle_causal_conv_silu(_ptr(x), _ptr(w), _ptr(y), cu.ctypes.data_as(_i64p),
                                         N, C, K, 0)
    if rc != 0:
        raise ValueError("oracle_causal_conv_silu rejected its arguments")
    return y


def l2norm(x, eps: float = 1e-6):
    """x / sqrt(sum(x^2) + eps) along the last axis."""
    x = _f64(x).copy()
    d = x.shape[-1]
    rc = _load().oracle_l2norm_rows(_ptr(x), x.size // d, d, float(eps))
    if rc != 0:
        raise ValueError("oracle_l2norm_rows rejected its arguments")
    return x


def gates(a, b, A, dt_bias=None):
    """(g = -A*softplus(a + dt_bias), beta = sigmoid(b)); a, b: [..., H]."""
    a, b, A = _f64(a), _f64(b), _f64(A)
    H = a.shape[-1]
    dtb = None if dt_bias is None else _f64(dt_bias)
    g = np.zeros_like(a)
    beta = np.zeros_like(a)
    rc = _load().oracle_gates(_ptr(a), _ptr(b), _ptr(A), _ptr(dtb), _ptr(g), _ptr(beta),
                              a.size // H, H)
    if rc != 0:
        raise ValueError("oracle_gates rejected its arguments")
    return g, beta


def gated_rmsnorm(y, z, w=None, eps: float = 1e-6):
    """w * y / sqrt(mean(y^2) + eps) * silu(z) along the last axis."""
    y, z = _f64(y), _f64(z)
    wa = None if w is None else _f64(w)
    d = y.shape[-1]
    out = np.zeros_like(y)
    rc = _load().oracle_gated_rmsnorm(_ptr(y), _ptr(z), _ptr(wa), _ptr(out), y.size // d, d,
                                      float(eps))
    if rc != 0:
        raise ValueError("oracle_gated_rmsnorm rejected its arguments")
    return out


def mixer(q_raw, k_raw, v_raw, z, a, b, conv_w, A, dt_bias=None, norm_w=None,
          scale: float = 1.0, eps: float = 1e-6, cu_seqlens=None,
          heads: Optional[Sequence[int]] = None, rows: Optional[Sequence[int]] = None,
          return_intermediates: bool = False):
    """The whole token mixer from pre-projected inputs, in the order of the
    "Gated DeltaNet body" of the Linear Attention chapter: causal conv + SiLU
    over the concatenated q|k|v channels, split, L2-norm of q and k (eps 1e-6),
    gates, the KV head expansion when q and k have fewer heads than v, the
    recurrence with ``scale``, then the gated RMSNorm with z.

    q_raw, k_raw: [B, T, H_k, d_k]; v_raw, z: [B, T, H, d_v]; a, b: [B, T, H];
    conv_w: [2 H_k d_k + H d_v, 4] in channel order q, k, v. ``heads``/``rows``
    restrict the computation to some value heads / batch rows (channels of
    other heads never mix with these ones). Returns out [b', T, h', d_v] (and
    the intermediates when asked; q and k there are per query/key head of the
    selection, before the expansion).
    """
    B, T, Hk, dk = q_raw.shape
    H, dv = v_raw.shape[2], v_raw.shape[3]
    if H % Hk != 0:
        raise ValueError("value heads must be a multiple of query/key heads")
    grp = H // Hk
    heads = list(range(H)) if heads is None else list(heads)
    kheads = sorted({h // grp for h in heads})     # query/key heads the selection reads
    rows = list(range(B)) if rows is None else list(rows)
    if cu_seqlens is not None and rows != [0]:
        raise ValueError("packed sequences use B == 1")
    cw = _f64(conv_w)
    ch_q = [kh * dk + j for kh in kheads for j in range(dk)]
    ch_k = [Hk * dk + kh * dk + j for kh in kheads for j in range(dk)]
    ch_v = [2 * Hk * dk + h * dv + j for h in heads for j in range(dv)]
    w_sel = cw[ch_q + ch_k + ch_v]
    sel = lambda x: _f64(x)[rows][:, :, heads]
    selk = lambda x: _f64(x)[rows][:, :, kheads]
    qs, ks, vs = selk(q_raw), selk(k_raw), sel(v_raw)
    nb, nh, nk = len(rows), len(heads), len(kheads)
    mixed = np.concatenate([qs.reshape(nb, T, nk * dk), ks.reshape(nb, T, nk * dk),
                            vs.reshape(nb, T, nh * dv)], axis=2)
    conv = causal_conv_silu(mixed, w_sel, cu_seqlens)
    qc = conv[:, :, :nk * dk].reshape(nb, T, nk, dk)
    kc = conv[:, :, nk * dk:2 * nk * dk].reshape(nb, T, nk, dk)
    vc = conv[:, :, 2 * nk * dk:].reshape(nb, T, nh, dv)
    qn, kn = l2norm(qc), l2norm(kc)
    # the expansion, restricted to the selected value heads
    pick = [kheads.index(h // grp) for h in heads]
    qe, ke = qn[:, :, pick], kn[:, :, pick]
    Asel = _f64(A)[heads]
    dtb = None if dt_bias is None else _f64(dt_bias)[heads]
    g, beta = gates(sel(a), sel(b), Asel, dtb)
    y, s1 = gdn_recurrent(qe, ke, vc, g, beta, None, cu_seqlens, scale)
    out = gated_rmsnorm(y, sel(z), norm_w, eps)
    if return_intermediates:
        return out, dict(q=qn, k=kn, v=vc, g=g, beta=beta, y=y, s_final=s1)
    return out


def mixer_decode_step(q_raw, k_raw, v_raw, z, a, b, conv_w, conv_state, A, state,
                      dt_bias=None, norm_w=None, scale: float = 1.0, eps: float = 1e-6):
    """One token of the token mixer for B sequences, in the order of the
    inference flow of "6.6 Gated DeltaNet" (section 6.6.8): the new token's
    q, k, v and gates, the state update, the read with q, the gated RMSNorm.
    The short convolution keeps, per channel, the inputs of the three previous
    tokens (the convolution state a deployment caches beside the matrix state,
    "Overwrite and Forget" section 13.4); the output for the new token is the
    causal convolution over that window, exactly as ``causal_conv_silu`` would
    produce it for the last token of the sequence.

    q_raw, k_raw: [B, H_k, d_k]; v_raw, z: [B, H, d_v]; a, b: [B, H];
    conv_w: [C, 4], C = 2 H_k d_k + H d_v (channel order q, k, v);
    conv_state: [B, 3, C], oldest input first; state: [B, H, d_v, d_k].
    Returns (out [B, H, d_v], new state, new conv_state), float64.
    """
    qr, kr, vr = _f64(q_raw), _f64(k_raw), _f64(v_raw)
    B, Hk, dk = qr.shape
    H, dv = vr.shape[1], vr.shape[2]
    x_t = np.concatenate([qr.reshape(B, -1), kr.reshape(B, -1), vr.reshape(B, -1)], axis=1)
    window = np.concatenate([_f64(conv_state), x_t[:, None, :]], axis=1)     # [B, 4, C]
    conv = causal_conv_silu(window, conv_w)[:, 3]                             # [B, C]
    q = l2norm(conv[:, :Hk * dk].reshape(B, 1, Hk, dk))
    k = l2norm(conv[:, Hk * dk:2 * Hk * dk].reshape(B, 1, Hk, dk))
    v = conv[:, 2 * Hk * dk:].reshape(B, 1, H, dv)
    g, beta = gates(_f64(a)[:, None], _f64(b)[:, None], A, dt_bias)
    y, s1 = gdn_recurrent(q, k, v, g, beta, _f64(state), None, scale)
    out = gated_rmsnorm(y[:, 0], z, norm_w, eps)
    return out, s1, np.ascontiguousarray(window[:, 1:])
