"""Helpers shared by the GPU parity tests: device copies and the error metric.

The metric follows one reading of "max relative error": for every
(sequence, head) slice, ||X - X_ref||_inf / ||X_ref||_inf, and the maximum
over slices, separately for outputs and final states. Elementwise relative
error is undefined where the reference is near zero, so it is not used.
"""
import numpy as np
import torch

TOL_F32 = 1e-4       # fp32 inputs and state
TOL_BF16 = 2e-2      # bf16 inputs, fp32 state

DEV = "cuda:0"


def dev(t):
    return None if t is None else t.to(DEV).contiguous()


def host64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def slice_rel_err(x, ref, axes):
    """max over slices of ||x - ref||_inf / ||ref||_inf, where ``axes`` are the
    axes reduced inside one slice (e.g. the token and channel axes of o)."""
    x, ref = host64(x), np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if x.size == 0:
        return 0.0
    num = np.abs(x - ref).max(axis=axes)
    den = np.abs(ref).max(axis=axes)
    den = np.where(den > 0, den, 1.0)
    if not np.all(np.isfinite(x)):
        return float("inf")
    return float((num / den).max())


def o_err(o, o_ref):
    """o: [B, T, H, d_v] -> per (batch row, head) slices."""
    return slice_rel_err(o, o_ref, axes=(1, 3))


def o_err_packed(o, o_ref, cu):
    """o: [1, T, H, d_v] packed; per (sequence, head) slices."""
    x, ref = host64(o), np.asarray(o_ref, dtype=np.float64)
    errs = [0.0]
    for a, b in zip(cu[:-1], cu[1:]):
        if b > a:
            errs.append(slice_rel_err(x[:, a:b], ref[:, a:b], axes=(1, 3)))
    return max(errs)


def s_err(s, s_ref):
    """states: [N, H, d_v, d_k] -> per (sequence, head) slices."""
    return slice_rel_err(s, s_ref, axes=(2, 3))


def report(name, **errs):
    msg = " ".join(f"{k}={v:.3e}" for k, v in errs.items())
    print(f"[parity] {name}: {msg}", flush=True)
