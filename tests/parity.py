"""Helpers shared by the GPU parity tests: device copies and the error metrics.

The bar follows one reading of "max relative error": for every (sequence,
head) slice, ||X - X_ref||_inf / ||X_ref||_inf, and the maximum over slices,
separately for outputs and final states. Elementwise relative error is
undefined where the reference is near zero, so it is not the bar.

Two finer figures are computed beside it for every output comparison and
printed by ``report``:

* ``row``: the same ratio per token row (one (token, head) output vector),
  ||o_t - o_ref_t||_inf / max(||o_ref_t||_inf, ROW_FLOOR * ||o_ref||_inf of
  the slice). The floor keeps rows whose reference is almost zero (a query
  nearly orthogonal to everything stored) from dividing by ~0; a row that is
  entirely wrong still shows up unless its reference is below 1/16 of the
  slice's largest value, where the bf16 output's own rounding of the
  slice's scale is already a large part of it.
* ``allclose``: the fraction of elements outside
  |x - ref| <= tol * ||ref||_inf(slice) + tol * |ref| (numpy's allclose
  with atol scaled to the slice), for the bf16 or fp32 tolerance.
"""
import numpy as np
import torch

TOL_F32 = 1e-4       # fp32 inputs and state
TOL_BF16 = 2e-2      # bf16 inputs, fp32 state
ROW_FLOOR = 1.0 / 16

DEV = "cuda:0"


class Err(float):
    """A slice error (the bar) that also carries the finer figures."""
    row: float = 0.0
    allclose: float = 0.0
    row_raw: float = 0.0


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


def row_metrics(x, ref, tol):
    """o-shaped [B, T, H, d_v] arrays: (row error with the floor, row error
    without it, fraction of elements outside the slice-scaled allclose)."""
    x, ref = host64(x), np.asarray(ref, dtype=np.float64)
    if x.size == 0:
        return 0.0, 0.0, 0.0
    if not np.all(np.isfinite(x)):
        return float("inf"), float("inf"), 1.0
    diff = np.abs(x - ref)
    slice_max = np.abs(ref).max(axis=(1, 3), keepdims=True)          # [B, 1, H, 1]
    row_max = np.abs(ref).max(axis=3, keepdims=True)                  # [B, T, H, 1]
    row_num = diff.max(axis=3, keepdims=True)
    den = np.maximum(row_max, ROW_FLOOR * slice_max)
    den = np.where(den > 0, den, 1.0)
    raw = np.where(row_max > 0, row_max, 1.0)
    viol = diff > tol * slice_max + tol * np.abs(ref)
    return float((row_num / den).max()), float((row_num / raw).max()), float(viol.mean())


def _err(x, ref, axes, tol):
    e = Err(slice_rel_err(x, ref, axes))
    e.row, e.row_raw, e.allclose = row_metrics(x, ref, tol)
    return e


def o_err(o, o_ref, tol=TOL_BF16):
    """o: [B, T, H, d_v] -> per (batch row, head) slices, with the row and
    allclose figures attached."""
    return _err(o, o_ref, (1, 3), tol)


def o_err_packed(o, o_ref, cu, tol=TOL_BF16):
    """o: [1, T, H, d_v] packed; per (sequence, head) slices."""
    x, ref = host64(o), np.asarray(o_ref, dtype=np.float64)
    worst = Err(0.0)
    for a, b in zip(cu[:-1], cu[1:]):
        if b > a:
            e = _err(x[:, a:b], ref[:, a:b], (1, 3), tol)
            if float(e) >= float(worst):
                e.row, e.row_raw, e.allclose = (max(e.row, worst.row),
                                                max(e.row_raw, worst.row_raw),
                                                max(e.allclose, worst.allclose))
                worst = e
            else:
                worst.row = max(e.row, worst.row)
                worst.row_raw = max(e.row_raw, worst.row_raw)
                worst.allclose = max(e.allclose, worst.allclose)
    return worst


def s_err(s, s_ref):
    """states: [N, H, d_v, d_k] -> per (sequence, head) slices."""
    return slice_rel_err(s, s_ref, axes=(2, 3))


# every report of the session, printed again in pytest's terminal summary
# (tests/conftest.py), so that the figures reach the log even with -q
REPORTS = []


def report(name, **errs):
    parts = []
    for k, v in errs.items():
        parts.append(f"{k}={float(v):.3e}")
        if isinstance(v, Err):
            parts.append(f"{k}_row={v.row:.3e} {k}_row_nofloor={v.row_raw:.3e} "
                         f"{k}_allclose_viol={v.allclose:.2e}")
    line = f"[parity] {name}: {' '.join(parts)}"
    REPORTS.append(line)
    print(line, flush=True)
