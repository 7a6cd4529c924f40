"""The chunkwise algorithm the GPU prefill implements, checked in fp64 on the CPU.

The chunk form of the "Linear Attention" chapter (section "Chunk
implementation of the Delta Rule", stages 1-3) is written out here with numpy,
independently of the oracle, and compared with the oracle's token-by-token
recurrence. Agreement to rounding shows that the chunk reorganisation is an
exact identity (not an approximation), including partial last chunks,
non-zero initial states and strong decay. It is a proof of the algorithm the
kernels implement, not a reference for the kernels.

Notation (state stored as S [d_v, d_k]; the chunk algebra uses M = S^T):
  gamma_i   = sum_{s<=i} g_s inside the chunk
  Gamma_ij  = exp(gamma_i - gamma_j) for j <= i, else 0
  A         = -strict_lower(diag(beta) K K^T * Gamma)
  Tm        = (I - A)^-1
  W         = Tm diag(beta * exp(gamma)) K,    U = Tm diag(beta) V
  Delta     = U - W M
  O         = scale * (diag(exp(gamma)) Q M + lower_incl_diag(Q K^T * Gamma) Delta)
  M'        = exp(gamma_last) M + (diag(exp(gamma_last - gamma)) K)^T Delta
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def decay_matrix(g):
    gam = np.cumsum(g)
    C = len(g)
    i, j = np.meshgrid(np.arange(C), np.arange(C), indexing="ij")
    expo = np.where(j <= i, gam[:, None] - gam[None, :], -np.inf)
    return np.exp(expo), gam


def unit_lower_inverse_rows(A):
    """(I - A)^-1 for strictly lower A, row by row: row i of X = (I-A)^-1 - I
    is A[i,:i] + A[i,:i] X[:i,:i] (the chapter's row recursion)."""
    C = A.shape[0]
    X = np.zeros_like(A)
    for i in range(1, C):
        row = A[i, :i]
        X[i, :i] = row + row @ X[:i, :i]
    return X + np.eye(C)


def chunk_form(q, k, v, g, beta, s0, C, scale):
    T, dk = k.shape
    dv = v.shape[1]
    pad = (-T) % C
    if pad:
        z = lambda x: np.concatenate([x, np.zeros((pad,) + x.shape[1:])], 0)
        q, k, v, g, beta = z(q), z(k), z(v), z(g), z(beta)
    M = s0.T.copy()
    out = np.zeros((T + pad, dv))
    for c in range((T + pad) // C):
        sl = slice(c * C, (c + 1) * C)
        Q, K, V, G, Bt = q[sl], k[sl], v[sl], g[sl], beta[sl]
        Gam, gam = decay_matrix(G)
        A = -np.tril(Bt[:, None] * (K @ K.T) * Gam, -1)
        Tm = unit_lower_inverse_rows(A)
        W = Tm @ ((Bt * np.exp(gam))[:, None] * K)
        U = Tm @ (Bt[:, None] * V)
        Delta = U - W @ M
        P = np.tril(Q @ K.T) * Gam
        out[sl] = scale * ((np.exp(gam)[:, None] * Q) @ M + P @ Delta)
        M = np.exp(gam[-1]) * M + (np.exp(gam[-1] - gam)[:, None] * K).T @ Delta
    return out[:T], M.T


def test_decay_matrix_golden():
    ex = json.load(open(os.path.join(GOLDEN, "decay_matrix_example.json")))
    Gam, gam = decay_matrix(np.array(ex["g"]))
    np.testing.assert_allclose(gam, ex["cumulative_g"], atol=1e-15)
    np.testing.assert_allclose(Gam, np.array(ex["decay"]), atol=1e-15)


def test_row_recursion_is_the_inverse():
    rng = np.random.default_rng(0)
    C = 16
    A = np.tril(rng.standard_normal((C, C)) * 0.3, -1)
    Tm = unit_lower_inverse_rows(A)
    np.testing.assert_allclose(Tm @ (np.eye(C) - A), np.eye(C), atol=1e-12)
    # A is nilpotent, so the Neumann series I + A + ... + A^(C-1) is exact
    np.testing.assert_array_equal(np.linalg.matrix_power(A, C), np.zeros((C, C)))
    series = sum(np.linalg.matrix_power(A, p) for p in range(C))
    np.testing.assert_allclose(series, Tm, atol=1e-12)


@pytest.mark.parametrize("T,d_k,d_v,C", [(37, 5, 7, 8), (64, 8, 8, 16), (100, 16, 12, 64),
                                         (64, 16, 16, 64), (3, 4, 4, 64)])
@pytest.mark.parametrize("strong", [False, True])
def test_chunk_form_equals_recurrence(oracle_mod, T, d_k, d_v, C, strong):
    rng = np.random.default_rng(T * 131 + C)
    q = rng.standard_normal((T, d_k))
    k = rng.standard_normal((T, d_k))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, d_v))
    a = rng.standard_normal(T)
    Ah = 2.0 if strong else 0.05
    g = -Ah * np.logaddexp(0, a)
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    s0 = rng.standard_normal((d_v, d_k)) * 0.5
    scale = d_k ** -0.5
    o_c, s_c = chunk_form(q, k, v, g, beta, s0, C, scale)
    o_r, s_r = oracle_mod.gdn_recurrent(q[None, :, None], k[None, :, None], v[None, :, None],
                                        g[None, :, None], beta[None, :, None],
                                        s0[None, None], scale=scale)
    assert np.abs(o_c - o_r[0, :, 0]).max() <= 1e-12 * max(1.0, np.abs(o_r).max())
    assert np.abs(s_c - s_r[0, 0]).max() <= 1e-12 * max(1.0, np.abs(s_r).max())
