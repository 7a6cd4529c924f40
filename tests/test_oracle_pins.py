"""Pins of the fp64 oracle to facts the pages and plain mathematics fix.

Each test checks the oracle against something other than itself: a worked
example printed on the pages, an invariant stated there, a closed form, an
independent algebraic form of the recurrence, or a library routine that the
operation reduces to. Every check uses deliberately asymmetric shapes
(d_v != d_k) so that a transposed state, a swapped operand, a misplaced decay
or a dropped term fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(rng, T, H, dk, dv, unit_keys=True):
    q = rng.standard_normal((1, T, H, dk))
    k = rng.standard_normal((1, T, H, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, H, dv))
    g = np.log(rng.uniform(0.5, 1.0, (1, T, H)))
    beta = rng.uniform(0.0, 1.0, (1, T, H))
    return q, k, v, g, beta


# --- Worked example printed on the pages -----------------------------------

def test_worked_example_identity_keys(oracle_mod):
    """"Linear Attention" chapter, chunk section running example: d=2,
    K=V=I, beta=1, g=0, q=k gives o=I unscaled, o=I/sqrt(2) scaled and the
    end state I; the state after token 0 is e0 e0^T."""
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_identity_keys.json")))
    q = np.array(ex["q"])[None, :, None, :]
    k = np.array(ex["k"])[None, :, None, :]
    v = np.array(ex["v"])[None, :, None, :]
    g = np.array(ex["g"])[None, :, None]
    beta = np.array(ex["beta"])[None, :, None]
    o, s = oracle_mod.gdn_recurrent(q, k, v, g, beta, scale=1.0)
    np.testing.assert_allclose(o[0, :, 0], np.array(ex["o_unscaled"]), atol=1e-15)
    np.testing.assert_allclose(s[0, 0], np.array(ex["state_end"]), atol=1e-15)
    o, _ = oracle_mod.gdn_recurrent(q, k, v, g, beta, scale=ex["scale"])
    np.testing.assert_allclose(o[0, :, 0], np.array(ex["o_scaled"]), atol=1e-15)
    _, s1 = oracle_mod.gdn_recurrent(q[:, :1], k[:, :1], v[:, :1], g[:, :1], beta[:, :1])
    np.testing.assert_allclose(s1[0, 0], np.array(ex["state_per_step"][0]), atol=1e-15)


# --- Invariants stated on the pages ----------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_overwrite_invariant(oracle_mod, seed):
    """"Overwrite and Forget" sections 2.2 and 4.3: for a unit key the new
    state maps k_t to (1 - beta_t) * (alpha_t S_{t-1} k_t) + beta_t v_t; with
    beta_t = 1 that is exactly v_t, whatever alpha_t and S_{t-1} are."""
    rng = np.random.default_rng(seed)
    H, dk, dv, T = 2, 7, 5, 9
    q, k, v, g, beta = _rand_case(rng, T, H, dk, dv)
    s0 = rng.standard_normal((1, H, dv, dk))
    for t in range(T):
        _, s_prev = oracle_mod.gdn_recurrent(q[:, :t], k[:, :t], v[:, :t], g[:, :t],
                                             beta[:, :t], s0)
        _, s_t = oracle_mod.gdn_recurrent(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1],
                                          g[:, :t + 1], beta[:, :t + 1], s0)
        for h in range(H):
            kt, vt = k[0, t, h], v[0, t, h]
            a, b = math.exp(g[0, t, h]), beta[0, t, h]
            lhs = s_t[0, h] @ kt
            rhs = (1 - b) * a * (s_prev[0, h] @ kt) + b * vt
            np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    # beta = 1 everywhere: every step stores v_t exactly at k_t
    beta1 = np.ones_like(beta)
    for t in range(T):
        _, s_t = oracle_mod.gdn_recurrent(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1],
                                          g[:, :t + 1], beta1[:, :t + 1], s0)
        for h in range(H):
            np.testing.assert_allclose(s_t[0, h] @ k[0, t, h], v[0, t, h], atol=1e-12)


def test_zero_update_gate(oracle_mod):
    """beta = 0 writes nothing: with alpha = 1 the state is unchanged, otherwise
    it is only scaled by alpha ("Overwrite and Forget" sections 2 and 4.1)."""
    rng = np.random.default_rng(3)
    H, dk, dv, T = 3, 6, 4, 5
    q, k, v, g, beta = _rand_case(rng, T, H, dk, dv)
    s0 = rng.standard_normal((1, H, dv, dk))
    zero = np.zeros_like(beta)
    _, s = oracle_mod.gdn_recurrent(q, k, v, np.zeros_like(g), zero, s0)
    np.testing.assert_array_equal(s, s0)
    _, s = oracle_mod.gdn_recurrent(q, k, v, g, zero, s0)
    decay = np.exp(g[0].sum(axis=0))                    # product of alphas per head
    np.testing.assert_allclose(s[0], s0[0] * decay[:, None, None], rtol=1e-13)


# --- Closed forms -----------------------------------------------------------

def _orthonormal_keys(rng, T, dk):
    m = rng.standard_normal((dk, dk))
    qm, _ = np.linalg.qr(m)
    return qm[:, :T].T.copy()             # T mutually orthonormal rows


@pytest.mark.parametrize("seed", [0, 1])
def test_orthogonal_keys_closed_form(oracle_mod, seed):
    """With mutually orthogonal unit keys and a zero initial state nothing is
    ever retrieved (S_{t-1} k_t = 0), so the delta rule reduces to decayed
    additive writes: o_t = scale * sum_{i<=t} (prod_{s=i+1..t} alpha_s)
    beta_i v_i (k_i . q_t). Brute force, O(T^2)."""
    rng = np.random.default_rng(seed)
    T, dk, dv, H = 6, 8, 3, 2
    q = rng.standard_normal((1, T, H, dk))
    k = np.stack([_orthonormal_keys(rng, T, dk) for _ in range(H)], axis=1)[None]
    v = rng.standard_normal((1, T, H, dv))
    g = np.log(rng.uniform(0.3, 1.0, (1, T, H)))
    beta = rng.uniform(0.1, 1.0, (1, T, H))
    scale = 0.37
    o, s = oracle_mod.gdn_recurrent(q, k, v, g, beta, scale=scale)
    for h in range(H):
        for t in range(T):
            ref = np.zeros(dv)
            for i in range(t + 1):
                dec = math.exp(g[0, i + 1:t + 1, h].sum())
                ref += dec * beta[0, i, h] * v[0, i, h] * (k[0, i, h] @ q[0, t, h])
            np.testing.assert_allclose(o[0, t, h], scale * ref, rtol=1e-12, atol=1e-13)
        # the end state is the decayed sum of outer products v_i k_i^T
        ref_s = sum(math.exp(g[0, i + 1:, h].sum()) * beta[0, i, h] *
                    np.outer(v[0, i, h], k[0, i, h]) for i in range(T))
        np.testing.assert_allclose(s[0, h], ref_s, rtol=1e-12, atol=1e-13)


def test_grouped_heads_closed_form(oracle_mod):
    """Grouped heads ("Linear Attention" chapter, "Gated DeltaNet body" layer
    code: q and k repeated along the head axis with repeat_interleave): with
    H_k = 2 query/key heads and H = 4 value heads, value head h reads key
    head h // 2 (heads 0, 1 -> 0; 2, 3 -> 1), checked against the orthogonal-
    keys closed form written with that index."""
    rng = np.random.default_rng(12)
    T, dk, dv, H, Hk = 5, 6, 3, 4, 2
    q = rng.standard_normal((1, T, Hk, dk))
    k = np.stack([_orthonormal_keys(rng, T, dk) for _ in range(Hk)], axis=1)[None]
    v = rng.standard_normal((1, T, H, dv))
    g = np.log(rng.uniform(0.3, 1.0, (1, T, H)))
    beta = rng.uniform(0.1, 1.0, (1, T, H))
    o, s = oracle_mod.gdn_recurrent(q, k, v, g, beta, scale=1.0)
    assert o.shape == (1, T, H, dv) and s.shape == (1, H, dv, dk)
    for h in range(H):
        kh = h // (H // Hk)
        for t in range(T):
            ref = np.zeros(dv)
            for i in range(t + 1):
                dec = math.exp(g[0, i + 1:t + 1, h].sum())
                ref += dec * beta[0, i, h] * v[0, i, h] * (k[0, i, kh] @ q[0, t, kh])
            np.testing.assert_allclose(o[0, t, h], ref, rtol=1e-12, atol=1e-13)
    # the sampled-heads form picks the same query/key heads
    o2, s2 = oracle_mod.gdn_recurrent_heads(q, k, v, g, beta, heads=[3, 0], scale=1.0)
    np.testing.assert_array_equal(o2, o[:, :, [3, 0]])
    np.testing.assert_array_equal(s2, s[:, [3, 0]])


def test_linear_attention_special_case(oracle_mod):
    """alpha = 1, beta = 1 and orthonormal keys: exactly causal linear attention
    o_t = sum_{i<=t} v_i (k_i . q_t) ("Overwrite and Forget" section 1)."""
    rng = np.random.default_rng(7)
    T, dk, dv = 5, 5, 2
    q = rng.standard_normal((1, T, 1, dk))
    k = _orthonormal_keys(rng, T, dk)[None, :, None, :]
    v = rng.standard_normal((1, T, 1, dv))
    o, _ = oracle_mod.gdn_recurrent(q, k, v, np.zeros((1, T, 1)), np.ones((1, T, 1)))
    scores = np.tril(q[0, :, 0] @ k[0, :, 0].T)          # [t, i] = k_i . q_t, i <= t
    np.testing.assert_allclose(o[0, :, 0], scores @ v[0, :, 0], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_product_form(oracle_mod, seed):
    """"Overwrite and Forget" section 7: with A_t = alpha_t (I - beta_t k_t k_t^T)
    and B_t = beta_t v_t k_t^T, S_t = S_0 A_1...A_t + sum_i B_i A_{i+1}...A_t.
    Dense d x d transition matrices, arbitrary (non-unit) keys, non-zero S_0."""
    rng = np.random.default_rng(seed)
    T, dk, dv, H = 7, 5, 3, 2
    q, k, v, g, beta = _rand_case(rng, T, H, dk, dv, unit_keys=False)
    s0 = rng.standard_normal((1, H, dv, dk))
    scale = 0.81
    o, s = oracle_mod.gdn_recurrent(q, k, v, g, beta, s0, scale=scale)
    for h in range(H):
        As = [math.exp(g[0, t, h]) * (np.eye(dk) - beta[0, t, h] *
                                      np.outer(k[0, t, h], k[0, t, h])) for t in range(T)]
        Bs = [beta[0, t, h] * np.outer(v[0, t, h], k[0, t, h]) for t in range(T)]
        for t in range(T):
            prod = lambda a, b: np.linalg.multi_dot([np.eye(dk)] + As[a:b] + [np.eye(dk)])
            s_t = s0[0, h] @ prod(0, t + 1)
            for i in range(t + 1):
                s_t = s_t + Bs[i] @ prod(i + 1, t + 1)
            np.testing.assert_allclose(o[0, t, h], scale * (s_t @ q[0, t, h]),
                                       rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(s[0, h], s_t, rtol=1e-11, atol=1e-12)


# --- Sequence handling ------------------------------------------------------

def test_split_resume_and_packing(oracle_mod):
    """Running T1 tokens, then T2 tokens from the returned state, equals one
    run of T1+T2 tokens (the prefill -> decode hand-off of "Overwrite and
    Forget" section 7); packed sequences equal separate batch rows; an empty
    sequence returns its initial state untouched."""
    rng = np.random.default_rng(11)
    T, H, dk, dv = 12, 2, 6, 4
    q, k, v, g, beta = _rand_case(rng, T, H, dk, dv)
    s0 = rng.standard_normal((1, H, dv, dk))
    o_all, s_all = oracle_mod.gdn_recurrent(q, k, v, g, beta, s0, scale=0.5)
    o1, s1 = oracle_mod.gdn_recurrent(q[:, :5], k[:, :5], v[:, :5], g[:, :5], beta[:, :5],
                                      s0, scale=0.5)
    o2, s2 = oracle_mod.gdn_recurrent(q[:, 5:], k[:, 5:], v[:, 5:], g[:, 5:], beta[:, 5:],
                                      s1, scale=0.5)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o_all, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(s2, s_all, rtol=1e-13, atol=1e-14)
    # packed: sequences of 5, 0, 7 tokens
    cu = [0, 5, 5, 12]
    s0p = rng.standard_normal((3, H, dv, dk))
    o_p, s_p = oracle_mod.gdn_recurrent(q, k, v, g, beta, s0p, cu_seqlens=cu, scale=0.5)
    oa, sa = oracle_mod.gdn_recurrent(q[:, :5], k[:, :5], v[:, :5], g[:, :5], beta[:, :5],
                                      s0p[:1], scale=0.5)
    ob, sb = oracle_mod.gdn_recurrent(q[:, 5:], k[:, 5:], v[:, 5:], g[:, 5:], beta[:, 5:],
                                      s0p[2:], scale=0.5)
    np.testing.assert_array_equal(o_p[:, :5], oa)
    np.testing.assert_array_equal(o_p[:, 5:], ob)
    np.testing.assert_array_equal(s_p[0], sa[0])
    np.testing.assert_array_equal(s_p[1], s0p[1])
    np.testing.assert_array_equal(s_p[2], sb[0])


# --- Prologue / epilogue pieces --------------------------------------------

def test_causal_conv_against_numpy_convolve(oracle_mod):
    """"Linear Attention" chapter, causal conv section: a depthwise causal
    convolution with 4 taps and zero left padding is, per channel, the first T
    samples of the full linear convolution with the flipped kernel; then SiLU
    (x * sigmoid(x)). Also: the history restarts at each packed sequence."""
    rng = np.random.default_rng(5)
    T, C, K = 11, 6, 4
    x = rng.standard_normal((2, T, C))
    w = rng.standard_normal((C, K))
    y = oracle_mod.causal_conv_silu(x, w)
    for b in range(2):
        for c in range(C):
            pre = np.convolve(x[b, :, c], w[c, ::-1])[:T]
            np.testing.assert_allclose(y[b, :, c], pre * expit(pre), rtol=1e-13, atol=1e-14)
    # the page's window picture: output 0 sees only x0 through the last tap
    pre0 = w[:, 3] * x[0, 0]
    np.testing.assert_allclose(y[0, 0], pre0 * expit(pre0), rtol=1e-13)
    # packed sequences [0,4) and [4,11) behave like two separate rows
    yp = oracle_mod.causal_conv_silu(x[:1], w, cu_seqlens=[0, 4, T])
    np.testing.assert_allclose(yp[0, :4], oracle_mod.causal_conv_silu(x[:1, :4], w)[0])
    np.testing.assert_allclose(yp[0, 4:], oracle_mod.causal_conv_silu(x[:1, 4:], w)[0])


def test_l2norm_and_gates(oracle_mod):
    rng = np.random.default_rng(6)
    x = rng.standard_normal((4, 3, 16)) * 3
    n = np.linalg.norm(oracle_mod.l2norm(x), axis=-1)
    ref = np.linalg.norm(x, axis=-1) / np.sqrt(np.linalg.norm(x, axis=-1) ** 2 + 1e-6)
    np.testing.assert_allclose(n, ref, rtol=1e-14)
    assert np.all(np.abs(n - 1) < 1e-6)
    # direction is kept
    cos = (oracle_mod.l2norm(x) * x).sum(-1) / np.linalg.norm(x, axis=-1)
    np.testing.assert_allclose(cos, n, rtol=1e-13)
    a = rng.standard_normal((5, 4)) * 4
    b = rng.standard_normal((5, 4)) * 4
    A = rng.uniform(0.5, 2.0, 4)
    dtb = rng.standard_normal(4)
    g, beta = oracle_mod.gates(a, b, A, dtb)
    np.testing.assert_allclose(g, -A * np.logaddexp(0.0, a + dtb), rtol=1e-14)
    np.testing.assert_allclose(beta, expit(b), rtol=1e-14)
    g0, _ = oracle_mod.gates(a, b, A, None)
    np.testing.assert_allclose(g0, -A * np.logaddexp(0.0, a), rtol=1e-14)
    assert np.all(g < 0) and np.all((beta > 0) & (beta < 1))


def test_gated_rmsnorm(oracle_mod):
    """"Linear Attention" chapter, gated RMSNorm: out = w * norm(y) * silu(z);
    dividing out by w * silu(z) leaves a vector parallel to y whose RMS is
    sqrt(m / (m + eps)), m = mean(y^2)."""
    rng = np.random.default_rng(8)
    d = 12
    y = rng.standard_normal((7, d)) * 0.01     # small rows make eps visible
    z = rng.standard_normal((7, d))
    w = rng.uniform(0.5, 1.5, d)
    eps = 1e-6
    out = oracle_mod.gated_rmsnorm(y, z, w, eps)
    r = out / (w * z * expit(z))
    m = (y ** 2).mean(-1)
    np.testing.assert_allclose(np.sqrt((r ** 2).mean(-1)), np.sqrt(m / (m + eps)), rtol=1e-12)
    np.testing.assert_allclose(r * np.sqrt(m + eps)[:, None], y, rtol=1e-12)
    np.testing.assert_allclose(oracle_mod.gated_rmsnorm(y, z, None, eps),
                               out / w, rtol=1e-13)


def test_mixer_composition(oracle_mod):
    """The mixer is: conv+SiLU over q|k|v channels -> split -> L2-norm q,k ->
    gates -> recurrence -> gated RMSNorm, rebuilt here from numpy/scipy
    pieces (np.convolve, expit, logaddexp) around the pinned recurrence, and
    head/row sampling returns exactly the full computation's slice."""
    rng = np.random.default_rng(9)
    B, T, H, dk, dv = 2, 9, 3, 4, 5
    qr = rng.standard_normal((B, T, H, dk))
    kr = rng.standard_normal((B, T, H, dk))
    vr = rng.standard_normal((B, T, H, dv))
    z = rng.standard_normal((B, T, H, dv))
    a = rng.standard_normal((B, T, H))
    b = rng.standard_normal((B, T, H))
    w = rng.standard_normal((H * (2 * dk + dv), 4)) * 0.5
    A = rng.uniform(0.5, 2, H)
    scale = dk ** -0.5
    out = oracle_mod.mixer(qr, kr, vr, z, a, b, w, A, scale=scale)

    def conv(x, wc):
        pre = np.convolve(x, wc[::-1])[:T]
        return pre * expit(pre)
    mixed = np.concatenate([qr.reshape(B, T, -1), kr.reshape(B, T, -1), vr.reshape(B, T, -1)], 2)
    y = np.stack([np.stack([conv(mixed[bb, :, c], w[c]) for c in range(mixed.shape[2])], 1)
                  for bb in range(B)])
    q = y[:, :, :H * dk].reshape(B, T, H, dk)
    k = y[:, :, H * dk:2 * H * dk].reshape(B, T, H, dk)
    v = y[:, :, 2 * H * dk:].reshape(B, T, H, dv)
    q = q / np.sqrt((q ** 2).sum(-1, keepdims=True) + 1e-6)
    k = k / np.sqrt((k ** 2).sum(-1, keepdims=True) + 1e-6)
    g = -A * np.logaddexp(0, a)
    beta = expit(b)
    core, _ = oracle_mod.gdn_recurrent(q, k, v, g, beta, scale=scale)
    ref = core / np.sqrt((core ** 2).mean(-1, keepdims=True) + 1e-6) * z * expit(z)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
    part = oracle_mod.mixer(qr, kr, vr, z, a, b, w, A, scale=scale, heads=[2, 0], rows=[1])
    np.testing.assert_allclose(part, out[[1]][:, :, [2, 0]], rtol=1e-13, atol=1e-14)


def test_mixer_composition_grouped_heads(oracle_mod):
    """The mixer with H_k = 2 query/key heads and H = 4 value heads: conv
    channels are 2 H_k d_k of q|k then H d_v of v, the gates are per value
    head, and value head h reads the normalised q, k of head h // 2; rebuilt
    from numpy/scipy pieces around the pinned recurrence."""
    rng = np.random.default_rng(10)
    B, T, H, Hk, dk, dv = 1, 8, 4, 2, 4, 3
    qr = rng.standard_normal((B, T, Hk, dk))
    kr = rng.standard_normal((B, T, Hk, dk))
    vr = rng.standard_normal((B, T, H, dv))
    z = rng.standard_normal((B, T, H, dv))
    a = rng.standard_normal((B, T, H))
    b = rng.standard_normal((B, T, H))
    w = rng.standard_normal((2 * Hk * dk + H * dv, 4)) * 0.5
    A = rng.uniform(0.5, 2, H)
    out = oracle_mod.mixer(qr, kr, vr, z, a, b, w, A, scale=0.5)

    def conv(x, wc):
        pre = np.convolve(x, wc[::-1])[:T]
        return pre * expit(pre)
    mixed = np.concatenate([qr.reshape(B, T, -1), kr.reshape(B, T, -1), vr.reshape(B, T, -1)], 2)
    y = np.stack([conv(mixed[0, :, c], w[c]) for c in range(mixed.shape[2])], 1)[None]
    q = y[:, :, :Hk * dk].reshape(B, T, Hk, dk)
    k = y[:, :, Hk * dk:2 * Hk * dk].reshape(B, T, Hk, dk)
    v = y[:, :, 2 * Hk * dk:].reshape(B, T, H, dv)
    q = q / np.sqrt((q ** 2).sum(-1, keepdims=True) + 1e-6)
    k = k / np.sqrt((k ** 2).sum(-1, keepdims=True) + 1e-6)
    idx = [h // (H // Hk) for h in range(H)]
    core, _ = oracle_mod.gdn_recurrent(q[:, :, idx], k[:, :, idx], v, -A * np.logaddexp(0, a),
                                       expit(b), scale=0.5)
    ref = core / np.sqrt((core ** 2).mean(-1, keepdims=True) + 1e-6) * z * expit(z)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
    part = oracle_mod.mixer(qr, kr, vr, z, a, b, w, A, scale=0.5, heads=[3, 1])
    np.testing.assert_allclose(part, out[:, :, [3, 1]], rtol=1e-13, atol=1e-14)


def test_mixer_decode_steps_continue_the_sequence(oracle_mod):
    """T single-token mixer steps from an empty conv cache and a zero state
    give the outputs and the final state of the pinned mixer over the same T
    tokens (the cache holds each channel's last three inputs, oldest first),
    and the cache then holds the last three raw inputs."""
    rng = np.random.default_rng(13)
    B, T, H, Hk, dk, dv = 2, 6, 4, 2, 4, 3
    qr = rng.standard_normal((B, T, Hk, dk))
    kr = rng.standard_normal((B, T, Hk, dk))
    vr = rng.standard_normal((B, T, H, dv))
    z = rng.standard_normal((B, T, H, dv))
    a = rng.standard_normal((B, T, H))
    b = rng.standard_normal((B, T, H))
    C = 2 * Hk * dk + H * dv
    w = rng.standard_normal((C, 4)) * 0.5
    A = rng.uniform(0.5, 2, H)
    dtb = rng.standard_normal(H)
    nw = rng.uniform(0.5, 1.5, dv)
    ref, mid = oracle_mod.mixer(qr, kr, vr, z, a, b, w, A, dt_bias=dtb, norm_w=nw, scale=0.5,
                                return_intermediates=True)
    cache = np.zeros((B, 3, C))
    st = np.zeros((B, H, dv, dk))
    for t in range(T):
        out, st, cache = oracle_mod.mixer_decode_step(qr[:, t], kr[:, t], vr[:, t], z[:, t],
                                                      a[:, t], b[:, t], w, cache, A, st,
                                                      dt_bias=dtb, norm_w=nw, scale=0.5)
        np.testing.assert_allclose(out, ref[:, t], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(st, mid["s_final"], rtol=1e-11, atol=1e-13)
    raw = np.concatenate([qr.reshape(B, T, -1), kr.reshape(B, T, -1), vr.reshape(B, T, -1)], 2)
    np.testing.assert_array_equal(cache, raw[:, T - 3:])


# --- Per-channel decay ("6.6 Gated DeltaNet", section 6.6.7) -------------------

def test_channel_decay_equal_channels_is_the_scalar_gate(oracle_mod):
    """With the same rate on every key channel the per-channel form is the
    pinned scalar-gated recurrence."""
    rng = np.random.default_rng(14)
    T, H, dk, dv = 9, 2, 6, 4
    q, k, v, g, beta = _rand_case(rng, T, H, dk, dv)
    s0 = rng.standard_normal((1, H, dv, dk))
    gc = np.repeat(g[..., None], dk, axis=-1)
    o1, s1 = oracle_mod.gdn_recurrent(q, k, v, g, beta, s0, scale=0.7)
    o2, s2 = oracle_mod.gdn_recurrent_channel(q, k, v, gc, beta, s0, scale=0.7)
    np.testing.assert_allclose(o2, o1, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(s2, s1, rtol=1e-13, atol=1e-14)


def test_channel_decay_coordinate_keys_closed_form(oracle_mod):
    """Keys on distinct coordinate axes (k_t = e_{c_t}) and a zero initial
    state: nothing is retrieved, the write of token i lands in state column
    c_i and then decays by that channel's rates only, so
    o_t = scale * sum_{i<=t} (prod_{s=i+1..t} alpha_s[c_i]) beta_i v_i q_t[c_i]."""
    rng = np.random.default_rng(15)
    T, dk, dv, H = 6, 8, 3, 2
    cols = np.stack([rng.permutation(dk)[:T] for _ in range(H)], axis=1)   # [T, H]
    k = np.zeros((1, T, H, dk))
    for t in range(T):
        for h in range(H):
            k[0, t, h, cols[t, h]] = 1.0
    q = rng.standard_normal((1, T, H, dk))
    v = rng.standard_normal((1, T, H, dv))
    g = np.log(rng.uniform(0.3, 1.0, (1, T, H, dk)))
    beta = rng.uniform(0.1, 1.0, (1, T, H))
    o, s = oracle_mod.gdn_recurrent_channel(q, k, v, g, beta, scale=0.6)
    for h in range(H):
        for t in range(T):
            ref = np.zeros(dv)
            for i in range(t + 1):
                c = cols[i, h]
                dec = math.exp(g[0, i + 1:t + 1, h, c].sum())
                ref += dec * beta[0, i, h] * v[0, i, h] * q[0, t, h, c]
            np.testing.assert_allclose(o[0, t, h], 0.6 * ref, rtol=1e-12, atol=1e-13)
        for i in range(T):
            c = cols[i, h]
            np.testing.assert_allclose(s[0, h][:, c], math.exp(g[0, i + 1:, h, c].sum()) *
                                       beta[0, i, h] * v[0, i, h], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed", [0, 1])
def test_channel_decay_product_form(oracle_mod, seed):
    """S_t = S_{t-1} A_t + B_t with A_t = diag(alpha_t) (I - beta_t k_t k_t^T)
    and B_t = beta_t v_t k_t^T, multiplied out with dense matrices."""
    rng = np.random.default_rng(20 + seed)
    T, dk, dv, H = 6, 5, 3, 2
    q, k, v, _, beta = _rand_case(rng, T, H, dk, dv, unit_keys=False)
    g = np.log(rng.uniform(0.4, 1.0, (1, T, H, dk)))
    s0 = rng.standard_normal((1, H, dv, dk))
    o, s = oracle_mod.gdn_recurrent_channel(q, k, v, g, beta, s0, scale=1.3)
    for h in range(H):
        st = s0[0, h]
        for t in range(T):
            A = np.diag(np.exp(g[0, t, h])) @ (np.eye(dk) - beta[0, t, h] *
                                                 np.outer(k[0, t, h], k[0, t, h]))
            st = st @ A + beta[0, t, h] * np.outer(v[0, t, h], k[0, t, h])
            np.testing.assert_allclose(o[0, t, h], 1.3 * (st @ q[0, t, h]), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(s[0, h], st, rtol=1e-11, atol=1e-12)
