"""Pins of the backward oracle (kda_oracle_bwd.c) against finite differences
of the forward oracle and closed forms.

The backward is the separate pass the pages test beside the forward (page
"feat(kda): integrate KDA attention with tokamax backend and CP support": its
CP gradient-equivalence test; the forward's Delta Rule formulation there
defines the function being differentiated).  The loss is
sum(o * d_o) + sum(final_state * d_final_state).
None of these re-types the oracle: the finite differences run the separate
forward oracle, the closed forms are derived by hand.
"""
import numpy as np
import pytest

import oracle


def _grid(shape, seed, scale=1.0):
    """fp32 values on a 2^-12 grid with |x| < 2, so x +- 2^-7 and x +- 2^-8
    are exact in fp32 (the forward oracle takes fp32 inputs)."""
    x = np.clip(scale * np.random.default_rng(seed).standard_normal(shape), -1.9, 1.9)
    return (np.round(x * 4096) / 4096).astype(np.float32)


def _case(l2norm, packed, seed=0):
    B, T, H, K, V = 2, 11, 2, 4, 3
    q, k, v = _grid((B, T, H, K), seed), _grid((B, T, H, K), seed + 1), _grid((B, T, H, V), seed + 2)
    if not l2norm:      # roughly unit vectors, still on the grid
        q, k = (np.round(a / np.linalg.norm(a, axis=-1, keepdims=True) * 4096).astype(np.float32) / 4096
                for a in (q, k))
    g = -np.abs(_grid((B, T, H, K), seed + 3, 0.5))
    beta = np.abs(_grid((B, T, H), seed + 4, 0.6))
    seg, n = None, 0
    if packed:
        seg = np.array([[1, 1, 1, 1, 2, 2, 0, 3, 3, 3, 3], [1] * T], np.int32)
        n = 3
    shape = (B, H, K, V) if seg is None else (B, n, H, K, V)
    S0 = _grid(shape, seed + 5, 0.5)
    rng = np.random.default_rng(seed + 6)
    d_o = rng.standard_normal((B, T, H, V))
    d_fin = rng.standard_normal(shape)
    return dict(q=q, k=k, v=v, g=g, beta=beta, initial_state=S0), seg, n, d_o, d_fin


def _loss(x, seg, n, d_o, d_fin, l2norm, scale):
    o, fin = oracle.kda_forward(x["q"], x["k"], x["v"], x["g"], x["beta"], scale=scale,
                                initial_state=x["initial_state"], output_final_state=True, use_qk_l2norm=l2norm,
                                segment_ids=seg, max_segments=n, num_threads=1)
    return float(np.sum(o * d_o) + np.sum(fin * d_fin))


@pytest.mark.parametrize("l2norm,packed", [(False, False), (True, True)])
def test_gradients_match_finite_differences(l2norm, packed):
    """Every gradient entry against a Richardson-extrapolated central
    difference of the forward oracle (steps 2^-7 and 2^-8, exact in fp32;
    truncation error O(h^4))."""
    x, seg, n, d_o, d_fin = _case(l2norm, packed)
    scale = 0.7
    gr = oracle.kda_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], d_o, scale=scale,
                             initial_state=x["initial_state"], d_final_state=d_fin, use_qk_l2norm=l2norm,
                             segment_ids=seg, max_segments=n)
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "initial_state": "d_initial_state"}
    for name, gname in names.items():
        a = x[name]
        fd = np.zeros(a.shape)
        for idx in np.ndindex(a.shape):
            d = []
            for h in (2.0 ** -7, 2.0 ** -8):
                vals = []
                for sgn in (1, -1):
                    xp = dict(x)
                    xp[name] = a.copy()
                    xp[name][idx] = np.float32(a[idx] + sgn * h)
                    assert float(xp[name][idx]) == float(a[idx]) + sgn * h      # the step is exact
                    vals.append(_loss(xp, seg, n, d_o, d_fin, l2norm, scale))
                d.append((vals[0] - vals[1]) / (2 * h))
            fd[idx] = (4 * d[1] - d[0]) / 3
        got = gr[gname]
        scale_ref = np.sqrt(np.mean(fd * fd)) + 1e-12
        err = np.max(np.abs(got - fd)) / scale_ref
        assert err < 2e-6, f"{gname}: max|analytic - fd| / rms = {err:.2e}"


def test_zero_beta_closed_form():
    """beta = 0 writes nothing: o_t = scale q_t^T diag(exp(G_t)) S0 with
    G_t = sum_{s<=t} g_s, so dq_t = scale diag(exp(G_t)) S0 do_t,
    dS0 = sum_t scale diag(exp(G_t)) q_t do_t^T + diag(exp(G_T)) dfin, and
    dk = dv = 0."""
    B, T, H, K, V = 1, 7, 1, 5, 4
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal(s).astype(np.float32) for s in ((B, T, H, K), (B, T, H, K), (B, T, H, V)))
    g = -np.abs(rng.standard_normal((B, T, H, K))).astype(np.float32) * 0.3
    beta = np.zeros((B, T, H), np.float32)
    S0 = rng.standard_normal((B, H, K, V)).astype(np.float32)
    d_o, d_fin = rng.standard_normal((B, T, H, V)), rng.standard_normal((B, H, K, V))
    gr = oracle.kda_backward(q, k, v, g, beta, d_o, scale=0.5, initial_state=S0, d_final_state=d_fin)
    G = np.cumsum(g[0, :, 0].astype(np.float64), axis=0)
    S = S0[0, 0].astype(np.float64)
    dS0 = np.exp(G[-1])[:, None] * d_fin[0, 0]
    for t in range(T):
        e = np.exp(G[t])
        np.testing.assert_allclose(gr["dq"][0, t, 0], 0.5 * e * (S @ d_o[0, t, 0]), rtol=1e-12, atol=1e-14)
        dS0 += 0.5 * np.outer(e * q[0, t, 0], d_o[0, t, 0])
    np.testing.assert_allclose(gr["d_initial_state"][0, 0], dS0, rtol=1e-12, atol=1e-14)
    assert np.all(gr["dk"] == 0) and np.all(gr["dv"] == 0)


def test_linear_attention_closed_form():
    """g = 0, beta = 1, orthonormal keys, zero start state: o_t = scale
    sum_{i<=t} (q_t . k_i) v_i, so dv_i = scale sum_{t>=i} (q_t . k_i) do_t and
    dq_t = scale sum_{i<=t} (v_i . do_t) k_i."""
    T, K, V = 6, 8, 3
    basis, _ = np.linalg.qr(np.random.default_rng(4).standard_normal((K, K)))
    k = basis[:T].astype(np.float32)[None, :, None, :]
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, T, 1, K)).astype(np.float32)
    v = rng.standard_normal((1, T, 1, V)).astype(np.float32)
    d_o = rng.standard_normal((1, T, 1, V))
    gr = oracle.kda_backward(q, k, v, np.zeros_like(q), np.ones((1, T, 1), np.float32), d_o, scale=0.25)
    kd, qd, vd = (a[0, :, 0].astype(np.float64) for a in (k, q, v))
    for i in range(T):
        dv = 0.25 * sum((qd[t] @ kd[i]) * d_o[0, t, 0] for t in range(i, T))
        dq = 0.25 * sum((vd[j] @ d_o[0, i, 0]) * kd[j] for j in range(i + 1))
        np.testing.assert_allclose(gr["dv"][0, i, 0], dv, atol=2e-7)      # keys are orthonormal to fp32
        np.testing.assert_allclose(gr["dq"][0, i, 0], dq, atol=2e-7)


def test_padding_and_segments():
    """Padding tokens get zero gradients; a packed row's gradients equal those
    of its segments run separately (the forward's segment isolation)."""
    x, seg, n, d_o, d_fin = _case(False, True, seed=20)
    gr = oracle.kda_backward(x["q"], x["k"], x["v"], x["g"], x["beta"], d_o, initial_state=x["initial_state"],
                             d_final_state=d_fin, segment_ids=seg, max_segments=n)
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        assert np.all(gr[name][0, 6] == 0.0)
    for s, (a, b) in enumerate(((0, 4), (4, 6), (7, 11))):
        sub = {k_: v_[0:1, a:b] for k_, v_ in x.items() if k_ != "initial_state"}
        alone = oracle.kda_backward(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], d_o[0:1, a:b],
                                    initial_state=x["initial_state"][0:1, s], d_final_state=d_fin[0:1, s])
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            np.testing.assert_array_equal(gr[name][0:1, a:b], alone[name])
        np.testing.assert_array_equal(gr["d_initial_state"][0:1, s], alone["d_initial_state"])
