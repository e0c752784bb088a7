"""Pins of the layer-step oracle (short convolution, gated RMSNorm) against
closed forms, library routines and invariants.  Sources: the layer pipeline
of the page "feat(kda): integrate KDA attention with tokamax backend and CP
support" (a causal depthwise 1D convolution with SiLU; a per-head RMSNorm
with a sigmoid output gate) and that page's review notes (the convolution
respects packed segments)."""
import numpy as np
import pytest

from oracle import layer_ops as lo


def _rand(shape, seed, scale=1.0):
    return (scale * np.random.default_rng(seed).standard_normal(shape)).astype(np.float32)


def _silu(x):
    return x / (1.0 + np.exp(-x))


def test_conv_matches_numpy_convolution_per_channel():
    """Without segments, each channel is a causal FIR filter: the first T
    samples of numpy's full convolution of x with the reversed-tap kernel
    (tap W-1 multiplies the current token), then SiLU."""
    B, T, D, W = 2, 23, 5, 4
    x, w = _rand((B, T, D), 1), _rand((D, W), 2)
    y = lo.short_conv(x, w)
    xd, wd = x.astype(np.float64), w.astype(np.float64)
    for b in range(B):
        for d in range(D):
            pre = np.convolve(xd[b, :, d], wd[d, ::-1])[:T]
            np.testing.assert_allclose(y[b, :, d], _silu(pre), rtol=1e-12, atol=1e-14)


def test_conv_special_kernels():
    """A one-tap kernel is SiLU of a scaled input; a kernel that keeps only the
    oldest tap shifts by W-1 tokens and reads zero before the sequence; SiLU(0)
    = 0 and SiLU is x/2 + x^2/4 + O(x^4) near 0."""
    B, T, D = 1, 9, 3
    x = _rand((B, T, D), 3)
    y1 = lo.short_conv(x, np.array([[2.0], [-1.0], [0.5]], np.float32))
    np.testing.assert_allclose(y1[0], _silu(x[0].astype(np.float64) * [2.0, -1.0, 0.5]), rtol=1e-12)
    w = np.zeros((D, 4), np.float32)
    w[:, 0] = 1.0
    ys = lo.short_conv(x, w)
    np.testing.assert_allclose(ys[0, 3:], _silu(x[0, :-3].astype(np.float64)), rtol=1e-12)
    assert np.all(ys[0, :3] == 0.0)
    small = np.full((1, 1, 1), 1e-3, np.float32)
    v = lo.short_conv(small, np.ones((1, 1), np.float32))[0, 0, 0]
    xs = float(np.float32(1e-3))
    assert abs(v - (xs / 2 + xs * xs / 4)) < 1e-12


def test_conv_packed_equals_independent_segments():
    """Segments packed in one row do not see each other (the review notes'
    segment-aware convolution): each segment's output equals a separate run
    on that segment alone; padding outputs zero."""
    T, D, W = 30, 4, 4
    x, w = _rand((1, T, D), 4), _rand((D, W), 5)
    seg = np.zeros((1, T), np.int32)
    seg[0, 0:7] = 1
    seg[0, 7:8] = 2
    seg[0, 8:20] = 3
    seg[0, 22:30] = 3        # same id after padding: a new segment
    y = lo.short_conv(x, w, segment_ids=seg)
    for a, b in ((0, 7), (7, 8), (8, 20), (22, 30)):
        alone = lo.short_conv(x[:, a:b], w)
        np.testing.assert_allclose(y[:, a:b], alone, rtol=1e-12, atol=1e-15)
    assert np.all(y[0, 20:22] == 0.0)


def test_conv_identity_activation_is_linear():
    """Before the activation the convolution is linear in x (integer-valued
    inputs keep every sum exact)."""
    B, T, D, W = 1, 12, 3, 3
    rng = np.random.default_rng(6)
    x1 = rng.integers(-8, 8, (B, T, D)).astype(np.float32)
    x2 = rng.integers(-8, 8, (B, T, D)).astype(np.float32)
    w = _rand((D, W), 8)
    f = lambda x: lo.short_conv(x, w, activation="identity")
    np.testing.assert_allclose(f(x1 + 2 * x2), f(x1) + 2 * f(x2), rtol=1e-12, atol=1e-12)


def test_rmsnorm_closed_forms():
    """A constant row c normalises to sign(c)/sqrt(1 + eps/c^2); a row of unit
    RMS is unchanged by the norm; sigmoid(0) = 1/2 halves the output."""
    V = 8
    w = np.linspace(0.5, 2.0, V).astype(np.float32)
    o = np.full((2, V), -3.0, np.float32)
    z = np.zeros((2, V), np.float32)
    y = lo.gated_rmsnorm(o, z, w, eps=1e-6)
    np.testing.assert_allclose(y, np.broadcast_to(-w.astype(np.float64) / np.sqrt(1 + 1e-6 / 9) * 0.5, (2, V)),
                               rtol=1e-13)
    unit = np.array([[1, -1, 1, -1, 1, -1, 1, -1]], np.float32)
    g = np.full((1, V), np.log(3.0), np.float32)     # sigmoid(ln 3) = 3/4
    y = lo.gated_rmsnorm(unit, g, w, eps=0.0)
    np.testing.assert_allclose(y, w * unit * 0.75, rtol=1e-7)


def test_rmsnorm_scale_invariance_and_per_row():
    """y(alpha o) = y(o) up to eps, and rows (heads) are normalised separately."""
    o, z, w = _rand((3, 4, 16), 9), _rand((3, 4, 16), 10), _rand((16,), 11)
    y = lo.gated_rmsnorm(o, z, w, eps=0.0)
    y2 = lo.gated_rmsnorm(o * np.float32(4.0), z, w, eps=0.0)
    np.testing.assert_allclose(y, y2, rtol=1e-12)
    y3 = lo.gated_rmsnorm(o[1:2, 2:3], z[1:2, 2:3], w, eps=0.0)
    np.testing.assert_allclose(y[1:2, 2:3], y3, rtol=1e-15)
    with pytest.raises(ValueError):
        lo.gated_rmsnorm(o, z[..., :8], w)
