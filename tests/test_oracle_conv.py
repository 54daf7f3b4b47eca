"""Pins of the factorized causal convolution oracle: brute force, torch conv3d,
causality, impulse response, linearity and special cases."""

import numpy as np
import pytest
import torch

from oracle import conv


def brute_force(x, ws, wt, bs=None, bt=None):
    """Direct nested-loop sums (pure Python), tiny shapes only."""
    B, Cin, T, H, W = x.shape
    Cout, _, _, k, _ = ws.shape
    p = (k - 1) // 2
    S = np.zeros((B, Cout, T, H, W))
    for b in range(B):
        for m in range(Cout):
            for t in range(T):
                for h in range(H):
                    for w in range(W):
                        acc = 0.0 if bs is None else bs[m]
                        for c in range(Cin):
                            for dy in range(k):
                                for dx in range(k):
                                    hh, ww = h + dy - p, w + dx - p
                                    if 0 <= hh < H and 0 <= ww < W:
                                        acc += ws[m, c, 0, dy, dx] * x[b, c, t, hh, ww]
                        S[b, m, t, h, w] = acc
    if wt is None:
        return S
    kt = wt.shape[2]
    Y = np.zeros((B, wt.shape[0], T, H, W))
    for b in range(B):
        for o in range(wt.shape[0]):
            for t in range(T):
                for h in range(H):
                    for w in range(W):
                        acc = 0.0 if bt is None else bt[o]
                        for m in range(Cout):
                            for dt in range(kt):
                                tt = t + dt - (kt - 1)
                                if tt >= 0:
                                    acc += wt[o, m, dt, 0, 0] * S[b, m, tt, h, w]
                        Y[b, o, t, h, w] = acc
    return Y


def rand_case(seed, B=1, Cin=3, Cout=4, T=4, H=5, W=5, k=3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, Cin, T, H, W))
    ws = rng.standard_normal((Cout, Cin, 1, k, k))
    wt = rng.standard_normal((Cout, Cout, k, 1, 1))
    return x, ws, wt


def test_brute_force_k3():
    x, ws, wt = rand_case(1)
    np.testing.assert_allclose(conv.causal_conv3d_fact(x, ws, wt), brute_force(x, ws, wt), atol=1e-12)


def test_brute_force_with_bias_and_batch():
    x, ws, wt = rand_case(2, B=2, Cin=2, Cout=3, T=3, H=4, W=3)
    rng = np.random.default_rng(20)
    bs, bt = rng.standard_normal(3), rng.standard_normal(3)
    np.testing.assert_allclose(conv.causal_conv3d_fact(x, ws, wt, bs, bt),
                               brute_force(x, ws, wt, bs, bt), atol=1e-12)


def test_matches_torch_conv3d_float64():
    x, ws, wt = rand_case(3, B=2, Cin=5, Cout=6, T=6, H=7, W=9)
    xt = torch.from_numpy(x)
    s = torch.nn.functional.conv3d(xt, torch.from_numpy(ws), padding=(0, 1, 1))
    s = torch.nn.functional.pad(s, (0, 0, 0, 0, 2, 0))
    y = torch.nn.functional.conv3d(s, torch.from_numpy(wt)).numpy()
    np.testing.assert_allclose(conv.causal_conv3d_fact(x, ws, wt), y, atol=1e-11)


def test_causality():
    x, ws, wt = rand_case(4, T=7)
    y = conv.causal_conv3d_fact(x, ws, wt)
    for t0 in range(7):
        xp = x.copy()
        xp[:, :, t0] += 1.0
        yp = conv.causal_conv3d_fact(xp, ws, wt)
        assert np.array_equal(y[:, :, :t0], yp[:, :, :t0])
        assert not np.allclose(y[:, :, t0], yp[:, :, t0])


def test_impulse_response_reproduces_weights():
    rng = np.random.default_rng(5)
    Cin, Cout, k = 2, 3, 3
    ws = rng.standard_normal((Cout, Cin, 1, k, k))
    x = np.zeros((1, Cin, 1, 5, 5))
    x[0, 1, 0, 2, 2] = 1.0
    s = conv.spatial_conv(x, ws)
    # cross-correlation: output (2 - (dy-1), 2 - (dx-1)) sees the impulse through tap (dy, dx)
    for dy in range(k):
        for dx in range(k):
            np.testing.assert_allclose(s[0, :, 0, 2 - (dy - 1), 2 - (dx - 1)], ws[:, 1, 0, dy, dx], atol=0)
    wt = rng.standard_normal((Cout, Cout, k, 1, 1))
    z = np.zeros((1, Cout, 4, 1, 1))
    z[0, 0, 1, 0, 0] = 1.0
    y = conv.temporal_conv(z, wt)
    for dt in range(k):
        t = 1 + (k - 1) - dt
        if t < 4:
            np.testing.assert_allclose(y[0, :, t, 0, 0], wt[:, 0, dt, 0, 0], atol=0)
    assert np.all(y[0, :, 0] == 0)


def test_linearity():
    x, ws, wt = rand_case(6)
    x2 = np.random.default_rng(60).standard_normal(x.shape)
    a, b = 0.7, -1.3
    lhs = conv.causal_conv3d_fact(a * x + b * x2, ws, wt)
    rhs = a * conv.causal_conv3d_fact(x, ws, wt) + b * conv.causal_conv3d_fact(x2, ws, wt)
    np.testing.assert_allclose(lhs, rhs, atol=1e-11)


def test_k1_is_channel_matmul():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, 5, 3, 4, 4))
    w = rng.standard_normal((6, 5, 1, 1, 1))
    y = conv.causal_conv3d_fact(x, w)
    ref = np.einsum("oc,bcthw->bothw", w[:, :, 0, 0, 0], x)
    np.testing.assert_allclose(y, ref, atol=1e-12)
    np.testing.assert_allclose(conv.pointwise(x, w[:, :, 0, 0, 0]), ref, atol=1e-12)
    b = rng.standard_normal(6)
    np.testing.assert_allclose(conv.pointwise(x, w, b), ref + b[None, :, None, None, None], atol=1e-12)


def test_single_frame_uses_last_temporal_tap_only():
    x, ws, wt = rand_case(8, T=1)
    y = conv.causal_conv3d_fact(x, ws, wt)
    s = conv.spatial_conv(x, ws)
    ref = np.einsum("om,bmthw->bothw", wt[:, :, 2, 0, 0], s)
    np.testing.assert_allclose(y, ref, atol=1e-12)


def test_bad_weights_raise():
    with pytest.raises(ValueError):
        conv.spatial_conv(np.zeros((1, 2, 1, 4, 4)), np.zeros((3, 2, 1, 2, 2)))
    with pytest.raises(ValueError):
        conv.spatial_conv(np.zeros((1, 2, 1, 4, 4)), np.zeros((3, 4, 1, 3, 3)))
