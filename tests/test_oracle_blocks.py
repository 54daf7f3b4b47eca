"""Pins of the residual / downsampling / upsampling block oracle: LayerNorm and
Swish against torch's float64 routines and closed forms, strided convolutions
against torch's conv3d with stride and padding, the residual block against a
composition written with torch ops, identity and causality properties, and the
compression factors the pages list."""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import blocks as ob
from oracle import conv as oconv
from oracle import haar as ohaar


def rng_arrays(seed, *shapes, scale=1.0):
    rng = np.random.default_rng(seed)
    return [rng.normal(size=s) * scale for s in shapes]


def test_swish_closed_forms_and_torch():
    assert ob.swish(0.0) == 0.0
    assert abs(ob.swish(1.0) - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16
    assert ob.swish(-800.0) == 0.0 and ob.swish(800.0) == 800.0
    (x,) = rng_arrays(1, (1000,), scale=6)
    assert np.max(np.abs(ob.swish(x) - F.silu(torch.from_numpy(x)).numpy())) < 1e-15


def test_layer_norm_against_torch_channels_last():
    x, g, b = rng_arrays(2, (2, 24, 3, 4, 5), (24,), (24,), scale=3)
    x = x + 7.0  # a large common offset: the mean is taken out before the variance
    ref = F.layer_norm(torch.from_numpy(x).permute(0, 2, 3, 4, 1), (24,), torch.from_numpy(g), torch.from_numpy(b),
                       eps=ob.LN_EPS).permute(0, 4, 1, 2, 3).numpy()
    assert np.max(np.abs(ob.layer_norm(x, g, b) - ref)) < 1e-12


def test_layer_norm_by_hand():
    # channels (1, 3): mean 2, variance 1 -> (-1, 1) / sqrt(1 + eps)
    x = np.array([1.0, 3.0]).reshape(1, 2, 1, 1, 1)
    y = ob.layer_norm(x, np.array([2.0, 1.0]), np.array([0.5, 0.0]))
    s = 1 / np.sqrt(1 + ob.LN_EPS)
    assert np.allclose(y.ravel(), [-2 * s + 0.5, s], rtol=0, atol=1e-15)


def test_strided_convs_against_torch():
    x, ws, wt, bs, bt = rng_arrays(3, (1, 5, 5, 8, 6), (7, 5, 1, 3, 3), (7, 7, 3, 1, 1), (7,), (7,))
    got = ob.downsample(x, ws, wt, bs, bt)
    tx = torch.from_numpy(x)
    s = F.conv3d(tx, torch.from_numpy(ws), torch.from_numpy(bs), stride=(1, 2, 2), padding=(0, 1, 1))
    ref = F.conv3d(F.pad(s, (0, 0, 0, 0, 2, 0)), torch.from_numpy(wt), torch.from_numpy(bt), stride=(2, 1, 1))
    assert got.shape == (1, 7, 3, 4, 3)
    assert np.max(np.abs(got - ref.numpy())) < 1e-12
    # spatial only / temporal only
    assert np.max(np.abs(ob.downsample(x, ws, None, bs) - s.numpy())) < 1e-12
    (x7,) = rng_arrays(4, (2, 7, 9, 2, 3))
    ref_t = F.conv3d(F.pad(torch.from_numpy(x7), (0, 0, 0, 0, 2, 0)), torch.from_numpy(wt), stride=(2, 1, 1))
    assert np.max(np.abs(ob.downsample(x7, None, wt) - ref_t.numpy())) < 1e-12


def test_temporal_downsample_keeps_the_causal_first_frame():
    x, wt = rng_arrays(5, (1, 4, 9, 2, 2), (4, 4, 3, 1, 1))
    y = ob.downsample(x, None, wt)
    assert y.shape[2] == 5  # 1 + (9 - 1) / 2
    x2 = x.copy()
    x2[:, :, 1:] += 1.0  # frame 0's output depends on frame 0 only
    y2 = ob.downsample(x2, None, wt)
    assert np.array_equal(y2[:, :, 0], y[:, :, 0]) and not np.allclose(y2[:, :, 1], y[:, :, 1])
    x3 = x.copy()
    x3[:, :, 5:] += 1.0  # output frame j sees frames <= 2j
    y3 = ob.downsample(x3, None, wt)
    assert np.array_equal(y3[:, :, :3], y[:, :, :3]) and not np.allclose(y3[:, :, 3], y[:, :, 3])


def torch_factorized(x, ws, wt):
    k = ws.shape[-1]
    s = F.conv3d(x, ws, padding=(0, (k - 1) // 2, (k - 1) // 2))
    return F.conv3d(F.pad(s, (0, 0, 0, 0, wt.shape[2] - 1, 0)), wt)


def torch_resblock(x, p):
    def ln_swish(h, g, b):
        h = F.layer_norm(h.permute(0, 2, 3, 4, 1), (h.shape[1],), g, b, eps=ob.LN_EPS).permute(0, 4, 1, 2, 3)
        return F.silu(h)
    t = {k: torch.from_numpy(v) for k, v in p.items()}
    h = torch_factorized(ln_swish(x, t["ln1_g"], t["ln1_b"]), t["c1_s"], t["c1_t"])
    h = torch_factorized(ln_swish(h, t["ln2_g"], t["ln2_b"]), t["c2_s"], t["c2_t"])
    return x + h


def block_params(seed, C, scale=0.2):
    rng = np.random.default_rng(seed)
    p = {"ln1_g": 1 + 0.1 * rng.normal(size=C), "ln1_b": 0.1 * rng.normal(size=C),
         "ln2_g": 1 + 0.1 * rng.normal(size=C), "ln2_b": 0.1 * rng.normal(size=C)}
    for c in ("c1", "c2"):
        p[c + "_s"] = rng.normal(size=(C, C, 1, 3, 3)) * scale
        p[c + "_t"] = rng.normal(size=(C, C, 3, 1, 1)) * scale
    return p


def test_resblock_against_torch_composition():
    (x,) = rng_arrays(6, (1, 8, 5, 6, 7))
    p = block_params(7, 8)
    ref = torch_resblock(torch.from_numpy(x), p).numpy()
    assert np.max(np.abs(ob.resblock(x, p) - ref)) < 1e-11


def test_resblock_identity_and_causality():
    (x,) = rng_arrays(8, (1, 6, 6, 4, 4))
    p = block_params(9, 6)
    zero = dict(p, c2_s=np.zeros_like(p["c2_s"]), c2_t=np.zeros_like(p["c2_t"]))
    assert np.array_equal(ob.resblock(x, zero), x)
    base = ob.resblock(x, p)
    x2 = x.copy()
    x2[:, :, 3:] += 1.0
    got = ob.resblock(x2, p)
    assert np.array_equal(got[:, :, :3], base[:, :, :3]) and not np.allclose(got[:, :, 3:], base[:, :, 3:])


def test_upsample_repeat_and_mirror_of_downsampling():
    (x,) = rng_arrays(10, (1, 3, 4, 2, 3))
    u = ob.upsample_repeat(x)
    assert u.shape == (1, 3, 7, 4, 6)  # 2T - 1 frames, 2H, 2W
    assert np.array_equal(u[:, :, 0, ::2, ::2], x[:, :, 0])
    for j in range(1, 4):
        for f in (2 * j - 1, 2 * j):
            assert np.array_equal(u[:, :, f, 1::2, 0::2], x[:, :, j])
    # every second frame / pixel of the repetition is the input again
    assert np.array_equal(u[:, :, ::2, ::2, ::2], x)
    # the upsampled length is what the temporal stride maps back: 1 + (2T - 2) / 2 = T
    assert 1 + (u.shape[2] - 1) // 2 == x.shape[2]


def test_upsample_block_against_torch():
    x, ws, wt = rng_arrays(11, (1, 4, 3, 3, 2), (5, 4, 1, 3, 3), (5, 5, 3, 1, 1))
    tx = torch.from_numpy(x)
    rep = torch.cat([tx[:, :, :1], tx[:, :, 1:].repeat_interleave(2, dim=2)], dim=2)
    rep = F.interpolate(rep, scale_factor=(1, 2, 2), mode="nearest")
    ref = torch_factorized(rep, torch.from_numpy(ws), torch.from_numpy(wt)).numpy()
    assert np.max(np.abs(ob.upsample(x, ws, wt) - ref)) < 1e-12


@pytest.mark.parametrize("factor,down_t,down_s,T,H,W,grid", [
    ((4, 8, 8), 0, 1, 9, 512, 512, (3, 64, 64)),       # the guide's 9-frame 512x512 example at 4x8x8
    ((8, 8, 8), 1, 1, 121, 720, 1280, (16, 90, 160)),  # CV8x8x8-720p on its 121-frame context
    ((8, 16, 16), 1, 2, 49, 720, 1280, (7, 45, 80)),   # DV8x16x16-720p on its 49-frame context
])
def test_compression_factors_compose_from_haar_and_stride2_blocks(factor, down_t, down_s, T, H, W, grid):
    # the Haar patcher gives 4 x 4 x 4; each stride-2 block halves T' - 1 (causal) or H', W'
    ft, fs = 4 * 2 ** down_t, 4 * 2 ** down_s
    assert (ft, fs, fs) == factor
    t = ohaar.latent_frames(T)
    h, w = H // 4, W // 4
    for _ in range(down_t):
        t = 1 + (t - 1) // 2
    for _ in range(down_s):
        h, w = h // 2, w // 2
    assert (t, h, w) == grid == (1 + (T - 1) // ft, H // fs, W // fs)


def test_bad_shapes_raise():
    x = np.zeros((1, 2, 4, 4, 4))
    with pytest.raises(ValueError):
        ob.downsample(x, None, np.zeros((2, 2, 3, 1, 1)))  # T = 4 is not 1 + 2k
    with pytest.raises(ValueError):
        ob.downsample(np.zeros((1, 2, 3, 5, 4)), np.zeros((2, 2, 1, 3, 3)))
