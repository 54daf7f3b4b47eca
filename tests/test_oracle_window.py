"""Pins of the sliding-window oracle: window lists and aligned sizes by brute-force
search, the padding against an independent bouncing-index walk, crop of pad =
identity, the windows restarting the causal clip, and a windowed Haar round trip
that reproduces the input."""

import itertools

import numpy as np
import pytest

from oracle import haar as ohaar
from oracle import window as ow


def test_window_list_examples_and_cover():
    assert ow.window_bounds(17, 17) == [(0, 17)]
    assert ow.window_bounds(40, 17) == [(0, 17), (17, 17), (34, 6)]
    assert ow.window_bounds(1, 17) == [(0, 1)]
    for T, win in itertools.product(range(1, 60), (1, 5, 17)):
        frames = [t0 + i for t0, nt in ow.window_bounds(T, win) for i in range(nt)]
        assert frames == list(range(T))
        assert all(1 <= nt <= win for _, nt in ow.window_bounds(T, win))


def brute_aligned(n, a):
    m = n
    while (m - 1) % a:
        m += 1
    return m


def test_aligned_sizes():
    # the guide's 9-frame 512x512 clip and the 17-frame window are already aligned
    assert ow.aligned_size(9, 512, 512, 4, 8) == (9, 512, 512)
    for a in (4, 8, 16):
        assert ow.aligned_size(17, 720, 1280, a, 16) == (17, 720, 1280)
    assert ow.aligned_size(6, 1080, 1920, 8, 16) == (9, 1088, 1920)
    assert ow.aligned_size(1, 3, 5, 4, 4) == (1, 4, 8)
    for n, a in itertools.product(range(1, 40), (1, 2, 4, 8)):
        Tp, Hp, Wp = ow.aligned_size(n, n, n + 3, a, a)
        assert Tp == brute_aligned(n, a)
        assert Hp % a == 0 and Hp - a < n <= Hp
        assert Wp % a == 0 and Wp - a < n + 3 <= Wp


def walk_index(t, n):
    """Frame read for padded position t of an n-frame window: walk t steps from
    frame 0, one frame per step, turning round at either end (no frame repeated at
    the turn); a one-frame window stays on its frame."""
    if n == 1:
        return 0
    i, step = 0, 1
    for _ in range(t):
        if not 0 <= i + step < n:
            step = -step
        i += step
    return i


def brute_pad(x, t0, nt, Tp, Hp, Wp):
    B, C, T, H, W = x.shape
    y = np.zeros((B, C, Tp, Hp, Wp))
    for b, c, t, h, w in itertools.product(range(B), range(C), range(Tp), range(Hp), range(Wp)):
        if h < H and w < W:
            y[b, c, t, h, w] = x[b, c, t0 + walk_index(t, nt), h, w]
    return y


@pytest.mark.parametrize("t0,nt,Tp", [(0, 5, 5), (2, 3, 9), (1, 2, 9), (4, 1, 5), (0, 6, 9), (3, 4, 13)])
def test_pad_against_bouncing_walk(t0, nt, Tp):
    rng = np.random.default_rng(t0 * 31 + nt)
    x = rng.normal(size=(2, 2, 8, 3, 5))
    got = ow.pad_window(x, t0, nt, Tp, 4, 8)
    assert np.array_equal(got, brute_pad(x, t0, nt, Tp, 4, 8))


def test_reflect_example_by_hand():
    x = np.arange(3, dtype=np.float64).reshape(1, 1, 3, 1, 1)  # frames a=0, b=1, c=2
    y = ow.pad_window(x, 0, 3, 9, 1, 1)[0, 0, :, 0, 0]
    assert y.tolist() == [0, 1, 2, 1, 0, 1, 2, 1, 0]


def test_crop_of_pad_is_identity_and_windowed_identity():
    rng = np.random.default_rng(3)
    x = rng.normal(size=(1, 3, 40, 7, 10))
    out = np.zeros_like(x)
    for t0, nt in ow.window_bounds(40, 17):
        Tp, Hp, Wp = ow.aligned_size(nt, 7, 10, 8, 8)
        ow.unpad_window(ow.pad_window(x, t0, nt, Tp, Hp, Wp), out, t0, nt)
    assert np.array_equal(out, x)
    assert np.array_equal(ow.windowed(x, lambda w: w, 17, 4, 4), x)


def test_windows_restart_the_causal_clip():
    # a process that subtracts its clip's first frame: zero exactly at each window start
    rng = np.random.default_rng(4)
    x = rng.normal(size=(1, 1, 30, 4, 4))
    out = ow.windowed(x, lambda w: w - w[:, :, :1], 17, 4, 4)
    for t0, _ in ow.window_bounds(30, 17):
        assert np.all(out[:, :, t0] == 0)
    assert np.all(out[:, :, 1] != 0)


def test_windowed_haar_round_trip_reproduces_the_input():
    rng = np.random.default_rng(5)
    x = rng.uniform(-1, 1, size=(1, 3, 23, 10, 13))
    rt = ow.windowed(x, lambda w: ohaar.haar3d_inv(ohaar.haar3d_fwd(w)), 17, 4, 4)
    assert np.max(np.abs(rt - x)) < 1e-12


def test_bad_windows_raise():
    x = np.zeros((1, 1, 5, 2, 2))
    with pytest.raises(ValueError):
        ow.pad_window(x, 3, 3, 5, 2, 2)
    with pytest.raises(ValueError):
        ow.pad_window(x, 0, 5, 4, 2, 2)
    with pytest.raises(ValueError):
        ow.window_bounds(0, 17)
