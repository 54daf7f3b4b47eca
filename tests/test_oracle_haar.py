"""Pins of the Haar oracle against closed forms, invariants and the pages' shapes."""

import json
import os

import numpy as np
import pytest
import scipy.linalg
from hypothesis import given, settings, strategies as st

from oracle import haar

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))

# Two orthonormal Haar levels along one axis of length 4, written out: row
# 2*b1 + b2 holds the level-1 band b1 refined by the level-2 band b2.
M4 = 0.5 * np.array([[1, 1, 1, 1],
                     [1, 1, -1, -1],
                     [1, -1, 1, -1],
                     [1, -1, -1, 1]], dtype=np.float64)


def pad_ref(x):
    """Causal extension by index: P[p] = x[max(p-3, 0)]."""
    T = x.shape[2]
    src = np.maximum(np.arange(T + 3) - 3, 0)
    return x[:, :, src]


def channel_of(rows, C, c):
    """Output channel of per-axis packet rows (2*b1 + b2 each), subband-major."""
    b1 = [r >> 1 for r in rows]
    b2 = [r & 1 for r in rows]
    n = len(rows)
    s1 = sum(b << (n - 1 - i) for i, b in enumerate(b1))
    s2 = sum(b << (n - 1 - i) for i, b in enumerate(b2))
    return s2 * (2 ** n) * C + s1 * C + c


def test_packet_matrix_is_scaled_hadamard_rows():
    H4 = scipy.linalg.hadamard(4).astype(np.float64) / 2.0
    assert sorted(map(tuple, M4)) == sorted(map(tuple, H4))
    np.testing.assert_allclose(M4 @ M4.T, np.eye(4), atol=1e-15)
    M3 = np.kron(np.kron(M4, M4), M4)
    np.testing.assert_allclose(M3 @ M3.T, np.eye(64), atol=1e-14)


def test_page_tap_is_one_over_sqrt2_to_four_digits():
    taps = GOLDEN["haar_tap"]["taps_4_digits"]
    for t in taps:
        assert round(haar.R, 4) == t


@pytest.mark.parametrize("shape", [(1, 2, 5, 8, 8), (2, 1, 9, 4, 12), (1, 3, 1, 8, 4)])
def test_fwd_3d_equals_explicit_block_matrix(shape):
    rng = np.random.default_rng(7)
    x = rng.standard_normal(shape)
    y = haar.haar3d_fwd(x, 2)
    B, C, T, H, W = shape
    P = pad_ref(x)
    Tq = (T + 3) // 4
    assert y.shape == (B, 64 * C, Tq, H // 4, W // 4)
    M3 = np.kron(np.kron(M4, M4), M4)
    for b in range(B):
        for c in range(C):
            for tq in range(Tq):
                for hq in range(H // 4):
                    for wq in range(W // 4):
                        blk = P[b, c, 4 * tq:4 * tq + 4, 4 * hq:4 * hq + 4, 4 * wq:4 * wq + 4].ravel()
                        coef = M3 @ blk
                        for rt in range(4):
                            for rh in range(4):
                                for rw in range(4):
                                    ch = channel_of((rt, rh, rw), C, c)
                                    assert abs(y[b, ch, tq, hq, wq] - coef[rt * 16 + rh * 4 + rw]) < 1e-13


def test_fwd_2d_equals_explicit_block_matrix():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((1, 3, 2, 8, 12))
    y = haar.haar3d_fwd(x, 0)
    assert y.shape == (1, 48, 2, 2, 3)
    M2 = np.kron(M4, M4)
    for c in range(3):
        for t in range(2):
            for hq in range(2):
                for wq in range(3):
                    coef = M2 @ x[0, c, t, 4 * hq:4 * hq + 4, 4 * wq:4 * wq + 4].ravel()
                    for rh in range(4):
                        for rw in range(4):
                            ch = channel_of((rh, rw), 3, c)
                            assert abs(y[0, ch, t, hq, wq] - coef[rh * 4 + rw]) < 1e-13


def test_one_hot_gives_matrix_column():
    x = np.zeros((1, 1, 5, 4, 4))
    x[0, 0, 2, 1, 3] = 1.0     # padded frame 5 = block 1, local t 1
    y = haar.haar3d_fwd(x, 2)
    M3 = np.kron(np.kron(M4, M4), M4)
    col = M3[:, 1 * 16 + 1 * 4 + 3]
    for rt in range(4):
        for rh in range(4):
            for rw in range(4):
                assert abs(y[0, channel_of((rt, rh, rw), 1, 0), 1, 0, 0] - col[rt * 16 + rh * 4 + rw]) < 1e-15
    assert np.all(y[:, :, 0] == 0)


@settings(max_examples=25, deadline=None)
@given(B=st.integers(1, 2), C=st.integers(1, 3), k=st.integers(0, 4),
       h=st.integers(1, 3), w=st.integers(1, 3), seed=st.integers(0, 2**31 - 1))
def test_perfect_reconstruction_3d(B, C, k, h, w, seed):
    x = np.random.default_rng(seed).standard_normal((B, C, 1 + 4 * k, 4 * h, 4 * w))
    np.testing.assert_allclose(haar.haar3d_inv(haar.haar3d_fwd(x, 2), 2), x, atol=1e-12)


@settings(max_examples=15, deadline=None)
@given(T=st.integers(1, 3), h=st.integers(1, 3), w=st.integers(1, 3), seed=st.integers(0, 2**31 - 1))
def test_perfect_reconstruction_2d(T, h, w, seed):
    x = np.random.default_rng(seed).standard_normal((1, 3, T, 4 * h, 4 * w))
    np.testing.assert_allclose(haar.haar3d_inv(haar.haar3d_fwd(x, 0), 0), x, atol=1e-12)


def test_parseval_on_padded_sequence():
    x = np.random.default_rng(3).standard_normal((2, 3, 9, 8, 16))
    y = haar.haar3d_fwd(x, 2)
    lhs = np.sum(y ** 2)
    rhs = np.sum(x ** 2) + 3 * np.sum(x[:, :, 0] ** 2)
    assert abs(lhs - rhs) < 1e-10 * rhs


def test_constant_video_only_dc_channels():
    v = 0.37
    x = np.full((1, 3, 9, 8, 8), v)
    y = haar.haar3d_fwd(x, 2)
    for ch in range(192):
        expect = 8 * v if ch < 3 else 0.0
        np.testing.assert_allclose(y[0, ch], expect, atol=1e-14)
    y2 = haar.haar3d_fwd(x, 0)
    for ch in range(48):
        np.testing.assert_allclose(y2[0, ch], 4 * v if ch < 3 else 0.0, atol=1e-14)


def test_first_latent_frame_has_no_temporal_detail():
    x = np.random.default_rng(4).standard_normal((1, 3, 5, 8, 8))
    y = haar.haar3d_fwd(x, 2)
    C = 3
    for ch in range(192):
        s2, rem = divmod(ch, 8 * C)
        s1 = rem // C
        if (s2 >> 2) or (s1 >> 2):          # any temporal-high band
            assert np.all(y[0, ch, 0] == 0.0)


def test_single_frame_3d_vs_2d():
    x = np.random.default_rng(5).standard_normal((1, 3, 1, 8, 12))
    y3 = haar.haar3d_fwd(x, 2)
    y2 = haar.haar3d_fwd(x, 0)
    C = 3
    for ch in range(192):
        s2, rem = divmod(ch, 8 * C)
        s1, c = divmod(rem, C)
        if (s2 >> 2) or (s1 >> 2):
            assert np.all(y3[0, ch] == 0.0)
        else:
            ch2 = (s2 & 3) * 4 * C + (s1 & 3) * C + c
            np.testing.assert_allclose(y3[0, ch], 2.0 * y2[0, ch2], atol=1e-13)


def test_one_copy_per_level_reading_is_identical():
    """Repeating frame 0 once before each level gives the same coefficients."""
    x = np.random.default_rng(6).standard_normal((1, 2, 9, 8, 8))
    a = haar.haar_level(np.concatenate([x[:, :, :1], x], axis=2), (2, 3, 4))
    a = haar.haar_level(np.concatenate([a[:, :, :1], a], axis=2), (2, 3, 4))
    np.testing.assert_allclose(a, haar.haar3d_fwd(x, 2), atol=1e-13)


def test_page_shapes():
    g = GOLDEN["haar2d_shapes"]["chw"]
    x = np.zeros((1,) + (g[0][0], 1) + tuple(g[0][1:]))
    one = haar.haar_level(x, (3, 4))
    assert one.shape[1:2] + one.shape[3:] == tuple(g[1])
    two = haar.haar3d_fwd(x, 0)
    assert two.shape[1:2] + two.shape[3:] == tuple(g[2])
    for T, t in GOLDEN["latent_frames"]["pairs"]:
        assert haar.latent_frames(T) == t
    for T in GOLDEN["context_frames"]["T"]:
        y = haar.haar3d_fwd(np.zeros((1, 3, T, 4, 4)), 2)
        assert y.shape == (1, 3 * 8 ** GOLDEN["channel_growth_3d"]["levels"], 1 + (T - 1) // 4, 1, 1)
    inp = GOLDEN["api_shapes"]["input"]
    assert haar.latent_frames(inp[2]) == GOLDEN["api_shapes"]["codes"][2]


def test_bad_shapes_raise():
    with pytest.raises(ValueError):
        haar.haar3d_fwd(np.zeros((1, 3, 4, 8, 8)), 2)
    with pytest.raises(ValueError):
        haar.haar3d_fwd(np.zeros((1, 3, 5, 6, 8)), 2)


def test_causality():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((1, 3, 17, 8, 8))
    y = haar.haar3d_fwd(x, 2)
    for tau in range(17):
        xp = x.copy()
        xp[:, :, tau] += rng.standard_normal(xp[:, :, tau].shape)
        yp = haar.haar3d_fwd(xp, 2)
        first_touched = (tau + 3) // 4
        assert np.array_equal(y[:, :, :first_touched], yp[:, :, :first_touched])
        assert not np.array_equal(y[:, :, first_touched], yp[:, :, first_touched])


def test_inverse_is_transpose_on_detail_blocks():
    """For a latent block other than 0 the inverse of a one-hot coefficient is
    the matching row of the block matrix."""
    M3 = np.kron(np.kron(M4, M4), M4)
    for rows in [(0, 0, 0), (3, 1, 2), (2, 3, 3)]:
        ch = channel_of(rows, 1, 0)
        y = np.zeros((1, 64, 2, 1, 1))
        y[0, ch, 1, 0, 0] = 1.0
        x = haar.haar3d_inv(y, 2)
        assert x.shape == (1, 1, 5, 4, 4)
        r = rows[0] * 16 + rows[1] * 4 + rows[2]
        np.testing.assert_allclose(x[0, 0, 1:5].ravel(), M3[r], atol=1e-15)
        assert np.all(x[0, 0, 0] == 0)


def test_continuation_chunks_equal_the_whole_clip():
    """A clip encoded as a first chunk (frames 0 .. 4a, causal first frame) followed by
    continuation chunks of 4k frames gives exactly the whole clip's latent frames, and
    the inverse of each chunk gives back its frames: the causal design makes a latent
    frame depend only on its own and earlier frames."""
    rng = np.random.default_rng(31)
    x = rng.normal(size=(2, 3, 1 + 4 * 5, 8, 12))
    whole = haar.haar3d_fwd(x, 2)
    parts = [haar.haar3d_fwd(x[:, :, :1 + 4 * 2], 2), haar.haar3d_fwd(x[:, :, 9:13], 3),
             haar.haar3d_fwd(x[:, :, 13:], 3)]
    assert [p.shape[2] for p in parts] == [3, 1, 2]
    assert np.array_equal(np.concatenate(parts, axis=2), whole)
    back = [haar.haar3d_inv(parts[0], 2), haar.haar3d_inv(parts[1], 3), haar.haar3d_inv(parts[2], 3)]
    assert np.max(np.abs(np.concatenate(back, axis=2) - x)) < 1e-12
    with pytest.raises(ValueError):
        haar.haar3d_fwd(x[:, :, :6], 3)
