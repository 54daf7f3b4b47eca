"""Pins of the FSQ oracle: exhaustive index round trips, closed-form special
values, symmetry, monotonicity, saturation and invalid inputs."""

import json
import os

import numpy as np
import pytest

from oracle import fsq

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))
LEVELS = tuple(GOLDEN["fsq"]["levels"])


def z_of(vals):
    """[6] values per position -> a [1, 6, N] latent."""
    return np.asarray(vals, dtype=np.float64).T[None]


def test_page_levels_and_codebook():
    assert LEVELS == fsq.DEFAULT_LEVELS
    assert fsq.codebook_size(LEVELS) == GOLDEN["fsq"]["codebook"] == 8 * 8 * 8 * 5 * 5 * 5
    assert tuple(fsq.basis(LEVELS)) == (1, 8, 64, 512, 2560, 12800)


def test_zero_and_small_latents_map_to_centre():
    # z = 0 is the centre code of every channel: digits (4,4,4,2,2,2)
    centre = 4 + 4 * 8 + 4 * 64 + 2 * 512 + 2 * 2560 + 2 * 12800
    assert centre == 32036
    for v in [0.0, -0.1, 0.1, 0.14, -0.14]:
        idx, codes, _ = fsq.quantize(np.full((1, 6, 1), v), LEVELS)
        assert idx[0, 0] == 32036, v
        assert np.all(codes == 0.0)


def test_saturation():
    idx, codes, _ = fsq.quantize(np.full((1, 6, 2), 0.0) + np.array([np.inf, -np.inf])[None, None], LEVELS)
    assert idx[0, 0] == 63999 and idx[0, 1] == 0
    np.testing.assert_array_equal(codes[0, :, 0], [0.75, 0.75, 0.75, 1, 1, 1])
    np.testing.assert_array_equal(codes[0, :, 1], [-1, -1, -1, -1, -1, -1])
    big, _, _ = fsq.quantize(np.full((1, 6, 1), 50.0), LEVELS)
    assert big[0, 0] == 63999


def lattice_centre(q, L, eps=1e-3):
    """The latent whose bound is exactly the integer q (inverse of tanh)."""
    h = (L - 1) * (1 + eps) / 2
    o = 0.5 if L % 2 == 0 else 0.0
    return np.arctanh((q + o) / h) - np.arctanh(o / h)


def test_all_indices_round_trip():
    n = 64000
    idx = np.arange(n)
    # digits by repeated division, independent of the oracle's basis
    rem = idx.copy()
    digs = []
    for L in LEVELS:
        digs.append(rem % L)
        rem = rem // L
    assert np.all(rem == 0)
    z = np.stack([lattice_centre(d - L // 2, L) for d, L in zip(digs, LEVELS)])[None]
    got, codes, dist = fsq.quantize(z, LEVELS)
    np.testing.assert_array_equal(got[0], idx)
    assert np.all(dist[0] > 0.49)
    deq, bad = fsq.dequantize(idx[None], LEVELS)
    assert bad == 0
    for i, L in enumerate(LEVELS):
        np.testing.assert_array_equal(deq[0, i], (digs[i] - L // 2) / (L // 2))
    np.testing.assert_array_equal(deq, codes)


def test_distinct_codes_per_channel_and_monotone():
    zs = np.linspace(-6, 6, 20001)
    for i, L in enumerate(LEVELS):
        z = np.zeros((1, 6, zs.size))
        z[0, i] = zs
        idx, codes, _ = fsq.quantize(z, LEVELS)
        ci = codes[0, i]
        half = L // 2
        assert sorted(set(ci.tolist())) == [(d - half) / half for d in range(L)]
        assert np.all(np.diff(ci) >= 0)
        assert np.all(np.diff(idx[0]) >= 0)


def test_symmetry_pins_shift_and_offset():
    rng = np.random.default_rng(1)
    u = rng.uniform(0, 3, 5000)
    for i, L in enumerate(LEVELS):
        h = (L - 1) * (1 + 1e-3) / 2
        if L % 2:
            qa = np.rint(fsq.bound(u, L))
            qb = np.rint(fsq.bound(-u, L))
            np.testing.assert_array_equal(qa, -qb)
        else:
            s = np.arctanh(0.5 / h)
            qa = np.rint(fsq.bound(-s + u, L))
            qb = np.rint(fsq.bound(-s - u, L))
            np.testing.assert_array_equal(qa, -1 - qb)
        assert abs(fsq.bound(0.0, L)) < 1e-15


def test_decision_changes_exactly_at_breakpoints():
    for i, L in enumerate(LEVELS):
        h = (L - 1) * (1 + 1e-3) / 2
        o = 0.5 if L % 2 == 0 else 0.0
        s = np.arctanh(o / h)
        half = L // 2
        for j in range(-half, L - half - 1):
            zb = np.arctanh((j + 0.5 + o) / h) - s
            lo = np.rint(fsq.bound(zb - 1e-9, L))
            hi = np.rint(fsq.bound(zb + 1e-9, L))
            assert lo == j and hi == j + 1


def test_nan_and_invalid():
    z = np.zeros((1, 6, 3))
    z[0, 2, 1] = np.nan
    idx, codes, _ = fsq.quantize(z, LEVELS)
    assert idx[0, 1] == -1 and idx[0, 0] == 32036
    assert np.all(np.isnan(codes[0, :, 1]))
    deq, bad = fsq.dequantize(np.array([[0, -1, 64000, 63999, 2**31 - 1]]), LEVELS)
    assert bad == 3
    assert np.all(np.isnan(deq[0, :, 1:3])) and np.all(np.isnan(deq[0, :, 4]))
    np.testing.assert_array_equal(deq[0, :, 0], [-1] * 6)


def test_level_mismatch_raises():
    with pytest.raises(ValueError):
        fsq.quantize(np.zeros((1, 5, 2)), LEVELS)


def test_float32_variant_agrees_off_the_boundary():
    z = np.random.default_rng(2).standard_normal((1, 6, 200000)).astype(np.float32) * 1.5
    i64, _, dist = fsq.quantize(z.astype(np.float64), LEVELS)
    i32 = fsq.quantize_f32(z, LEVELS)
    off = dist > 1e-6
    np.testing.assert_array_equal(i64[off], i32[off])
