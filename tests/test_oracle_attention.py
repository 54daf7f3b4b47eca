"""Pins of the factorized causal self-attention oracle: brute force, torch's
scaled_dot_product_attention in float64, closed forms, invariants, causality and
the head/layout convention."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as at


def brute_core(q, k, v, causal):
    """Pure-Python loops with math.exp: softmax(q k^T / sqrt(d)) v, tiny inputs."""
    n, d = len(q), len(q[0])
    out = []
    for i in range(n):
        keys = range(i + 1) if causal else range(n)
        s = [sum(q[i][c] * k[j][c] for c in range(d)) / math.sqrt(d) for j in keys]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        out.append([sum(e[jj] * v[j][c] for jj, j in enumerate(keys)) / z for c in range(d)])
    return np.array(out)


@pytest.mark.parametrize("causal", [False, True])
def test_core_brute_force(causal):
    rng = np.random.default_rng(1)
    q, k, v = (rng.normal(size=(6, 5)) for _ in range(3))
    got = at.attention(q, k, v, causal=causal)
    assert np.max(np.abs(got - brute_core(q.tolist(), k.tolist(), v.tolist(), causal))) < 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_core_matches_torch_sdpa_float64(causal):
    rng = np.random.default_rng(2)
    q, k, v = (rng.normal(size=(3, 4, 17, 8)) * 2 for _ in range(3))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal).numpy()
    assert np.max(np.abs(at.attention(q, k, v, causal=causal) - ref)) < 1e-12


def test_two_token_scale_by_hand():
    # q0 . k0 = 2, d = 4: score 2 / sqrt(4) = 1 against 0, so the weight of v0 is e / (1 + e)
    q = np.array([[2.0, 0, 0, 0], [0, 0, 0, 0]])
    k = np.array([[1.0, 0, 0, 0], [0, 0, 0, 0]])
    v = np.array([[1.0, 0, 0, 0], [0, 0, 0, 0]])
    out = at.attention(q, k, v)
    assert abs(out[0, 0] - math.e / (1 + math.e)) < 1e-15
    assert abs(out[1, 0] - 0.5) < 1e-15  # a zero query weighs both keys equally


def test_equal_keys_give_the_mean_of_values():
    rng = np.random.default_rng(3)
    q = rng.normal(size=(9, 4)) * 3
    k = np.tile(rng.normal(size=(1, 4)), (9, 1))
    v = rng.normal(size=(9, 4))
    assert np.max(np.abs(at.attention(q, k, v) - v.mean(axis=0))) < 1e-14
    prefix = np.cumsum(v, axis=0) / np.arange(1, 10)[:, None]
    assert np.max(np.abs(at.attention(q, k, v, causal=True) - prefix)) < 1e-14


def test_causal_first_query_returns_first_value():
    rng = np.random.default_rng(4)
    q, k, v = (rng.normal(size=(2, 7, 6)) * 4 for _ in range(3))
    assert np.array_equal(at.attention(q, k, v, causal=True)[:, 0], v[:, 0])


def test_key_shift_invariance_and_token_permutation():
    rng = np.random.default_rng(5)
    q, k, v = (rng.normal(size=(11, 8)) for _ in range(3))
    base = at.attention(q, k, v)
    # adding one vector to every key adds a per-query constant to the scores
    assert np.max(np.abs(at.attention(q, k + rng.normal(size=(1, 8)), v) - base)) < 1e-12
    perm = rng.permutation(11)
    assert np.max(np.abs(at.attention(q[perm], k[perm], v[perm]) - base[perm])) < 1e-12


def test_sharp_keys_select_their_values():
    # orthogonal queries/keys at scale a: the diagonal score a^2 / sqrt(d) dominates
    d, a = 8, 12.0
    q = k = np.eye(d) * a
    v = np.arange(d * 3, dtype=np.float64).reshape(d, 3)
    out = at.attention(q, k, v)
    leak = (d - 1) * math.exp(-a * a / math.sqrt(d))
    assert np.max(np.abs(out - v)) < leak * np.abs(v).max() * 2


def layout_brute(q, k, v, heads, spatial):
    """Tokens gathered by explicit indexing from [B, C, T, H, W] (head g = channels
    g*d .. g*d+d-1), attended with the core, scattered back."""
    B, C, T, H, W = q.shape
    d = C // heads
    out = np.zeros_like(q, dtype=np.float64)
    for b in range(B):
        for g in range(heads):
            ch = slice(g * d, (g + 1) * d)
            if spatial:
                for t in range(T):
                    tok = lambda x: np.stack([x[b, ch, t, h, w] for h in range(H) for w in range(W)])
                    o = at.attention(tok(q), tok(k), tok(v))
                    for n, (h, w) in enumerate((h, w) for h in range(H) for w in range(W)):
                        out[b, ch, t, h, w] = o[n]
            else:
                for h in range(H):
                    for w in range(W):
                        tok = lambda x: np.stack([x[b, ch, t, h, w] for t in range(T)])
                        o = at.attention(tok(q), tok(k), tok(v), causal=True)
                        for t in range(T):
                            out[b, ch, t, h, w] = o[t]
    return out


@pytest.mark.parametrize("spatial", [True, False])
def test_layout_and_heads_against_explicit_gather(spatial):
    rng = np.random.default_rng(6)
    q, k, v = (rng.normal(size=(2, 12, 4, 3, 5)) for _ in range(3))
    fn = at.spatial_attention if spatial else at.temporal_attention
    got = fn(q, k, v, heads=3)
    assert np.max(np.abs(got - layout_brute(q, k, v, 3, spatial))) < 1e-13


def test_heads_are_independent():
    rng = np.random.default_rng(7)
    q, k, v = (rng.normal(size=(1, 8, 3, 2, 4)) for _ in range(3))
    base = at.spatial_attention(q, k, v, heads=2)
    k2 = k.copy()
    k2[:, 4:] = rng.normal(size=k2[:, 4:].shape)  # change head 1's keys only
    other = at.spatial_attention(q, k2, v, heads=2)
    assert np.array_equal(other[:, :4], base[:, :4])
    assert not np.allclose(other[:, 4:], base[:, 4:])


def test_temporal_causality_bit_exact():
    rng = np.random.default_rng(8)
    q, k, v = (rng.normal(size=(1, 8, 6, 3, 3)) for _ in range(3))
    base = at.temporal_attention(q, k, v, heads=2)
    t0 = 3
    for x in (q, k, v):
        x2 = x.copy()
        x2[:, :, t0:] += rng.normal(size=x2[:, :, t0:].shape)
        args = [x2 if y is x else y for y in (q, k, v)]
        got = at.temporal_attention(*args, heads=2)
        assert np.array_equal(got[:, :, :t0], base[:, :, :t0])
        assert not np.allclose(got[:, :, t0:], base[:, :, t0:])


def test_spatial_attention_ignores_other_frames():
    rng = np.random.default_rng(9)
    q, k, v = (rng.normal(size=(1, 4, 3, 2, 3)) for _ in range(3))
    base = at.spatial_attention(q, k, v, heads=1)
    k2 = k.copy()
    k2[:, :, 1] += 5.0 * rng.normal(size=k2[:, :, 1].shape)
    got = at.spatial_attention(q, k2, v, heads=1)
    assert np.array_equal(got[:, :, 0], base[:, :, 0]) and np.array_equal(got[:, :, 2], base[:, :, 2])


def test_attention_rows_equal_full_rows():
    rng = np.random.default_rng(10)
    q, k, v = (rng.normal(size=(40, 16)) for _ in range(3))
    full = at.attention(q, k, v)
    rows = [0, 7, 39]
    assert np.max(np.abs(at.attention_rows(q[rows], k, v) - full[rows])) < 1e-14


def test_single_frame_temporal_is_identity_on_values():
    rng = np.random.default_rng(11)
    q, k, v = (rng.normal(size=(2, 8, 1, 3, 4)) for _ in range(3))
    assert np.array_equal(at.temporal_attention(q, k, v, heads=4), v)


def test_bad_heads_raise():
    x = np.zeros((1, 6, 1, 2, 2))
    with pytest.raises(ValueError):
        at.spatial_attention(x, x, x, heads=4)
