"""GPU parity of cvt_attention3d (factorized self-attention: spatial flash attention on
bf16 MFMA, causal temporal attention in fp32) against the float64 oracle on the same
bf16 inputs: |g - o| <= 2e-2 (|o| + rms(o)) element by element (bf16 inputs, fp32
softmax and accumulation, bf16 probabilities in the P v product, bf16 output)."""

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import attention as oat
from oracle import bf16 as obf16
from tests.gpu_helpers import assert_rel, bits_to_torch, log, to_bits, to_f64

pytestmark = pytest.mark.gpu

cvt = pytest.importorskip("causal_video_tokenizer_amd")
TOL = 2e-2


def qkv(shape, seed, q_std=1.0):
    out = []
    for i, std in enumerate((q_std, 1.0, 1.0)):
        bits = si.to_bf16_bits(si.normal(shape, seed + i, std))
        out.append((bits_to_torch(bits, channels_last=True), obf16.decode(bits)))
    return out


SPATIAL = [
    # B, C, T, H, W, heads, q_std
    (1, 64, 2, 8, 8, 1, 1.0),       # 64 tokens: one key block, one partial query tile
    (2, 128, 3, 10, 13, 2, 1.0),    # 130 tokens: ragged last key block (2 keys)
    (1, 256, 2, 24, 20, 4, 1.0),    # 480 tokens: 8 key blocks, 2 query tiles
    (1, 64, 1, 40, 40, 1, 3.0),     # 1600 tokens, sharp softmax (scores ~ N(0, 9))
    (1, 192, 1, 7, 9, 3, 2.0),      # 63 tokens, 3 heads
    (1, 64, 2, 9, 15, 2, 1.0),      # head dim 32: 135 tokens, ragged key block and query tile
    (1, 128, 1, 40, 40, 4, 3.0),    # head dim 32, sharp softmax
    (2, 128, 2, 10, 13, 1, 1.0),    # head dim 128: 130 tokens, 32 queries per wave
    (1, 256, 1, 24, 25, 2, 2.0),    # head dim 128: 600 tokens, 10 key blocks
    (1, 48, 2, 6, 11, 3, 1.0),      # head dim 16: the one-thread-per-query kernel
    (1, 192, 1, 9, 9, 1, 1.0),      # head dim 192: three 64-channel output slices
]


@pytest.mark.parametrize("case", SPATIAL)
def test_spatial_parity(case):
    B, C, T, H, W, heads, qs = case
    log(f"spatial attention {case}")
    (q, q64), (k, k64), (v, v64) = qkv((B, C, T, H, W), 300 + C + H, qs)
    o = cvt.attention3d(q, k, v, heads, "spatial")
    torch.cuda.synchronize()
    assert_rel(to_f64(o), oat.spatial_attention(q64, k64, v64, heads), TOL, f"spatial {case}")


TEMPORAL = [
    # B, C, T, H, W, heads, q_std
    (1, 64, 5, 6, 7, 1, 1.0),
    (2, 128, 16, 9, 11, 2, 1.0),     # 99 positions: ragged last position tile
    (1, 128, 23, 5, 7, 2, 1.0),      # 23 frames: three 8-frame row loads per tensor
    (1, 256, 32, 4, 6, 4, 1.5),      # 32 frames: the matrix-core kernel's largest T
    (1, 256, 16, 8, 12, 4, 2.0),
    (1, 64, 31, 5, 5, 2, 1.0),       # head dim 32, 31 frames
    (1, 256, 64, 3, 3, 4, 1.0),      # T * C at the 16384 limit: one position per workgroup
    (1, 512, 40, 3, 4, 8, 1.0),      # T * C = 20480 beyond the LDS tile: one-thread-per-query kernel
    (2, 256, 17, 4, 5, 2, 2.0),      # head dim 128: one-thread-per-query kernel
    (1, 120, 9, 5, 6, 5, 1.0),       # head dim 24
]


@pytest.mark.parametrize("case", TEMPORAL)
def test_temporal_parity(case):
    B, C, T, H, W, heads, qs = case
    log(f"temporal attention {case}")
    (q, q64), (k, k64), (v, v64) = qkv((B, C, T, H, W), 400 + C + T, qs)
    o = cvt.attention3d(q, k, v, heads, "temporal")
    torch.cuda.synchronize()
    assert_rel(to_f64(o), oat.temporal_attention(q64, k64, v64, heads), TOL, f"temporal {case}")


def test_temporal_single_frame_returns_values_bit_exact():
    (q, _), (k, _), (v, _) = qkv((1, 128, 1, 6, 10), 500)
    o = cvt.attention3d(q, k, v, 2, "temporal")
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(o), to_bits(v))


def test_temporal_causality_and_determinism_bit_exact():
    shape = (1, 128, 12, 6, 9)
    (q, _), (k, _), (v, _) = qkv(shape, 510)
    base = to_bits(cvt.attention3d(q, k, v, 2, "temporal"))
    assert np.array_equal(base, to_bits(cvt.attention3d(q, k, v, 2, "temporal")))
    t0 = 5
    for which in range(3):
        args = [x.clone() for x in (q, k, v)]
        args[which][:, :, t0:] += 0.5
        got = to_bits(cvt.attention3d(*args, 2, "temporal"))
        assert np.array_equal(got[:, :, :t0], base[:, :, :t0])
        assert not np.array_equal(got[:, :, t0:], base[:, :, t0:])


def test_spatial_frames_independent_and_deterministic():
    shape = (1, 128, 3, 12, 14)
    (q, _), (k, _), (v, _) = qkv(shape, 520)
    base = to_bits(cvt.attention3d(q, k, v, 2, "spatial"))
    assert np.array_equal(base, to_bits(cvt.attention3d(q, k, v, 2, "spatial")))
    k2 = k.clone()
    k2[:, :, 1] += 1.0
    got = to_bits(cvt.attention3d(q, k2, v, 2, "spatial"))
    assert np.array_equal(got[:, :, 0], base[:, :, 0]) and np.array_equal(got[:, :, 2], base[:, :, 2])
    assert not np.array_equal(got[:, :, 1], base[:, :, 1])


def test_token_grid_full_size_sampled():
    """The 16 x 90 x 160 token grid, 256 channels in 4 heads: spatial outputs at sampled
    queries (every frame, every head, first / last query tiles) against the oracle on the
    full key set of their frame; temporal outputs at sampled positions."""
    wl = si.WORKLOADS["attn_cv8x8x8_720p_tokens"]
    shape, heads = wl["x"], wl["heads"]
    B, C, T, H, W = shape
    d = C // heads
    (q, _), (k, _), (v, _) = qkv(shape, wl["seed"], wl["std"])
    log(f"spatial attention {shape} heads={heads}")
    o = cvt.attention3d(q, k, v, heads, "spatial")
    ot = cvt.attention3d(q, k, v, heads, "temporal")
    torch.cuda.synchronize()
    g_sp, g_tm = to_f64(o), to_f64(ot)
    q64, k64, v64 = (to_f64(x) for x in (q, k, v))
    rng = np.random.default_rng(7)
    N = H * W
    got, ref = [], []
    for t in range(T):
        for g in range(heads):
            ch = slice(g * d, (g + 1) * d)
            toks = lambda x: x[0, ch, t].reshape(d, N).T
            rows = np.unique(np.concatenate([[0, 255, 256, N - 1], rng.integers(0, N, 4)]))
            ref.append(oat.attention_rows(toks(q64)[rows], toks(k64), toks(v64)))
            got.append(toks(g_sp)[rows])
    assert_rel(np.concatenate(got), np.concatenate(ref), TOL, "spatial sampled")
    pos = rng.integers(0, N, 48)
    sub = lambda x: x[:, :, :, pos // W, pos % W][..., None]
    ref_t = oat.temporal_attention(sub(q64), sub(k64), sub(v64), heads)
    assert_rel(sub(g_tm), ref_t, TOL, "temporal sampled")


def test_generic_temporal_causality_and_single_frame_bit_exact():
    """The one-thread-per-query kernel (here head dim 128): a later frame's change leaves
    every earlier frame's output unchanged, and a one-frame clip returns v."""
    shape = (1, 256, 10, 4, 6)
    (q, _), (k, _), (v, _) = qkv(shape, 520)
    base = to_bits(cvt.attention3d(q, k, v, 2, "temporal"))
    k2, v2 = k.clone(), v.clone()
    k2[:, :, 6:] = -k2[:, :, 6:]
    v2[:, :, 6:] = 2 * v2[:, :, 6:]
    pert = to_bits(cvt.attention3d(q, k2, v2, 2, "temporal"))
    assert np.array_equal(base[:, :, :6], pert[:, :, :6])
    assert not np.array_equal(base[:, :, 6:], pert[:, :, 6:])
    (q1, _), (k1, _), (v1, _) = qkv((1, 256, 1, 4, 6), 525)
    o1 = cvt.attention3d(q1, k1, v1, 2, "temporal")
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(o1), to_bits(v1))


def test_invalid_arguments_raise():
    (q, _), (k, _), (v, _) = qkv((1, 128, 2, 4, 4), 530)
    with pytest.raises(cvt.CvtError):
        cvt.attention3d(q, k, v, 32, "spatial")      # head dim 4: not a multiple of 8
    with pytest.raises(cvt.CvtError):
        cvt.attention3d(q, k, v, 3, "temporal")      # 3 does not divide 128
    with pytest.raises(ValueError):
        cvt.attention3d(q.contiguous(), k, v, 2, "spatial")
    with pytest.raises(ValueError):
        cvt.attention3d(q, k, v, 2, "diagonal")
