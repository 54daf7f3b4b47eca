"""GPU parity of the encoder / decoder blocks against the float64 oracle (oracle/blocks.py):
LayerNorm (+ Swish), the residual block (LayerNorm + Swish and the residual add fused
into the temporal conv's epilogue), the stride-2 downsampling block and the upsampling
block whose repetition happens inside the conv's loads.  Criterion |g - o| <= tol (|o| +
rms(o)) on the same bf16 inputs; the upsampling block is also checked bit for bit against
the convolution of the materialized repetition, and the residual block for causality."""

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import bf16 as obf16
from oracle import blocks as ob
from tests.gpu_helpers import assert_rel, bits_to_torch, f32_to_torch, log, rel_report, to_bits, to_f64

pytestmark = pytest.mark.gpu

cvt = pytest.importorskip("causal_video_tokenizer_amd")
TOL = 2e-2
LN_TOL = 1e-2


def bf16_pair(shape, seed, std, cl=False, offset=0.0):
    bits = si.to_bf16_bits(si.normal(shape, seed, std) + np.float32(offset))
    return bits_to_torch(bits, channels_last=cl), obf16.decode(bits)


def f32_pair(shape, seed, std, mean=0.0):
    a = si.normal(shape, seed, std) + np.float32(mean)
    return f32_to_torch(a), a.astype(np.float64)


@pytest.mark.parametrize("C,swish,shape", [(256, True, (1, 3, 5, 16)), (64, False, (2, 2, 3, 7)),
                                           (192, True, (1, 4, 4, 9)), (1024, True, (1, 2, 3, 5)),
                                           (8, True, (1, 1, 6, 6))])
def test_layernorm_parity(C, swish, shape):
    B, T, H, W = shape
    log(f"layernorm C={C} swish={swish} {shape}")
    x, x64 = bf16_pair((B, C, T, H, W), 800 + C, 2.0, cl=True, offset=3.0)
    g, g64 = f32_pair((C,), 801, 0.2, mean=1.0)
    b, b64 = f32_pair((C,), 802, 0.3)
    y = cvt.layernorm3d(x, g, b, swish=swish)
    torch.cuda.synchronize()
    ref = ob.norm_swish(x64, g64, b64) if swish else ob.layer_norm(x64, g64, b64)
    assert_rel(to_f64(y), ref, LN_TOL, "layernorm")
    # in place gives the same bits
    x2 = x.clone(memory_format=torch.channels_last_3d)
    cvt.layernorm3d(x2, g, b, swish=swish, out=x2)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(x2), to_bits(y))


def block_params_dev(C, seed, bias):
    p, ref = {}, {}
    for i, k in enumerate(("ln1_g", "ln2_g")):
        p[k], ref[k] = f32_pair((C,), seed + i, 0.1, mean=1.0)
    for i, k in enumerate(("ln1_b", "ln2_b")):
        p[k], ref[k] = f32_pair((C,), seed + 2 + i, 0.1)
    for i, c in enumerate(("c1", "c2")):
        p[c + "_s"], ref[c + "_s"] = bf16_pair((C, C, 1, 3, 3), seed + 4 + 4 * i, 0.02)
        p[c + "_t"], ref[c + "_t"] = bf16_pair((C, C, 3, 1, 1), seed + 5 + 4 * i, 0.03)
        if bias:
            p[c + "_bs"], ref[c + "_bs"] = f32_pair((C,), seed + 6 + 4 * i, 0.1)
            p[c + "_bt"], ref[c + "_bt"] = f32_pair((C,), seed + 7 + 4 * i, 0.1)
    return p, ref


RES_CASES = [
    # B, C, T, H, W, bias: 64 and 128 channels on the 4-wave 128-channel tiles, 136 and 192 on
    # the 3-wave 192-channel tiles (136: channels past Cout left out of the statistics), 232 and
    # 256 on the 256-channel tiles, 320 on the plain conv + layernorm path
    (1, 64, 5, 7, 9, False),
    (2, 128, 3, 6, 10, True),
    (1, 136, 3, 6, 7, True),
    (1, 192, 4, 5, 8, False),
    (1, 232, 3, 5, 6, True),
    (1, 256, 6, 9, 13, True),
    (1, 320, 2, 4, 6, False),
]


@pytest.mark.parametrize("case", RES_CASES)
def test_resblock_parity(case):
    B, C, T, H, W, bias = case
    log(f"resblock {case}")
    x, x64 = bf16_pair((B, C, T, H, W), 810 + C, 1.0, cl=True)
    p, ref = block_params_dev(C, 820, bias)
    y = cvt.resblock3d(x, p)
    torch.cuda.synchronize()
    o = ob.resblock(x64, ref)
    assert_rel(to_f64(y), o, TOL, "resblock")
    # the residual branch alone, so that a wrong branch cannot hide behind x: its elements
    # carry the output's bf16 rounding (relative to |y|, not to the branch), so the branch is
    # checked in relative L2 norm
    _, _, rel = rel_report(to_f64(y) - x64, o - x64, TOL)
    log(f"  resblock branch relL2={rel:.3g}")
    assert rel < 5e-2


def test_resblock_causality_and_determinism():
    B, C, T, H, W = 1, 128, 6, 5, 8
    x, _ = bf16_pair((B, C, T, H, W), 830, 1.0, cl=True)
    p, _ = block_params_dev(C, 831, True)
    y0 = to_bits(cvt.resblock3d(x, p))
    x2 = x.clone(memory_format=torch.channels_last_3d)
    x2[:, :, 3:] += 1.0
    y2 = to_bits(cvt.resblock3d(x2, p))
    y1 = to_bits(cvt.resblock3d(x, p))
    torch.cuda.synchronize()
    assert np.array_equal(y0, y1)
    assert np.array_equal(y2[:, :, :3], y0[:, :, :3]) and not np.array_equal(y2[:, :, 3:], y0[:, :, 3:])


@pytest.mark.parametrize("C", [256, 320])
def test_resblock_in_place_equals_out_of_place(C):
    # the residual epilogue reads each residual chunk before the same wave overwrites it
    B, T, H, W = 1, 5, 9, 70
    x, _ = bf16_pair((B, C, T, H, W), 835, 1.0, cl=True)
    p, _ = block_params_dev(C, 836, True)
    y = to_bits(cvt.resblock3d(x, p))
    x2 = x.clone(memory_format=torch.channels_last_3d)
    cvt.resblock3d(x2, p, out=x2)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(x2), y)


DOWN_CASES = [
    # B, Cin, Cout, T, H, W, space, time, bias
    (1, 64, 128, 5, 8, 12, True, True, True),
    (2, 192, 256, 2, 10, 6, True, False, False),
    (1, 64, 64, 7, 6, 10, False, True, True),
    (1, 256, 256, 9, 18, 32, True, True, False),     # 9 x 16 output positions per frame: 3 row tiles of 3
    (1, 200, 256, 3, 14, 20, True, True, True),      # K chunk tail on the 3-row tiles, 7 output rows (3 + 3 + 1)
    (2, 64, 64, 3, 10, 150, True, True, True),       # 75 output columns: two column tiles, ragged
    (1, 72, 128, 5, 6, 8, True, False, False),       # input channels not a multiple of the K chunk
    (1, 320, 320, 5, 4, 4, False, True, False),      # temporal above 256 channels (8-wave tiles)
    (1, 64, 48, 5, 8, 8, True, True, True),          # Cout below 64: the implicit-GEMM fallback
]


@pytest.mark.parametrize("case", DOWN_CASES)
def test_downsample_parity(case):
    B, Cin, Cout, T, H, W, space, time, bias = case
    log(f"downsample {case}")
    x, x64 = bf16_pair((B, Cin, T, H, W), 840 + Cin, 1.0, cl=True)
    ws, ws64 = bf16_pair((Cout, Cin, 1, 3, 3), 841, 0.02) if space else (None, None)
    wt, wt64 = bf16_pair((Cout, Cout if space else Cin, 3, 1, 1), 842, 0.03) if time else (None, None)
    bs, bs64 = f32_pair((Cout,), 843, 0.1) if (bias and space) else (None, None)
    bt, bt64 = f32_pair((Cout,), 844, 0.1) if (bias and time) else (None, None)
    y = cvt.downsample3d(x, ws, wt, bs, bt)
    torch.cuda.synchronize()
    assert_rel(to_f64(y), ob.downsample(x64, ws64, wt64, bs64, bt64), TOL, "downsample")


UP_CASES = [
    # B, Cin, Cout, T, H, W, space, time, bias
    (1, 64, 64, 3, 4, 6, True, True, False),
    (2, 128, 64, 2, 5, 7, True, False, True),
    (1, 64, 128, 4, 5, 7, False, True, False),
    (1, 256, 256, 3, 9, 40, True, True, True),       # 80-pixel rows: two column tiles, ragged
]


@pytest.mark.parametrize("case", UP_CASES)
def test_upsample_parity_and_equals_materialized_repeat(case):
    B, Cin, Cout, T, H, W, space, time, bias = case
    log(f"upsample {case}")
    x, x64 = bf16_pair((B, Cin, T, H, W), 850 + Cin, 1.0, cl=True)
    ws, ws64 = bf16_pair((Cout, Cin, 1, 3, 3), 851, 0.02)
    wt, wt64 = bf16_pair((Cout, Cout, 3, 1, 1), 852, 0.03)
    bs, bs64 = f32_pair((Cout,), 853, 0.1) if bias else (None, None)
    bt, bt64 = f32_pair((Cout,), 854, 0.1) if bias else (None, None)
    y = cvt.upsample3d(x, ws, wt, bs, bt, space=space, time=time)
    # the same conv on the repetition written out (torch indexing, test scaffolding only)
    rep = x
    if time:
        rep = torch.cat([rep[:, :, :1], rep[:, :, 1:].repeat_interleave(2, dim=2)], dim=2)
    if space:
        rep = rep.repeat_interleave(2, dim=3).repeat_interleave(2, dim=4)
    rep = rep.contiguous(memory_format=torch.channels_last_3d)
    s = cvt.causal_conv3d_fact(rep, ws, None, b_s=bs)
    y2 = cvt.causal_conv3d_fact(s, None, wt, b_t=bt)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(y), to_bits(y2))
    assert_rel(to_f64(y), ob.upsample(x64, ws64, wt64, bs64, bt64, space, time), TOL, "upsample")


def test_packed_resblock_full_grid_sampled():
    """The route the benchmark times at its size: the residual block on packed weights over the
    31 x 180 x 320 x 256 grid of a 121-frame 720p clip, against the float64 oracle on sampled
    windows (corners and the middle).  The oracle runs on a crop holding each window's
    receptive field (4 frames back, 2 positions each way in space: two factorized convs); where
    the crop meets the tensor's edge it is the tensor's own zero padding."""
    wl = si.WORKLOADS["blocks_cv8x8x8_720p"]
    B, C, T, H, W = wl["x"]
    log(f"packed resblock full grid {wl['x']}")
    xb = si.to_bf16_bits(si.normal((B, C, T, H, W), 840, 1.0))
    x = bits_to_torch(xb, channels_last=True)
    p, ref = block_params_dev(C, 841, True)
    q = dict(p)
    for k in ("c1_s", "c1_t", "c2_s", "c2_t"):
        q[k] = cvt.conv_weights_pack(p[k])
    y = cvt.resblock3d_packed(x, q)
    torch.cuda.synchronize()
    for (t0, t1), (y0, y1), (x0, x1) in [((0, 2), (0, 3), (0, 3)), ((14, 16), (88, 91), (150, 153)),
                                         ((28, 30), (176, 179), (316, 319))]:
        ct, cy, cx = max(t0 - 4, 0), max(y0 - 2, 0), max(x0 - 2, 0)
        crop = obf16.decode(xb[:, :, ct:t1 + 1, cy:min(y1 + 2, H - 1) + 1, cx:min(x1 + 2, W - 1) + 1])
        o = ob.resblock(crop, ref)[:, :, t0 - ct:, y0 - cy:y0 - cy + y1 - y0 + 1, x0 - cx:x0 - cx + x1 - x0 + 1]
        g = to_f64(y[:, :, t0:t1 + 1, y0:y1 + 1, x0:x1 + 1])
        assert g.shape == o.shape == (B, C, t1 - t0 + 1, y1 - y0 + 1, x1 - x0 + 1), (g.shape, o.shape)
        assert_rel(g, o, TOL, f"resblock window t {t0}-{t1} y {y0}-{y1} x {x0}-{x1}")
    del x, y
    torch.cuda.empty_cache()


def _packed_pair(shape, seed, std):
    w, w64 = bf16_pair(shape, seed, std)
    return cvt.conv_weights_pack(w), w64


def test_packed_downsample_full_grid_sampled():
    """The benchmark's downsampling route at its size: packed weights, 31 x 180 x 320 x 256 ->
    16 x 90 x 160, against the oracle on sampled output windows.  Each crop starts on an even
    input row, column and frame, so the stride-2 grid of the crop is the tensor's, and holds
    the window's receptive field (input rows 2 y' - 1 .. 2 y' + 1, frames 2 t' - 2 .. 2 t')."""
    wl = si.WORKLOADS["blocks_cv8x8x8_720p"]
    B, C, T, H, W = wl["x"]
    log(f"packed downsample full grid {wl['x']}")
    xb = si.to_bf16_bits(si.normal((B, C, T, H, W), 850, 1.0))
    x = bits_to_torch(xb, channels_last=True)
    (pws, ws64), (pwt, wt64) = _packed_pair((C, C, 1, 3, 3), 851, 0.02), _packed_pair((C, C, 3, 1, 1), 852, 0.03)
    bs, bs64 = f32_pair((C,), 853, 0.1)
    bt, bt64 = f32_pair((C,), 854, 0.1)
    y = cvt.downsample3d_packed(x, pws, pwt, bs, bt)
    torch.cuda.synchronize()

    def crop(o0, o1, n, temporal):  # input range [c0, c1] and the first wanted crop output
        c0 = max(0, 2 * o0 - 2)
        c1 = 2 * o1 if temporal else min(n - 1, 2 * o1 + 1)
        return c0, c1, o0 - c0 // 2
    for wt_, wy, wx in [((0, 1), (0, 3), (0, 3)), ((8, 9), (44, 47), (80, 83)), ((14, 15), (86, 89), (156, 159))]:
        (t0, t1, jt), (y0, y1, jy), (x0, x1, jx) = crop(*wt_, T, True), crop(*wy, H, False), crop(*wx, W, False)
        o = ob.downsample(obf16.decode(xb[:, :, t0:t1 + 1, y0:y1 + 1, x0:x1 + 1]), ws64, wt64, bs64, bt64)
        o = o[:, :, jt:jt + wt_[1] - wt_[0] + 1, jy:jy + wy[1] - wy[0] + 1, jx:jx + wx[1] - wx[0] + 1]
        g = to_f64(y[:, :, wt_[0]:wt_[1] + 1, wy[0]:wy[1] + 1, wx[0]:wx[1] + 1])
        assert g.shape == o.shape == (B, C, wt_[1] - wt_[0] + 1, wy[1] - wy[0] + 1, wx[1] - wx[0] + 1), (g.shape, o.shape)
        assert_rel(g, o, TOL, f"downsample window t' {wt_} y' {wy} x' {wx}")
    del x, y
    torch.cuda.empty_cache()


def test_packed_upsample_full_grid_sampled():
    """The benchmark's upsampling route at its size: packed weights, 16 x 90 x 160 x 256 ->
    31 x 180 x 320, against the oracle on sampled output windows.  The crops keep every input
    frame (the causal repetition doubles every frame but the first) and the input rows and
    columns whose repetitions the window's 3 x 3 taps reach."""
    wl = si.WORKLOADS["blocks_cv8x8x8_720p"]
    B, C, Ti, Hi, Wi = wl["low"]
    log(f"packed upsample full grid {wl['low']}")
    xb = si.to_bf16_bits(si.normal((B, C, Ti, Hi, Wi), 860, 1.0))
    x = bits_to_torch(xb, channels_last=True)
    (pws, ws64), (pwt, wt64) = _packed_pair((C, C, 1, 3, 3), 861, 0.02), _packed_pair((C, C, 3, 1, 1), 862, 0.03)
    bs, bs64 = f32_pair((C,), 863, 0.1)
    bt, bt64 = f32_pair((C,), 864, 0.1)
    y = cvt.upsample3d_packed(x, pws, pwt, bs, bt)
    torch.cuda.synchronize()

    def crop(o0, o1, n):  # low-resolution input range and the crop output row of o0
        c0, c1 = max(0, (o0 - 1) // 2), min(n - 1, (o1 + 1) // 2)
        return c0, c1, o0 - 2 * c0
    for wt_, wy, wx in [((0, 2), (0, 3), (0, 3)), ((14, 16), (89, 92), (157, 160)), ((28, 30), (176, 179), (316, 319))]:
        (y0, y1, jy), (x0, x1, jx) = crop(*wy, Hi), crop(*wx, Wi)
        o = ob.upsample(obf16.decode(xb[:, :, :, y0:y1 + 1, x0:x1 + 1]), ws64, wt64, bs64, bt64)
        o = o[:, :, wt_[0]:wt_[1] + 1, jy:jy + wy[1] - wy[0] + 1, jx:jx + wx[1] - wx[0] + 1]
        g = to_f64(y[:, :, wt_[0]:wt_[1] + 1, wy[0]:wy[1] + 1, wx[0]:wx[1] + 1])
        assert g.shape == o.shape == (B, C, wt_[1] - wt_[0] + 1, wy[1] - wy[0] + 1, wx[1] - wx[0] + 1), (g.shape, o.shape)
        assert_rel(g, o, TOL, f"upsample window t {wt_} y {wy} x {wx}")
    del x, y
    torch.cuda.empty_cache()
