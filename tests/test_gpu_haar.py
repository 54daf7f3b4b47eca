"""GPU parity of cvt_haar3d_fwd / cvt_haar3d_inv against the float64 oracle."""

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import bf16 as obf16
from oracle import haar as ohaar
from tests.gpu_helpers import (assert_bf16_ulp, assert_rel, bits_to_torch, f32_to_torch, log, to_bits,
                               to_f64)

pytestmark = pytest.mark.gpu

cvt = pytest.importorskip("causal_video_tokenizer_amd")


def video(shape, seed, dtype, gen="sin"):
    a = (si.video_sin if gen == "sin" else si.video_trans)(shape, seed)
    if dtype == "bf16":
        bits = si.to_bf16_bits(a)
        return bits_to_torch(bits), obf16.decode(bits)
    return f32_to_torch(a), a.astype(np.float64)


CASES = [
    # shape, temporal_levels, in dtype, out dtype, layout
    ((1, 3, 1, 64, 64), 0, "f32", "f32", "NTHWC"),      # single image, 2D patcher
    ((1, 3, 1, 64, 64), 0, "f32", "f32", "NCTHW"),
    ((1, 3, 17, 256, 256), 2, "bf16", "bf16", "NTHWC"),  # short video
    ((2, 3, 9, 16, 280), 2, "bf16", "bf16", "NTHWC"),   # W' = 70: ragged 64-wide runs, B = 2
    ((2, 3, 9, 16, 280), 2, "f32", "f32", "NCTHW"),
    ((1, 3, 5, 8, 264), 2, "f32", "bf16", "NTHWC"),
    ((1, 3, 5, 8, 264), 2, "bf16", "f32", "NTHWC"),
    ((1, 3, 1, 8, 8), 2, "f32", "f32", "NTHWC"),        # T = 1 through the 3D patcher
    ((1, 3, 3, 12, 20), 0, "bf16", "bf16", "NTHWC"),    # 2D patcher on several frames
    ((1, 2, 5, 8, 8), 2, "f32", "f32", "NTHWC"),        # C != 3 (runtime channel count)
    ((1, 5, 5, 8, 8), 2, "bf16", "bf16", "NTHWC"),      # C = 5, LDS-staged rows of 160 dwords
    ((1, 5, 5, 8, 8), 2, "f32", "f32", "NTHWC"),        # rows too long for LDS staging: direct stores
    ((1, 8, 5, 8, 12), 2, "bf16", "bf16", "NTHWC"),
]


@pytest.mark.parametrize("shape,tl,idt,odt,lay", CASES)
def test_haar_fwd_inv_parity(shape, tl, idt, odt, lay):
    log(f"haar case shape={shape} tl={tl} in={idt} out={odt} layout={lay}")
    x, x64 = video(shape, 11, idt)
    tdt = torch.bfloat16 if odt == "bf16" else torch.float32
    y = cvt.haar3d_fwd(x, temporal_levels=tl, out_dtype=tdt, layout=lay)
    torch.cuda.synchronize()
    o = ohaar.haar3d_fwd(x64, tl)
    assert tuple(y.shape) == o.shape
    if lay == "NTHWC":
        assert y.is_contiguous(memory_format=torch.channels_last_3d)
    if odt == "bf16":
        assert_bf16_ulp(to_bits(y), o, "fwd")
    else:
        assert_rel(to_f64(y), o, 1e-5, "fwd")
    # inverse of the GPU coefficients against the oracle inverse of the same bits
    y64 = to_f64(y)
    xr = cvt.haar3d_inv(y, temporal_levels=tl, out_dtype=x.dtype)
    torch.cuda.synchronize()
    orr = ohaar.haar3d_inv(y64, tl)
    assert tuple(xr.shape) == orr.shape == x64.shape
    if x.dtype == torch.bfloat16:
        assert_bf16_ulp(to_bits(xr), orr, "inv")
    else:
        assert_rel(to_f64(xr), orr, 1e-5, "inv")


def test_inverse_of_arbitrary_coefficients():
    """Coefficients outside the forward range (latent block 0 inconsistent):
    the inverse keeps reconstructed padded frame 3 of block 0."""
    y = si.normal((2, 192, 4, 3, 70), 5, 1.0)
    for lay in ("NCTHW", "NTHWC"):
        yt = f32_to_torch(y, channels_last=(lay == "NTHWC"))
        xr = cvt.haar3d_inv(yt, temporal_levels=2)
        torch.cuda.synchronize()
        assert_rel(to_f64(xr), ohaar.haar3d_inv(y.astype(np.float64), 2), 1e-5, f"inv {lay}")


def test_fwd_determinism_and_causality():
    x, _ = video((1, 3, 17, 32, 64), 12, "bf16")
    y1 = to_bits(cvt.haar3d_fwd(x))
    y2 = to_bits(cvt.haar3d_fwd(x))
    assert np.array_equal(y1, y2)
    for tau in (0, 1, 4, 5, 12, 16):
        xp = x.clone()
        xp[:, :, tau] = -xp[:, :, tau]
        yp = to_bits(cvt.haar3d_fwd(xp))
        first = (tau + 3) // 4
        assert np.array_equal(y1[:, :, :first], yp[:, :, :first]), tau
        assert not np.array_equal(y1[:, :, first], yp[:, :, first]), tau


def _crop_check(x, y, gen_bits, H, W, regions, tl=2):
    """Compare GPU coefficients with the oracle on 4-aligned spatial crops of
    the pixel input over the full time axis (the transform is block-local)."""
    for (r0, r1, c0, c1) in regions:
        xc = obf16.decode(gen_bits[:, :, :, 4 * r0:4 * r1, 4 * c0:4 * c1])
        o = ohaar.haar3d_fwd(xc, tl)
        g = y[:, :, :, r0:r1, c0:c1]
        assert_bf16_ulp(g, o, f"crop rows {r0}:{r1} cols {c0}:{c1}")


@pytest.mark.parametrize("name", ["c3_cv8x8x8_720p_121f", "c4_dv8x16x16_720p_49f"])
def test_full_size_720p_sampled(name):
    wl = si.WORKLOADS[name]
    shape = wl["x"]
    log(f"full-size haar {name} {shape}")
    bits = si.to_bf16_bits(si.video_trans(shape, wl["seed"]))
    x = bits_to_torch(bits)
    y = cvt.haar3d_fwd(x)
    torch.cuda.synchronize()
    B, C, T, H, W = shape
    Hq, Wq = H // 4, W // 4
    ybits = to_bits(y)
    regions = [(0, 6, 0, 8), (87, 93, 150, 166), (Hq - 5, Hq, Wq - 9, Wq)]
    _crop_check(x, ybits, bits, H, W, regions)
    # round trip through the inverse on the full tensor, checked on the same crops
    xr = cvt.haar3d_inv(y)
    torch.cuda.synchronize()
    xrb = to_bits(xr)
    for (r0, r1, c0, c1) in regions:
        o = ohaar.haar3d_inv(obf16.decode(ybits[:, :, :, r0:r1, c0:c1]), 2)
        assert_bf16_ulp(xrb[:, :, :, 4 * r0:4 * r1, 4 * c0:4 * c1], o, f"inv crop {r0}:{r1},{c0}:{c1}")
    del x, y, xr
    torch.cuda.empty_cache()


def test_decode_side_inverse_full_size_sampled():
    """8 x 192 x 13 x 90 x 160 coefficients -> 8 x 3 x 49 x 360 x 640 pixels."""
    shape = (8, 192, 13, 90, 160)
    ybits = si.to_bf16_bits(si.normal(shape, 1005, 0.5))
    y = bits_to_torch(ybits, channels_last=True)
    xr = cvt.haar3d_inv(y)
    torch.cuda.synchronize()
    assert tuple(xr.shape) == (8, 3, 49, 360, 640)
    xb = to_bits(xr)
    for b, (r0, r1, c0, c1) in [(0, (0, 4, 0, 4)), (3, (40, 46, 60, 70)), (7, (86, 90, 150, 160))]:
        o = ohaar.haar3d_inv(obf16.decode(ybits[b:b + 1, :, :, r0:r1, c0:c1]), 2)
        assert_bf16_ulp(xb[b:b + 1, :, :, 4 * r0:4 * r1, 4 * c0:4 * c1], o, f"b={b} crop")


def test_errors_raise():
    x = torch.zeros((1, 3, 4, 8, 8), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(cvt.CvtError):
        cvt.haar3d_fwd(x)
