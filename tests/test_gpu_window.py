"""Sliding windows on the GPU: padding and cropping are bit-exact copies checked
element by element against the oracle (every vector width and ragged-row path of
the kernels, both dtypes, one-frame windows, pads longer than the window, 720p and
1080p frames), and a clip of any length goes through pad -> Haar -> inverse Haar ->
crop window by window back to itself, as the oracle's windowed round trip does.  The
windowed Haar calls (padding inside the forward transform's loads, cropping inside the
inverse's stores) equal the separate pad / crop calls bit for bit and the oracle's padded
transform within float32 rounding."""

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import haar as ohaar
from oracle import window as ow
from tests.gpu_helpers import assert_rel, log

pytestmark = pytest.mark.gpu

cvt = pytest.importorskip("causal_video_tokenizer_amd")
DEV = "cuda:0"


def clip(shape, seed, dtype):
    a = si.normal(shape, seed, 1.0).astype(np.float32)
    if dtype == "bf16":
        bits = si.to_bf16_bits(a)
        t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
        return t.to(DEV), bits
    return torch.from_numpy(a).to(DEV), a.view(np.uint32)


def host_bits(t):
    a = t.detach().cpu().contiguous()
    return a.view(torch.int16).numpy().view(np.uint16) if a.dtype == torch.bfloat16 else a.numpy().view(np.uint32)


PAD_CASES = [
    # B, C, T, H, W, t0, nt, Tp, Hp, Wp, dtype
    (1, 3, 40, 30, 48, 34, 6, 9, 32, 48, "bf16"),     # 16-byte vectors, source rows aligned
    (1, 3, 40, 30, 50, 34, 6, 9, 32, 56, "bf16"),     # 16-byte vectors, ragged source rows
    (2, 3, 21, 13, 50, 17, 4, 5, 16, 52, "bf16"),     # 8-byte vectors, ragged rows
    (1, 2, 10, 6, 44, 2, 5, 5, 8, 44, "bf16"),        # 8-byte vectors, aligned rows
    (1, 2, 9, 5, 7, 3, 2, 9, 5, 7, "bf16"),           # single elements; pad longer than the window
    (1, 3, 18, 8, 16, 17, 1, 5, 8, 16, "f32"),        # one-frame window
    (1, 3, 40, 30, 50, 0, 17, 17, 32, 52, "f32"),     # full window, 16-byte f32 vectors, ragged rows
    (2, 1, 12, 7, 9, 5, 7, 13, 8, 10, "f32"),         # 8-byte f32 vectors
]


@pytest.mark.parametrize("case", PAD_CASES)
def test_pad_bit_exact(case):
    B, C, T, H, W, t0, nt, Tp, Hp, Wp, dt = case
    log(f"pad {case}")
    x, xb = clip((B, C, T, H, W), 700 + T + W, dt)
    y = cvt.video_pad(x, t0, nt, Tp, Hp, Wp)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y), ow.pad_window(xb, t0, nt, Tp, Hp, Wp))


@pytest.mark.parametrize("case", PAD_CASES)
def test_unpad_bit_exact_and_leaves_other_frames(case):
    B, C, T, H, W, t0, nt, Tp, Hp, Wp, dt = case
    log(f"unpad {case}")
    y, yb = clip((B, C, Tp, Hp, Wp), 710 + Tp + Wp, dt)
    dst, db = clip((B, C, T, H, W), 720 + T, dt)
    cvt.video_unpad(y, dst, t0, nt)
    torch.cuda.synchronize()
    want = db.copy()
    ow.unpad_window(yb, want, t0, nt)
    assert np.array_equal(host_bits(dst), want)


@pytest.mark.parametrize("shape,t0,nt,s_align", [((1, 3, 40, 720, 1280), 34, 6, 16),
                                                 ((1, 3, 20, 1080, 1920), 17, 3, 16)])
def test_pad_and_crop_full_frames(shape, t0, nt, s_align):
    B, C, T, H, W = shape
    log(f"full-frame window {shape} t0={t0} nt={nt}")
    _, _, _, Tp, Hp, Wp = cvt.video_window(T, H, W, 17, 8, s_align, t0 // 17)
    x, xb = clip(shape, 730, "bf16")
    y = cvt.video_pad(x, t0, nt, Tp, Hp, Wp)
    dst = torch.zeros_like(x)
    cvt.video_unpad(y, dst, t0, nt)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y), ow.pad_window(xb, t0, nt, Tp, Hp, Wp))
    got = host_bits(dst)
    assert np.array_equal(got[:, :, t0:t0 + nt], xb[:, :, t0:t0 + nt])
    assert not got[:, :, :t0].any() and not got[:, :, t0 + nt:].any()


@pytest.mark.parametrize("T,H,W", [(40, 30, 50), (23, 12, 20), (1, 8, 8)])
def test_windowed_haar_round_trip(T, H, W):
    """f32 clip -> per window: pad (t_align 4, s_align 4) -> Haar (2 levels) -> inverse -> crop."""
    log(f"windowed Haar round trip T={T} H={H} W={W}")
    x, _ = clip((1, 3, T, H, W), 740 + T, "f32")
    x = x.clamp_(-1, 1)
    out = torch.empty_like(x)
    for t0, nt, Tp, Hp, Wp in cvt.video_windows(T, H, W, 17, 4, 4):
        win = cvt.video_pad(x, t0, nt, Tp, Hp, Wp)
        rec = cvt.haar3d_inv(cvt.haar3d_fwd(win, 2, out_dtype=torch.float32))
        cvt.video_unpad(rec, out, t0, nt)
    torch.cuda.synchronize()
    x64 = x.cpu().double().numpy()
    ref = ow.windowed(x64, lambda w: ohaar.haar3d_inv(ohaar.haar3d_fwd(w)), 17, 4, 4)
    assert_rel(out.cpu().double().numpy(), ref, 1e-5, "windowed round trip vs oracle")
    assert np.max(np.abs(out.cpu().double().numpy() - x64)) < 1e-5


HAAR_WIN_CASES = [
    # B, C, T, H, W, t0, nt, Tp, Hp, Wp, temporal_levels, x dtype, coefficient dtype, layout
    (1, 3, 40, 30, 48, 34, 6, 9, 32, 48, 2, "bf16", "bf16", "NTHWC"),   # staged kernels, W % 4 == 0
    (1, 3, 40, 30, 50, 34, 6, 9, 32, 52, 2, "bf16", "bf16", "NTHWC"),   # ragged rows: element path
    (2, 3, 21, 13, 300, 17, 4, 9, 16, 304, 2, "f32", "f32", "NTHWC"),   # 76 columns of 4: two chunks
    (1, 2, 10, 6, 44, 2, 5, 5, 8, 48, 2, "bf16", "f32", "NCTHW"),       # generic kernels
    (1, 3, 9, 5, 7, 3, 2, 9, 8, 8, 2, "f32", "bf16", "NTHWC"),          # pad longer than the window
    (1, 3, 18, 8, 16, 17, 1, 5, 8, 16, 2, "bf16", "bf16", "NTHWC"),     # one-frame window
    (1, 3, 12, 7, 22, 4, 5, 6, 8, 24, 0, "f32", "f32", "NTHWC"),        # per-frame patcher
    (1, 1, 12, 9, 20, 7, 5, 5, 12, 20, 0, "bf16", "bf16", "NCTHW"),
]


def _dtype(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


@pytest.mark.parametrize("case", HAAR_WIN_CASES)
def test_haar_fwd_window_equals_pad_then_haar(case):
    B, C, T, H, W, t0, nt, Tp, Hp, Wp, tl, xdt, ydt, lay = case
    log(f"haar fwd window {case}")
    x, xb = clip((B, C, T, H, W), 750 + T + W, xdt)
    y = cvt.haar3d_fwd_window(x, t0, nt, Tp, Hp, Wp, tl, out_dtype=_dtype(ydt), layout=lay)
    y2 = cvt.haar3d_fwd(cvt.video_pad(x, t0, nt, Tp, Hp, Wp), tl, out_dtype=_dtype(ydt), layout=lay)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y), host_bits(y2))
    x64 = x.cpu().double().numpy()
    ref = ohaar.haar3d_fwd(ow.pad_window(x64, t0, nt, Tp, Hp, Wp), tl)
    assert_rel(y.cpu().double().numpy(), ref, 1e-5 if ydt == "f32" else 1e-2, "windowed Haar vs oracle")


@pytest.mark.parametrize("case", HAAR_WIN_CASES)
def test_haar_inv_window_equals_haar_then_crop(case):
    B, C, T, H, W, t0, nt, Tp, Hp, Wp, tl, xdt, ydt, lay = case
    log(f"haar inv window {case}")
    G = 64 if tl == 2 else 16
    Tq = 1 + (Tp - 1) // 4 if tl == 2 else Tp
    y, _ = clip((B, G * C, Tq, Hp // 4, Wp // 4), 760 + Tp + Wp, ydt)
    if lay == "NTHWC":
        y = y.contiguous(memory_format=torch.channels_last_3d)
    dst, _ = clip((B, C, T, H, W), 770 + T, xdt)
    want = dst.clone()
    cvt.haar3d_inv_window(y, dst, t0, nt, tl)
    cvt.video_unpad(cvt.haar3d_inv(y, tl, out_dtype=_dtype(xdt)), want, t0, nt)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(dst), host_bits(want))


def test_windowed_haar_fused_round_trip_1080p():
    """The 50-frame 1080p clip in windows of 17 (padded to 1088 rows): the fused forward and
    inverse give the unfused windowed round trip's coefficients and pixels bit for bit."""
    B, C, T, H, W = 1, 3, 50, 1080, 1920
    log(f"fused windowed Haar round trip {(B, C, T, H, W)}")
    x, _ = clip((B, C, T, H, W), 780, "bf16")
    out, out2 = torch.zeros_like(x), torch.zeros_like(x)
    for t0, nt, Tp, Hp, Wp in cvt.video_windows(T, H, W, 17, 4, 16):
        c = cvt.haar3d_fwd_window(x, t0, nt, Tp, Hp, Wp, 2)
        c2 = cvt.haar3d_fwd(cvt.video_pad(x, t0, nt, Tp, Hp, Wp), 2)
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), c2.view(torch.int16))
        cvt.haar3d_inv_window(c, out, t0, nt, 2)
        cvt.video_unpad(cvt.haar3d_inv(c2, 2), out2, t0, nt)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert (out.float() - x.float()).abs().max().item() < 0.1
