"""Sliding windows on the GPU: padding and cropping are bit-exact copies checked
element by element against the oracle (every vector width and ragged-row path of
the kernels, both dtypes, one-frame windows, pads longer than the window, 720p and
1080p frames), and a clip of any length goes through pad -> Haar -> inverse Haar ->
crop window by window back to itself, as the oracle's windowed round trip does."""

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
