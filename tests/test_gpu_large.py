"""Activations of 2 GiB or more on the row-tiled conv kernels.

Each tile addresses its region from its own first input row, so the kernels take tensors of
any size; these tests run them where the byte offsets of the last frames lie beyond 2 GiB.
The oracle (float64) recomputes sampled windows from the GPU's actual input bits with enough
causal and spatial context, |g - o| <= 2e-2 (|o| + rms(o)).
"""

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import bf16 as obf16
from oracle import conv as oconv
from oracle import haar as ohaar
from tests.gpu_helpers import assert_rel, bits_to_torch, log, to_bits

pytestmark = pytest.mark.gpu

cvt = pytest.importorskip("causal_video_tokenizer_amd")
TOL = 2e-2


def _w(shape, seed, std=0.02):
    bits = si.to_bf16_bits(si.normal(shape, seed, std))
    return bits_to_torch(bits), obf16.decode(bits)


def _window64(t, f0, f1, r0, r1, c0, c1):
    """bf16 NTHWC device tensor window -> float64 [B, C, n, rows, cols] (exact)."""
    return obf16.decode(to_bits(t[:, :, f0:f1, r0:r1, c0:c1]))


def test_conv_fact_input_above_2gib():
    wl = si.WORKLOADS["large_256x40x270x480"]
    B, C, T, H, W = wl["x"]
    log(f"generating {wl['x']} ({B * C * T * H * W * 2 / 2**30:.2f} GiB in bf16)")
    x = bits_to_torch(si.to_bf16_bits(si.normal(wl["x"], wl["seed"], 1.0)), channels_last=True)
    assert x.numel() * 2 >= 2**31
    ws, ws64 = _w((C, C, 1, 3, 3), wl["seed"] + 1)
    wt, wt64 = _w((C, C, 3, 1, 1), wl["seed"] + 2)
    wp, wp64 = _w((16, C, 1, 1, 1), wl["seed"] + 3)
    y = cvt.causal_conv3d_fact(x, ws, wt)
    lat = cvt.causal_conv3d_fact_proj(x, None, wt, wp)
    torch.cuda.synchronize()
    # windows: output frame t, rows [r0, r1), cols [c0, c1); the last frames sit past 2 GiB
    for t, (r0, r1), (c0, c1) in [(39, (262, 270), (440, 480)), (36, (100, 108), (0, 37)), (33, (0, 4), (200, 233)),
                                  (1, (130, 140), (470, 480))]:
        log(f"  window t={t} rows={r0}:{r1} cols={c0}:{c1}")
        f0 = max(0, t - 2)
        R0, R1, C0, C1 = max(0, r0 - 1), min(H, r1 + 1), max(0, c0 - 1), min(W, c1 + 1)
        xin = _window64(x, f0, t + 1, R0, R1, C0, C1)
        o = oconv.causal_conv3d_fact(xin, ws64, wt64)[:, :, -1:, r0 - R0:r1 - R0, c0 - C0:c1 - C0]
        assert_rel(_window64(y, t, t + 1, r0, r1, c0, c1), o, TOL, "factorized conv")
        xt = _window64(x, f0, t + 1, r0, r1, c0, c1)
        ot = oconv.pointwise(obf16.round_to_bf16(oconv.temporal_conv(xt, wt64)[:, :, -1:]), wp64)
        assert_rel(_window64(lat, t, t + 1, r0, r1, c0, c1), ot, TOL, "temporal conv + 1x1")
    del x, y, lat
    torch.cuda.empty_cache()


def test_clip_1080p_129f_chain_last_frames():
    """Haar -> spatial 192 -> 256 (2.19 GB out) -> temporal 256 -> 256 with the 1x1 -> 16, on a
    129-frame 1080p clip: latent frames 0 and 32 in full, stage by stage."""
    wl = si.WORKLOADS["clip_1080p_129f"]
    log(f"generating {wl['x']}")
    xb = si.to_bf16_bits(si.video_trans(wl["x"], wl["seed"]))
    x = bits_to_torch(xb)
    ws, ws64 = _w((256, 192, 1, 3, 3), wl["seed"] + 1)
    wt, wt64 = _w((256, 256, 3, 1, 1), wl["seed"] + 2)
    wp, wp64 = _w((16, 256, 1, 1, 1), wl["seed"] + 3)
    hz = cvt.haar3d_fwd(x)
    s1 = cvt.causal_conv3d_fact(hz, ws, None)
    assert s1.numel() * 2 >= 2**31
    lat = cvt.causal_conv3d_fact_proj(s1, None, wt, wp)
    torch.cuda.synchronize()
    _, _, Tq, Hq, Wq = s1.shape
    h32 = obf16.round_to_bf16(ohaar.haar3d_fwd(obf16.decode(xb[:, :, 125:129]), 3))
    g32 = _window64(hz, 32, 33, 0, Hq, 0, Wq)
    assert np.max(np.abs(g32 - h32)) <= 2.0 ** -7 * np.max(np.abs(h32)), "Haar frame 32"
    for f in (0, 32):
        o = oconv.spatial_conv(_window64(hz, f, f + 1, 0, Hq, 0, Wq), ws64)
        assert_rel(_window64(s1, f, f + 1, 0, Hq, 0, Wq), o, TOL, f"spatial frame {f}")
        f0 = max(0, f - 2)
        ot = oconv.temporal_conv(_window64(s1, f0, f + 1, 0, Hq, 0, Wq), wt64)[:, :, -1:]
        assert_rel(_window64(lat, f, f + 1, 0, Hq, 0, Wq), oconv.pointwise(obf16.round_to_bf16(ot), wp64), TOL,
                   f"temporal + 1x1 frame {f}")
    del x, hz, s1, lat
    torch.cuda.empty_cache()
