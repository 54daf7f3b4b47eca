"""GPU parity of cvt_causal_conv3d_fact (bf16 MFMA implicit GEMM, fp32
accumulation) against the float64 oracle: |g - o| <= 2e-2 (|o| + rms(o))."""

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import bf16 as obf16
from oracle import conv as oconv
from oracle import fsq as ofsq
from oracle import haar as ohaar
from tests.gpu_helpers import assert_rel, bits_to_torch, f32_to_torch, log, to_bits, to_f64

pytestmark = pytest.mark.gpu

cvt = pytest.importorskip("causal_video_tokenizer_amd")
TOL = 2e-2


def bf16_input(shape, seed, std):
    bits = si.to_bf16_bits(si.normal(shape, seed, std))
    return bits, obf16.decode(bits)


def make_case(B, Cin, Cout, T, H, W, k, temporal, bias, seed):
    xb, x64 = bf16_input((B, Cin, T, H, W), seed, 1.0)
    wsb, ws64 = bf16_input((Cout, Cin, 1, k, k), seed + 1, 0.02)
    wtb, wt64 = bf16_input((Cout, Cout, k, 1, 1), seed + 2, 0.02) if temporal else (None, None)
    bs = si.normal((Cout,), seed + 3, 0.1) if bias else None
    bt = si.normal((Cout,), seed + 4, 0.1) if (bias and temporal) else None
    dev = dict(x=bits_to_torch(xb, channels_last=True), w_s=bits_to_torch(wsb),
               w_t=bits_to_torch(wtb) if temporal else None,
               b_s=f32_to_torch(bs) if bias else None, b_t=f32_to_torch(bt) if bt is not None else None)
    ref = dict(x=x64, ws=ws64, wt=wt64, bs=bs, bt=bt)
    return dev, ref


CASES = [
    # B, Cin, Cout, T, H, W, k, temporal, bias
    (1, 48, 64, 1, 16, 16, 3, True, False),      # single image grid (T = 1: last temporal tap only)
    (2, 64, 256, 5, 12, 20, 3, True, False),     # 2400 positions: 19 position tiles, ragged tail
    (1, 256, 256, 3, 9, 13, 3, True, True),      # 256 -> 256 with biases
    (1, 192, 192, 4, 10, 10, 3, True, False),    # 192 output channels (3-wave 192-channel tiles)
    (1, 40, 160, 3, 7, 9, 3, True, True),        # Cin tail on the 3-wave tiles, Cout 160 of 192
    (2, 192, 176, 5, 6, 37, 3, True, False),     # Cout 176 of 192, ragged column and frame tiles, 2 clips
    (1, 136, 40, 3, 7, 9, 3, True, False),       # Cin tail inside a 64-channel step, Cout tail
    (1, 8, 8, 3, 5, 5, 3, True, False),
    (1, 256, 16, 3, 8, 8, 1, False, False),      # 1x1 projection to the 16-dim latent
    (1, 256, 6, 3, 8, 8, 1, False, True),        # 1x1 to 6 channels (unaligned stores)
    (1, 64, 6, 1, 16, 16, 1, False, False),
    (1, 6, 192, 3, 8, 8, 1, False, True),        # 6 -> 192 lift after dequantization (small-Cin path)
    (1, 16, 24, 2, 4, 4, 1, True, False),        # k = 1 with a temporal 1x1x1 part
    (2, 128, 128, 7, 6, 11, 3, True, True),      # frame tiles of 4 and 3 output frames, 2 clips
    (1, 64, 96, 6, 9, 9, 3, True, False),        # frame tiles of 4 and 2, Cout tail in a 128 tile
    (1, 96, 256, 2, 5, 70, 3, True, True),       # 2 frames only: every region frame but the last two is padding
]


@pytest.mark.parametrize("case", CASES)
def test_conv_parity(case):
    B, Cin, Cout, T, H, W, k, temporal, bias = case
    log(f"conv case {case}")
    dev, ref = make_case(*case, seed=100 + Cin + Cout)
    y = cvt.causal_conv3d_fact(**dev)
    torch.cuda.synchronize()
    assert y.is_contiguous(memory_format=torch.channels_last_3d)
    o = oconv.causal_conv3d_fact(ref["x"], ref["ws"], ref["wt"], ref["bs"], ref["bt"])
    assert_rel(to_f64(y), o, TOL, "conv")


def test_conv_short_video_full():
    """Short video grid 1 x 192 x 5 x 64 x 64 -> 256 (k = 3) -> 1x1 -> 16, full compare."""
    wl = si.WORKLOADS["c2_video_17x256"]
    xb = si.to_bf16_bits(si.video_sin(wl["x"], wl["seed"]))
    x = bits_to_torch(xb)
    hz = cvt.haar3d_fwd(x)
    w1s, w1s64 = bf16_input((256, 192, 1, 3, 3), si.weight_seed(2, 0), 0.02)
    w1t, w1t64 = bf16_input((256, 256, 3, 1, 1), si.weight_seed(2, 1), 0.02)
    w2, w264 = bf16_input((16, 256, 1, 1, 1), si.weight_seed(2, 2), 0.02)
    y1 = cvt.causal_conv3d_fact(hz, bits_to_torch(w1s), bits_to_torch(w1t))
    y2 = cvt.causal_conv3d_fact(y1, bits_to_torch(w2))
    torch.cuda.synchronize()
    h64 = obf16.round_to_bf16(ohaar.haar3d_fwd(obf16.decode(xb), 2))
    o1 = oconv.causal_conv3d_fact(h64, w1s64, w1t64)
    assert_rel(to_f64(y1), o1, TOL, "layer 1")
    o2 = oconv.pointwise(obf16.round_to_bf16(o1), w264)
    assert_rel(to_f64(y2), o2, TOL, "1x1 to 16")


def test_conv_causality_and_determinism():
    dev, _ = make_case(1, 64, 64, 6, 8, 8, 3, True, False, seed=7)
    y0 = to_bits(cvt.causal_conv3d_fact(**dev))
    y1 = to_bits(cvt.causal_conv3d_fact(**dev))
    assert np.array_equal(y0, y1)
    for t0 in (0, 2, 5):
        d = dict(dev)
        d["x"] = dev["x"].clone()
        d["x"][:, :, t0] = 1.0
        yp = to_bits(cvt.causal_conv3d_fact(**d))
        assert np.array_equal(y0[:, :, :t0], yp[:, :, :t0]), t0
        assert not np.array_equal(y0[:, :, t0], yp[:, :, t0]), t0


def test_conv_invalid_raises():
    dev, _ = make_case(1, 64, 64, 2, 4, 4, 3, True, False, seed=9)
    with pytest.raises(cvt.CvtError):
        cvt.causal_conv3d_fact(dev["x"], dev["w_s"], dev["w_t"], workspace=torch.empty(16, dtype=torch.uint8,
                                                                                       device="cuda"))


# ---------------------------------------------------------------- full-size chains, sampled

def _oracle_chain_crop(xbits, tq1, rows, cols, layers, proj, halo, lookback):
    """Oracle for latent frame tq1 on the spatial window rows x cols of the
    post-Haar grid: Haar on a pixel crop with enough causal and spatial context,
    then the conv layers (bf16 storage between stages), then the 1x1."""
    B, C, T, H, W = xbits.shape
    Hq, Wq = H // 4, W // 4
    tq0 = max(0, tq1 - lookback)
    r0, r1 = max(0, rows[0] - halo), min(Hq, rows[1] + halo)
    c0, c1 = max(0, cols[0] - halo), min(Wq, cols[1] + halo)
    if tq0 == 0:
        px = xbits[:, :, 0:4 * tq1 + 1]
        drop = 0
    else:
        px = xbits[:, :, 4 * tq0 - 4:4 * tq1 + 1]
        drop = 1
    px = px[:, :, :, 4 * r0:4 * r1, 4 * c0:4 * c1]
    h = obf16.round_to_bf16(ohaar.haar3d_fwd(obf16.decode(px), 2)[:, :, drop:])
    outs = []
    for ws, wt in layers:
        h = oconv.causal_conv3d_fact(h, ws, wt)
        outs.append(h)
        h = obf16.round_to_bf16(h)
    p = oconv.pointwise(h, proj)
    sl = (slice(None), slice(None), slice(tq1 - tq0, tq1 - tq0 + 1),
          slice(rows[0] - r0, rows[1] - r0), slice(cols[0] - c0, cols[1] - c0))
    return [o[sl] for o in outs], p[sl]


def _gpu_window(t, tq1, rows, cols):
    return to_f64(t[:, :, tq1:tq1 + 1, rows[0]:rows[1], cols[0]:cols[1]])


def test_cv8x8x8_720p_chain_sampled():
    """1 x 3 x 121 x 720 x 1280: Haar -> conv 192->256 -> conv 256->256 -> 1x1 -> 16, sampled."""
    cid = 3
    wl = si.WORKLOADS["c3_cv8x8x8_720p_121f"]
    log("generating the 121-frame 720p video")
    xb = si.to_bf16_bits(si.video_trans(wl["x"], wl["seed"]))
    x = bits_to_torch(xb)
    ws = [bf16_input((256, 192, 1, 3, 3), si.weight_seed(cid, 0), 0.02),
          bf16_input((256, 256, 3, 1, 1), si.weight_seed(cid, 1), 0.02),
          bf16_input((256, 256, 1, 3, 3), si.weight_seed(cid, 2), 0.02),
          bf16_input((256, 256, 3, 1, 1), si.weight_seed(cid, 3), 0.02)]
    pj = bf16_input((16, 256, 1, 1, 1), si.weight_seed(cid, 4), 0.02)
    hz = cvt.haar3d_fwd(x)
    del x
    y1 = cvt.causal_conv3d_fact(hz, bits_to_torch(ws[0][0]), bits_to_torch(ws[1][0]))
    del hz
    y2 = cvt.causal_conv3d_fact(y1, bits_to_torch(ws[2][0]), bits_to_torch(ws[3][0]))
    y3 = cvt.causal_conv3d_fact(y2, bits_to_torch(pj[0]))
    torch.cuda.synchronize()
    layers = [(ws[0][1], ws[1][1]), (ws[2][1], ws[3][1])]
    for tq1, rows, cols in [(0, (0, 4), (0, 8)), (1, (100, 104), (200, 206)), (30, (176, 180), (312, 320)),
                            (17, (60, 63), (0, 5))]:
        log(f"  window t'={tq1} rows={rows} cols={cols}")
        (o1, o2), o3 = _oracle_chain_crop(xb, tq1, rows, cols, layers, pj[1], halo=2, lookback=4)
        assert_rel(_gpu_window(y1, tq1, rows, cols), o1, TOL, "layer 1")
        assert_rel(_gpu_window(y2, tq1, rows, cols), o2, TOL, "layer 2")
        assert_rel(_gpu_window(y3, tq1, rows, cols), o3, TOL, "1x1 to 16")
    del y1, y2, y3
    torch.cuda.empty_cache()


def test_dv8x16x16_720p_chain_sampled():
    """1 x 3 x 49 x 720 x 1280: Haar -> conv 192->256 -> 1x1 -> 6 -> FSQ, sampled;
    FSQ indices must equal the oracle's wherever the oracle latent is farther
    from a rounding boundary than the convolution tolerance can move it."""
    cid = 4
    wl = si.WORKLOADS["c4_dv8x16x16_720p_49f"]
    xb = si.to_bf16_bits(si.video_trans(wl["x"], wl["seed"]))
    x = bits_to_torch(xb)
    w1s = bf16_input((256, 192, 1, 3, 3), si.weight_seed(cid, 0), 0.02)
    w1t = bf16_input((256, 256, 3, 1, 1), si.weight_seed(cid, 1), 0.02)
    pj = bf16_input((6, 256, 1, 1, 1), si.weight_seed(cid, 2), 0.02)
    hz = cvt.haar3d_fwd(x)
    y1 = cvt.causal_conv3d_fact(hz, bits_to_torch(w1s[0]), bits_to_torch(w1t[0]))
    lat = cvt.causal_conv3d_fact(y1, bits_to_torch(pj[0]))
    idx = cvt.fsq_quantize(lat)
    torch.cuda.synchronize()
    for tq1, rows, cols in [(0, (0, 6), (0, 10)), (12, (170, 180), (300, 320)), (6, (90, 95), (150, 160))]:
        (o1,), o2 = _oracle_chain_crop(xb, tq1, rows, cols, [(w1s[1], w1t[1])], pj[1], halo=1, lookback=2)
        assert_rel(_gpu_window(y1, tq1, rows, cols), o1, TOL, "layer 1")
        assert_rel(_gpu_window(lat, tq1, rows, cols), o2, TOL, "1x1 to 6")
        oi, _, _ = ofsq.quantize(o2, ofsq.DEFAULT_LEVELS)
        gi = idx[:, tq1:tq1 + 1, rows[0]:rows[1], cols[0]:cols[1]].cpu().numpy()
        # distance (in bound units) the tolerance allows: |dz| <= TOL (|z| + rms), |db/dz| <= h <= 3.51
        rms = np.sqrt(np.mean(o2 ** 2))
        margin = np.max(3.51 * TOL * (np.abs(o2) + rms), axis=1)
        bvals = np.stack([ofsq.bound(o2[:, i], L) for i, L in enumerate(ofsq.DEFAULT_LEVELS)], axis=1)
        dist = np.min(np.abs(bvals - (np.floor(bvals) + 0.5)), axis=1)
        safe = dist > margin
        log(f"  FSQ window t'={tq1}: safe positions {int(safe.sum())}/{safe.size}, "
            f"mismatches on safe {int(np.sum((gi != oi) & safe))}, elsewhere {int(np.sum((gi != oi) & ~safe))}")
        assert np.all(gi[safe] == oi[safe])
        assert safe.sum() > 0.5 * safe.size


PROJ_CASES = [
    # B, Cin, Cout, Cp, T, H, W, spatial, bias
    (1, 192, 256, 6, 5, 12, 20, True, True),    # the 49-frame chain's shape family: conv -> 1x1 to the FSQ latent
    (1, 256, 256, 16, 7, 9, 13, False, True),   # temporal-only, 16-dim continuous latent, frame tiles of 4 and 3
    (2, 96, 192, 6, 6, 5, 70, True, False),     # Cout 192 on the 3-wave 192-channel tiles, ragged columns, 2 clips
    (1, 64, 144, 16, 5, 7, 9, True, True),      # Cout 144 of 192 (staged zeros past Cout), Cp 16
    (1, 64, 64, 3, 2, 8, 8, True, True),        # narrow channels, 2 frames
    (1, 64, 128, 24, 3, 6, 6, True, True),      # Cp > 16: conv then a separate 1x1 pass
]


@pytest.mark.parametrize("case", PROJ_CASES)
def test_conv_proj_parity(case):
    """Fused conv + 1x1 against the oracle: conv in float64, rounded to bf16 (the stored
    intermediate of the unfused chain), then the 1x1 projection; |g - o| <= 2e-2 (|o| + rms)."""
    B, Cin, Cout, Cp, T, H, W, spatial, bias = case
    log(f"conv+proj case {case}")
    seed = 300 + Cin + Cout + Cp
    dev, ref = make_case(B, Cin, Cout, T, H, W, 3, True, bias, seed)
    if not spatial:
        xb, x64 = bf16_input((B, Cout, T, H, W), seed + 9, 1.0)
        dev["x"], ref["x"] = bits_to_torch(xb, channels_last=True), x64
        dev["w_s"], dev["b_s"], ref["ws"], ref["bs"] = None, None, None, None
    wpb, wp64 = bf16_input((Cp, Cout, 1, 1, 1), seed + 5, 0.05)
    bp = si.normal((Cp,), seed + 6, 0.1) if bias else None
    y = cvt.causal_conv3d_fact_proj(dev["x"], dev["w_s"], dev["w_t"], bits_to_torch(wpb), b_s=dev["b_s"],
                                    b_t=dev["b_t"], b_p=f32_to_torch(bp) if bias else None)
    torch.cuda.synchronize()
    assert y.shape == (B, Cp, T, H, W) and y.is_contiguous(memory_format=torch.channels_last_3d)
    if spatial:
        o1 = oconv.causal_conv3d_fact(ref["x"], ref["ws"], ref["wt"], ref["bs"], ref["bt"])
    else:
        o1 = oconv.temporal_conv(ref["x"], ref["wt"], ref["bt"])
    o = oconv.pointwise(obf16.round_to_bf16(o1), wp64, bp)
    assert_rel(to_f64(y), o, TOL, "conv+proj")
    # the unfused GPU chain on the same inputs agrees to a bf16 ulp or so
    y1 = cvt.causal_conv3d_fact(dev["x"], dev["w_s"], dev["w_t"], dev["b_s"], dev["b_t"]) if spatial else \
        cvt.causal_conv3d_fact(dev["x"], None, dev["w_t"], None, dev["b_t"])
    y2 = cvt.causal_conv3d_fact(y1, bits_to_torch(wpb), None, f32_to_torch(bp) if bias else None)
    torch.cuda.synchronize()
    assert_rel(to_f64(y), to_f64(y2), 1e-2, "fused vs unfused")


def test_dv4x8x8_360p_decode_chain_sampled():
    """8 clips, int32 indices 8 x 13 x 90 x 160 -> dequantize -> 1x1 6->192 -> conv
    192->192 (k = 3) -> inverse Haar to 8 x 3 x 49 x 360 x 640, sampled.  The oracle runs
    the chain on a latent window with 3 frames of causal context and a 1-pixel halo, and
    inverts the window's coefficients; the conv output and the pixels of the window are
    compared (the pixels inherit the conv tolerance)."""
    cid = 5
    wl = si.WORKLOADS["c5_dv4x8x8_360p_decode"]
    idx = si.uniform_indices(wl["indices"], wl["seed"])
    lift, lift64 = bf16_input((192, 6, 1, 1, 1), si.weight_seed(cid, 0), 0.02)
    wsb, ws64 = bf16_input((192, 192, 1, 3, 3), si.weight_seed(cid, 1), 0.02)
    wtb, wt64 = bf16_input((192, 192, 3, 1, 1), si.weight_seed(cid, 2), 0.02)
    codes = cvt.fsq_dequantize(torch.from_numpy(idx).cuda(), dtype=torch.bfloat16, layout="NTHWC")
    z = cvt.causal_conv3d_fact(codes, bits_to_torch(lift))
    y = cvt.causal_conv3d_fact(z, bits_to_torch(wsb), bits_to_torch(wtb))
    del codes, z
    x = cvt.haar3d_inv(y)
    torch.cuda.synchronize()
    assert tuple(x.shape) == wl["out_x"]
    _, Tq, Hq, Wq = idx.shape
    for b, tq1, rows, cols in [(0, 0, (0, 3), (0, 4)), (3, 5, (40, 43), (100, 104)), (7, 12, (87, 90), (156, 160)),
                               (5, 1, (10, 12), (0, 3))]:
        log(f"  clip {b} window t'={tq1} rows={rows} cols={cols}")
        tq0 = max(0, tq1 - 3)
        r0, r1 = max(0, rows[0] - 1), min(Hq, rows[1] + 1)
        c0, c1 = max(0, cols[0] - 1), min(Wq, cols[1] + 1)
        oc, _ = ofsq.dequantize(idx[b:b + 1, tq0:tq1 + 1, r0:r1, c0:c1], ofsq.DEFAULT_LEVELS)
        oz = obf16.round_to_bf16(oconv.pointwise(oc, lift64))
        oy = oconv.causal_conv3d_fact(oz, ws64, wt64)
        f0 = max(0, tq1 - 1)  # the inverse of latent frames f0..tq1 ends with latent frame tq1's pixels
        sl = (slice(None), slice(None), slice(f0 - tq0, tq1 - tq0 + 1),
              slice(rows[0] - r0, rows[1] - r0), slice(cols[0] - c0, cols[1] - c0))
        assert_rel(to_f64(y[b:b + 1, :, f0:tq1 + 1, rows[0]:rows[1], cols[0]:cols[1]]), oy[sl], TOL, "conv 192->192")
        ox = ohaar.haar3d_inv(obf16.round_to_bf16(oy[sl]), 2)
        npx = 1 if tq1 == 0 else 4  # pixel frames of latent frame tq1
        gx = to_f64(x[b:b + 1, :, max(0, 4 * tq1 - 3):4 * tq1 + 1, 4 * rows[0]:4 * rows[1], 4 * cols[0]:4 * cols[1]])
        assert_rel(gx, ox[:, :, -npx:], TOL, "pixels")
    del y, x
    torch.cuda.empty_cache()
