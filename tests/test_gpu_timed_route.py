"""The route bench.py times, at the full sizes it times it on, against the float64 oracle.

The 49-frame DV8x16x16-720p-shaped step runs Haar, the spatial conv on its own
(causal_conv3d_fact_packed with pw_t = None, on weights packed once as the benchmark
packs them) and then the causal temporal conv with the 1x1 -> 6 projection in its
epilogue (causal_conv3d_fact_proj_packed with pw_s = None) and FSQ; the 121-frame
CV8x8x8-720p-shaped chain runs Haar, spatial, temporal, spatial, and the temporal conv
with the 1x1 -> 16 fused, all on packed weights.  The calls that repack per call use the
same kernels and are bit-identical (tests/test_gpu_packed.py).  Each call is checked stage by stage on whole
latent frames (every column and channel tile of the frame), each stage's oracle taking
the GPU's actual input to that stage (its bf16 bits): the spatial conv on the frame,
the temporal conv on the frame and its two predecessors, its output rounded to bf16 (the
value the epilogue stages) and then the 1x1.  Criterion |g - o| <= 2e-2 (|o| + rms(o)).
FSQ indices of the GPU latent must equal the oracle's on the same bits away from
rounding boundaries, and the oracle's on the oracle latent wherever the tolerance
cannot move the bound across one.
"""

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import bf16 as obf16
from oracle import conv as oconv
from oracle import fsq as ofsq
from oracle import haar as ohaar
from tests.gpu_helpers import assert_rel, bits_to_torch, log, to_bits

pytestmark = pytest.mark.gpu

cvt = pytest.importorskip("causal_video_tokenizer_amd")
TOL = 2e-2


def _w(shape, seed):
    bits = si.to_bf16_bits(si.normal(shape, seed, 0.02))
    return bits_to_torch(bits), obf16.decode(bits)


def _frames64(t, f0, f1):
    """bf16 NTHWC device tensor, latent frames f0..f1-1 -> float64 [B, C, n, H, W] (exact)."""
    return obf16.decode(to_bits(t[:, :, f0:f1]))


def _check_spatial(hin, hout, w64, frames, what):
    for f in frames:
        o = oconv.spatial_conv(_frames64(hin, f, f + 1), w64)
        assert_rel(_frames64(hout, f, f + 1), o, TOL, f"{what} frame {f}")


def _check_temporal(sin, out, wt64, frames, what, wp64=None):
    """out frame f from sin frames f-2..f (zeros before frame 0); with wp64 the temporal
    output is rounded to bf16 and projected."""
    outs = {}
    for f in frames:
        f0 = max(0, f - 2)
        o = oconv.temporal_conv(_frames64(sin, f0, f + 1), wt64)[:, :, -1:]
        if wp64 is not None:
            o = oconv.pointwise(obf16.round_to_bf16(o), wp64)
        assert_rel(_frames64(out, f, f + 1), o, TOL, f"{what} frame {f}")
        outs[f] = o
    return outs


def test_dv8x16x16_720p_timed_route_full_frames():
    """1 x 3 x 49 x 720 x 1280 through the step's calls; latent frames 0, 3, 4, 7, 12 in full
    (13 frames split 4 + 3 + 3 + 3 over the temporal row tiles: first and last frames of
    tiles, and the causal start)."""
    cid = 4
    wl = si.WORKLOADS["c4_dv8x16x16_720p_49f"]
    log("generating the 49-frame 720p clip")
    xb = si.to_bf16_bits(si.video_trans(wl["x"], wl["seed"]))
    x = bits_to_torch(xb)
    w_s, ws64 = _w((256, 192, 1, 3, 3), si.weight_seed(cid, 0))
    w_t, wt64 = _w((256, 256, 3, 1, 1), si.weight_seed(cid, 1))
    w_p, wp64 = _w((6, 256, 1, 1, 1), si.weight_seed(cid, 2))
    pw_s, pw_t, pw_p = cvt.conv_weights_pack(w_s), cvt.conv_weights_pack(w_t), cvt.conv_weights_pack(w_p)
    hz = cvt.haar3d_fwd(x)
    s1 = cvt.causal_conv3d_fact_packed(hz, pw_s, None)
    lat = cvt.causal_conv3d_fact_proj_packed(s1, None, pw_t, pw_p)
    idx = cvt.fsq_quantize(lat)
    torch.cuda.synchronize()
    assert tuple(lat.shape) == (1, 6, 13, 180, 320)
    # the coefficients the convs consumed are the oracle's (bf16 within 1 ulp, tested
    # elsewhere); here a frame of them against the oracle's Haar of the same pixels
    h64 = obf16.round_to_bf16(ohaar.haar3d_fwd(obf16.decode(xb[:, :, 45:49]), 3))
    g64 = _frames64(hz, 12, 13)
    assert np.max(np.abs(g64 - h64)) <= 2.0 ** -7 * np.max(np.abs(h64)), "Haar frame 12"
    frames = (0, 3, 4, 7, 12)
    _check_spatial(hz, s1, ws64, frames, "spatial 192->256")
    o_lat = _check_temporal(s1, lat, wt64, frames, "temporal 256->256 + 1x1 ->6", wp64)
    for f in frames:
        gl = _frames64(lat, f, f + 1)
        gi = idx[:, f:f + 1].cpu().numpy()
        oi, _, dist = ofsq.quantize(gl, ofsq.DEFAULT_LEVELS)        # FSQ on the GPU latent's bits
        assert np.all((gi == oi) | (dist < 1e-6)), f"FSQ on the GPU latent, frame {f}"
        ol = o_lat[f]
        oi2, _, _ = ofsq.quantize(ol, ofsq.DEFAULT_LEVELS)           # FSQ on the oracle latent
        rms = np.sqrt(np.mean(ol ** 2))
        margin = np.max(3.51 * TOL * (np.abs(ol) + rms), axis=1)   # |db/dz| <= h <= 3.51
        bvals = np.stack([ofsq.bound(ol[:, i], L) for i, L in enumerate(ofsq.DEFAULT_LEVELS)], axis=1)
        safe = np.min(np.abs(bvals - (np.floor(bvals) + 0.5)), axis=1) > margin
        log(f"  FSQ frame {f}: safe {int(safe.sum())}/{safe.size}, mismatches on safe "
            f"{int(np.sum((gi != oi2) & safe))}, elsewhere {int(np.sum((gi != oi2) & ~safe))}")
        assert np.all(gi[safe] == oi2[safe])
        assert safe.sum() > 0.5 * safe.size
    del x, hz, s1, lat, idx
    torch.cuda.empty_cache()


def test_cv8x8x8_720p_timed_route_full_frames():
    """1 x 3 x 121 x 720 x 1280 through the chain's calls (spatial and temporal layers as
    separate calls, the last temporal conv with the 1x1 -> 16 fused); latent frames 0, 1,
    27, 28, 30 in full (31 frames split 4 x 7 + 3 over the row tiles)."""
    cid = 3
    wl = si.WORKLOADS["c3_cv8x8x8_720p_121f"]
    log("generating the 121-frame 720p clip")
    xb = si.to_bf16_bits(si.video_trans(wl["x"], wl["seed"]))
    x = bits_to_torch(xb)
    del xb
    (w1s, w1s64), (w1t, w1t64), (w2s, w2s64), (w2t, w2t64) = [
        _w(shape, si.weight_seed(cid, i)) for i, shape in enumerate([(256, 192, 1, 3, 3), (256, 256, 3, 1, 1),
                                                                     (256, 256, 1, 3, 3), (256, 256, 3, 1, 1)])]
    w_p, wp64 = _w((16, 256, 1, 1, 1), si.weight_seed(cid, 4))
    p1s, p1t, p2s, p2t, pp = (cvt.conv_weights_pack(w) for w in (w1s, w1t, w2s, w2t, w_p))
    hz = cvt.haar3d_fwd(x)
    del x
    a1 = cvt.causal_conv3d_fact_packed(hz, p1s, None)
    b1 = cvt.causal_conv3d_fact_packed(a1, None, p1t)
    a2 = cvt.causal_conv3d_fact_packed(b1, p2s, None)
    lat = cvt.causal_conv3d_fact_proj_packed(a2, None, p2t, pp)
    torch.cuda.synchronize()
    assert tuple(lat.shape) == (1, 16, 31, 180, 320)
    frames = (0, 1, 27, 28, 30)
    _check_spatial(hz, a1, w1s64, (0, 28), "layer 1 spatial 192->256")
    _check_temporal(a1, b1, w1t64, frames, "layer 1 temporal 256->256")
    _check_spatial(b1, a2, w2s64, (1, 30), "layer 2 spatial 256->256")
    _check_temporal(a2, lat, w2t64, frames, "layer 2 temporal 256->256 + 1x1 ->16", wp64)
    del hz, a1, b1, a2, lat
    torch.cuda.empty_cache()
