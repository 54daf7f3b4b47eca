"""The library's calls under HIP graph capture (torch.cuda.CUDAGraph on the caller's stream):
a pass of the hot path (Haar, the packed-weight convs with the fused 1x1, FSQ of that latent
and of a separate one, dequantize, inverse Haar) captured once and replayed three times,
with eager work and synchronisations between the replays, every replay's outputs equal to
the eager pass bit for bit; and the preallocated-scratch conv (the entry point meant for
callers under capture) captured and replayed on new input contents, equal to the
workspace call bit for bit.  The kernels allocate nothing and record no memset."""

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from tests.gpu_helpers import bits_to_torch, log, to_bits

pytestmark = pytest.mark.gpu

cvt = pytest.importorskip("causal_video_tokenizer_amd")


def _bf(shape, seed, std):
    return bits_to_torch(si.to_bf16_bits(si.normal(shape, seed, std)))


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # one eager pass on the capture stream first, as torch recommends
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return np.array_equal(to_bits(a), to_bits(b))
    return torch.equal(a, b)


def test_hot_path_pass_replays_equal_eager():
    B, T, H, W = 1, 17, 128, 192
    Tq, Hq, Wq = 1 + (T - 1) // 4, H // 4, W // 4
    log(f"graph capture of one pass over {B}x3x{T}x{H}x{W}")
    dev = torch.device("cuda:0")
    x = bits_to_torch(si.to_bf16_bits(si.video_sin((B, 3, T, H, W), 2900)))
    z_sep = bits_to_torch(si.to_bf16_bits(si.normal((B, 6, Tq, Hq, Wq), 2901, 1.5)), channels_last=True)
    pw_s = cvt.conv_weights_pack(_bf((256, 192, 1, 3, 3), 2902, 0.02))
    pw_t = cvt.conv_weights_pack(_bf((256, 256, 3, 1, 1), 2903, 0.02))
    pw_p = cvt.conv_weights_pack(_bf((6, 256, 1, 1, 1), 2904, 0.02))
    cl = torch.channels_last_3d
    hz = torch.empty((B, 192, Tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl)
    s1 = torch.empty((B, 256, Tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl)
    lat = torch.empty((B, 6, Tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl)
    idx = torch.empty((B, Tq, Hq, Wq), dtype=torch.int32, device=dev)
    idx2 = torch.empty_like(idx)
    codes = torch.empty((B, 6, Tq, Hq, Wq), dtype=torch.bfloat16, device=dev, memory_format=cl)
    xr = torch.empty_like(x)

    def step():
        cvt.haar3d_fwd(x, out=hz)
        cvt.causal_conv3d_fact_packed(hz, pw_s, None, out=s1)
        cvt.causal_conv3d_fact_proj_packed(s1, None, pw_t, pw_p, out=lat)
        cvt.fsq_quantize(lat, indices=idx)
        cvt.fsq_quantize(z_sep, indices=idx2)
        cvt.fsq_dequantize(idx2, out=codes)
        cvt.haar3d_inv(hz, out=xr)

    outs = (hz, s1, lat, idx, idx2, codes, xr)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    g = _capture(step)
    for rep in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = [_same(a, b) for a, b in zip(outs, ref)]
        log(f"  replay {rep}: {same}")
        assert all(same), f"replay {rep} differs from the eager pass: {same}"
        step()  # eager work between the replays
        torch.cuda.synchronize()


def test_noalloc_conv_under_capture_on_new_inputs():
    B, C, T, H, W = 1, 192, 5, 20, 40
    log("graph capture of the preallocated-scratch conv")
    dev = torch.device("cuda:0")
    x = bits_to_torch(si.to_bf16_bits(si.normal((B, C, T, H, W), 2910, 1.0)), channels_last=True)
    w_s = _bf((256, C, 1, 3, 3), 2911, 0.02)
    w_t = _bf((256, 256, 3, 1, 1), 2912, 0.02)
    y = torch.empty((B, 256, T, H, W), dtype=torch.bfloat16, device=dev, memory_format=torch.channels_last_3d)
    g = _capture(lambda: cvt.causal_conv3d_fact_noalloc(x, w_s, w_t, out=y))
    for k in range(2):
        x.copy_(bits_to_torch(si.to_bf16_bits(si.normal((B, C, T, H, W), 2920 + k, 1.0)), channels_last=True))
        torch.cuda.synchronize()
        g.replay()
        r = cvt.causal_conv3d_fact(x, w_s, w_t)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(y), to_bits(r)), f"replay {k} differs from the workspace call"
