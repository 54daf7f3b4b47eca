"""Streaming (chunk by chunk) encode on the GPU: a clip cut into a first chunk
(causal first frame) and continuation chunks, with the temporal convolution
reading the previous chunk's last two frames, gives bit for bit the result of
one call over the whole clip - for the Haar patcher and its inverse, for the
causal temporal convolution (with and without the fused 1x1 projection) and for
the whole 49-frame-style chain down to the FSQ indices.  The whole-clip results
are themselves checked against the oracle by the other GPU tests; the stream is
additionally checked against the oracle here on the final latent."""

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import bf16 as obf16
from oracle import conv as oconv
from tests.gpu_helpers import assert_rel, bits_to_torch, f32_to_torch, log, to_bits, to_f64

pytestmark = pytest.mark.gpu

cvt = pytest.importorskip("causal_video_tokenizer_amd")


def bf16_dev(shape, seed, std, cl=False):
    bits = si.to_bf16_bits(si.normal(shape, seed, std))
    return bits_to_torch(bits, channels_last=cl), obf16.decode(bits)


def test_haar_chunks_equal_whole_clip():
    x, _ = bf16_dev((2, 3, 37, 16, 24), 600, 0.5)
    whole = cvt.haar3d_fwd(x, 2)
    cuts = [(0, 13, 2), (13, 21, 3), (21, 37, 3)]  # pixel frames; latent frames 0-3, 4-5, 6-9
    parts = [cvt.haar3d_fwd(x[:, :, a:b].contiguous(), tl) for a, b, tl in cuts]
    torch.cuda.synchronize()
    assert np.array_equal(np.concatenate([to_bits(p) for p in parts], axis=2), to_bits(whole))
    back = [cvt.haar3d_inv(p, tl) for p, (_, _, tl) in zip(parts, cuts)]
    torch.cuda.synchronize()
    assert np.array_equal(np.concatenate([to_bits(b) for b in back], axis=2), to_bits(cvt.haar3d_inv(whole, 2)))


STREAM_CASES = [
    # B, C, T, H, W, Cp, bias, chunk lengths
    (1, 256, 10, 9, 14, 0, False, (4, 2, 4)),
    (1, 256, 10, 9, 14, 6, True, (3, 1, 6)),     # a one-frame chunk; projection to 6
    (2, 128, 9, 7, 11, 0, True, (5, 4)),         # two clips: history as its own tensor
    (1, 192, 8, 6, 10, 16, False, (2, 3, 3)),    # 192 channels, projection to 16
    (1, 64, 7, 5, 9, 0, False, (2, 5)),          # 64 channels
    (1, 128, 6, 4, 8, 0, True, (1, 1, 4)),       # one-frame chunks: history padded with a zero frame
]


@pytest.mark.parametrize("case", STREAM_CASES)
def test_temporal_stream_equals_whole_clip(case):
    B, C, T, H, W, Cp, bias, chunks = case
    log(f"temporal stream {case}")
    s, _ = bf16_dev((B, C, T, H, W), 610 + C, 1.0, cl=True)
    w_t, _ = bf16_dev((C, C, 3, 1, 1), 611, 0.02)
    b_t = f32_to_torch(si.normal((C,), 612, 0.1)) if bias else None
    w_p = bf16_dev((Cp, C, 1, 1, 1), 613, 0.02)[0] if Cp else None
    b_p = f32_to_torch(si.normal((Cp,), 614, 0.1)) if (bias and Cp) else None
    if Cp:
        whole = cvt.causal_conv3d_fact_proj(s, None, w_t, w_p, b_t=b_t, b_p=b_p)
    else:
        whole = cvt.causal_conv3d_fact(s, None, w_t, b_t=b_t)
    outs, t0 = [], 0
    for n in chunks:
        x = s[:, :, t0:t0 + n]
        if B > 1:
            x = x.contiguous(memory_format=torch.channels_last_3d)
        hist = None
        if t0 >= 2:
            hist = s[:, :, t0 - 2:t0]
            if B > 1:
                hist = hist.contiguous(memory_format=torch.channels_last_3d)
        elif t0 == 1:  # a stream that has seen one frame: the causal zero frame comes first
            hist = torch.cat([torch.zeros_like(s[:, :, :1]), s[:, :, :1]], dim=2)
            hist = hist.contiguous(memory_format=torch.channels_last_3d)
        outs.append(cvt.causal_conv3d_temporal_stream(x, w_t, hist=hist, w_p=w_p, b_t=b_t, b_p=b_p))
        t0 += n
    torch.cuda.synchronize()
    assert np.array_equal(np.concatenate([to_bits(o) for o in outs], axis=2), to_bits(whole))


def test_streamed_encode_chain_equals_whole_clip_and_oracle():
    """Haar -> spatial conv 192->256 -> causal temporal conv 256->256 with the 1x1 ->6 ->
    FSQ, once over a 37-frame clip and once in three chunks that carry two frames of the
    spatial conv's output; the FSQ indices and the latent are identical, and the streamed
    latent matches the oracle's whole-clip chain."""
    x, x64 = bf16_dev((1, 3, 37, 32, 64), 620, 0.5)
    w_s, ws64 = bf16_dev((256, 192, 1, 3, 3), 621, 0.02)
    w_t, wt64 = bf16_dev((256, 256, 3, 1, 1), 622, 0.02)
    w_p, wp64 = bf16_dev((6, 256, 1, 1, 1), 623, 0.02)
    hz = cvt.haar3d_fwd(x, 2)
    s_whole = cvt.causal_conv3d_fact(hz, w_s, None)
    lat_whole = cvt.causal_conv3d_fact_proj(s_whole, None, w_t, w_p)
    idx_whole = cvt.fsq_quantize(lat_whole)

    cuts = [(0, 13, 2), (13, 21, 3), (21, 37, 3)]
    prev_s, lats, idxs = None, [], []
    for a, b, tl in cuts:
        hzc = cvt.haar3d_fwd(x[:, :, a:b].contiguous(), tl)
        sc = cvt.causal_conv3d_fact(hzc, w_s, None)
        hist = None if prev_s is None else prev_s[:, :, -2:]
        lat = cvt.causal_conv3d_temporal_stream(sc, w_t, hist=hist, w_p=w_p)
        lats.append(lat)
        idxs.append(cvt.fsq_quantize(lat))
        prev_s = sc
    torch.cuda.synchronize()
    lat_stream = np.concatenate([to_bits(l) for l in lats], axis=2)
    assert np.array_equal(lat_stream, to_bits(lat_whole))
    assert np.array_equal(np.concatenate([i.cpu().numpy() for i in idxs], axis=1), idx_whole.cpu().numpy())
    # the oracle's whole-clip chain on the GPU's bf16 intermediate (stage-wise, as in the
    # other chain tests): temporal conv + 1x1 of the spatial output
    s64 = to_f64(s_whole)
    ref = oconv.pointwise(oconv.temporal_conv(s64, wt64), wp64[:, :, 0, 0, 0])
    assert_rel(obf16.decode(lat_stream), ref, 2e-2, "streamed latent vs oracle")
