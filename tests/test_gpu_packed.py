"""Conv weights packed once (cvt_conv_weights_pack) and the packed-weight convs
(cvt_causal_conv3d_fact_packed, cvt_causal_conv3d_fact_proj_packed) against the calls that
repack the weights on every call: bit-identical outputs (same kernels, same weights), for
spatial only, temporal only and both parts, with and without biases, on the 4-wave
256-channel, 3-wave 192-channel and 128 x 64 tiles, ragged grids and two clips; the same
packed weights reused on a second input; one case also against the float64 oracle,
|g - o| <= 2e-2 (|o| + rms(o)).  The blocks on packed weights (cvt_resblock3d_packed,
cvt_downsample3d_packed, cvt_upsample3d_packed) against the blocks that repack: bit-identical."""

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import bf16 as obf16
from oracle import conv as oconv
from tests.gpu_helpers import assert_rel, bits_to_torch, f32_to_torch, log, to_bits, to_f64

pytestmark = pytest.mark.gpu

cvt = pytest.importorskip("causal_video_tokenizer_amd")

CASES = [
    # B, Cin, Cout, T, H, W, bias
    (1, 192, 256, 5, 12, 40, True),
    (2, 256, 256, 9, 7, 33, False),
    (1, 160, 192, 6, 9, 20, True),     # 3-wave 192-channel tiles
    (1, 64, 128, 4, 10, 70, False),    # 128-channel tiles of 64 columns
    (1, 96, 64, 1, 5, 9, True),
    (1, 40, 64, 3, 6, 10, True),       # input-channel tail (40 = 32 + 8): the chunk past Cin reads zeros
]


def _w(shape, seed, std=0.02):
    bits = si.to_bf16_bits(si.normal(shape, seed, std))
    return bits_to_torch(bits), obf16.decode(bits)


def _inputs(B, Cin, Cout, T, H, W, bias, seed):
    xb = si.to_bf16_bits(si.normal((B, Cin, T, H, W), seed, 1.0))
    w_s, ws64 = _w((Cout, Cin, 1, 3, 3), seed + 1)
    w_t, wt64 = _w((Cout, Cout, 3, 1, 1), seed + 2)
    bs = si.normal((Cout,), seed + 3, 0.1) if bias else None
    bt = si.normal((Cout,), seed + 4, 0.1) if bias else None
    dev = dict(x=bits_to_torch(xb, channels_last=True), w_s=w_s, w_t=w_t,
               b_s=f32_to_torch(bs) if bias else None, b_t=f32_to_torch(bt) if bias else None)
    ref = dict(x=obf16.decode(xb), ws=ws64, wt=wt64, bs=bs, bt=bt)
    return dev, ref


def _same(a, b, what):
    ga, gb = to_bits(a), to_bits(b)
    nd = int(np.count_nonzero(ga != gb))
    assert nd == 0, f"{what}: {nd} of {ga.size} outputs differ from the unpacked call"


@pytest.mark.parametrize("case", CASES)
def test_packed_conv_equals_unpacked(case):
    B, Cin, Cout, T, H, W, bias = case
    log(f"packed conv {case}")
    d, _ = _inputs(*case, seed=2400 + Cin + Cout + T)
    pw_s, pw_t = cvt.conv_weights_pack(d["w_s"]), cvt.conv_weights_pack(d["w_t"])
    for s_part, t_part in ((True, True), (True, False), (False, True)):
        x = d["x"] if s_part else bits_to_torch(si.to_bf16_bits(si.normal((B, Cout, T, H, W), 2500 + T, 1.0)),
                                                channels_last=True)
        y = cvt.causal_conv3d_fact_packed(x, pw_s if s_part else None, pw_t if t_part else None,
                                          d["b_s"] if s_part else None, d["b_t"] if t_part else None)
        r = cvt.causal_conv3d_fact(x, d["w_s"] if s_part else None, d["w_t"] if t_part else None,
                                   d["b_s"] if s_part else None, d["b_t"] if t_part else None)
        torch.cuda.synchronize()
        _same(y, r, f"parts spatial={s_part} temporal={t_part}")


@pytest.mark.parametrize("Cp", [6, 16])
def test_packed_conv_proj_equals_unpacked_and_oracle(Cp):
    B, Cin, Cout, T, H, W = 1, 192, 256, 6, 9, 35
    log(f"packed conv + 1x1 -> {Cp}")
    d, ref = _inputs(B, Cin, Cout, T, H, W, True, seed=2600 + Cp)
    w_p, wp64 = _w((Cp, Cout, 1, 1, 1), 2610 + Cp, 0.05)
    bp = si.normal((Cp,), 2620 + Cp, 0.1)
    b_p = f32_to_torch(bp)
    pw_s, pw_t, pw_p = (cvt.conv_weights_pack(w) for w in (d["w_s"], d["w_t"], w_p))
    y = cvt.causal_conv3d_fact_proj_packed(d["x"], pw_s, pw_t, pw_p, d["b_s"], d["b_t"], b_p)
    r = cvt.causal_conv3d_fact_proj(d["x"], d["w_s"], d["w_t"], w_p, d["b_s"], d["b_t"], b_p)
    s = cvt.causal_conv3d_fact_packed(d["x"], pw_s, None, d["b_s"])
    yt = cvt.causal_conv3d_fact_proj_packed(s, None, pw_t, pw_p, None, d["b_t"], b_p)
    rt = cvt.causal_conv3d_fact_proj(s, None, d["w_t"], w_p, None, d["b_t"], b_p)
    torch.cuda.synchronize()
    _same(y, r, "both parts + projection")
    _same(yt, rt, "temporal + projection")
    # the oracle on the same bits: conv in float64, rounded to bf16 where the kernels round
    # (the spatial output and the temporal output before the 1x1), then the projection
    h = obf16.round_to_bf16(oconv.spatial_conv(ref["x"], ref["ws"], ref["bs"]))
    c = obf16.round_to_bf16(oconv.temporal_conv(h, ref["wt"], ref["bt"]))
    o = oconv.pointwise(c, wp64, bp)
    assert_rel(to_f64(y), o, 2e-2, f"packed conv + 1x1 -> {Cp} vs oracle")


def test_packed_weights_reused_on_new_inputs():
    B, Cin, Cout, T, H, W = 1, 192, 256, 5, 8, 24
    log("packed weights on two inputs in a row")
    d, _ = _inputs(B, Cin, Cout, T, H, W, True, seed=2700)
    pw_s, pw_t = cvt.conv_weights_pack(d["w_s"]), cvt.conv_weights_pack(d["w_t"])
    ws = torch.empty(cvt.conv_packed_workspace_bytes(d["x"].shape, Cout), dtype=torch.uint8, device=d["x"].device)
    for k in range(2):
        x = bits_to_torch(si.to_bf16_bits(si.normal((B, Cin, T, H, W), 2710 + k, 1.0)), channels_last=True)
        y = cvt.causal_conv3d_fact_packed(x, pw_s, pw_t, d["b_s"], d["b_t"], workspace=ws)
        r = cvt.causal_conv3d_fact(x, d["w_s"], d["w_t"], d["b_s"], d["b_t"])
        torch.cuda.synchronize()
        _same(y, r, f"call {k}")


def test_packed_binding_rejects_mismatched_weights():
    d, _ = _inputs(1, 192, 256, 5, 8, 8, False, seed=2800)
    pw_s, pw_t = cvt.conv_weights_pack(d["w_s"]), cvt.conv_weights_pack(d["w_t"])
    with pytest.raises(ValueError):
        cvt.causal_conv3d_fact_packed(d["x"], pw_t, None)        # a temporal packing as the spatial weights
    with pytest.raises(ValueError):
        cvt.causal_conv3d_fact_packed(d["x"], d["w_s"], None)    # unpacked weights
    x2 = torch.empty((1, 128, 5, 8, 8), dtype=torch.bfloat16, device=d["x"].device,
                     memory_format=torch.channels_last_3d)
    with pytest.raises(ValueError):
        cvt.causal_conv3d_fact_packed(x2, pw_s, pw_t)            # packed for 192 input channels


RESBLOCK_CASES = [
    # B, C, T, H, W, bias, in place: 256 (4-wave tiles), 192 (192-channel tiles), 320 (plain conv +
    # LayerNorm kernel), 64 (128-channel tiles)
    (1, 256, 5, 9, 35, True, False),
    (2, 192, 4, 6, 20, False, True),
    (1, 320, 3, 5, 9, True, False),
    (1, 64, 6, 7, 12, False, False),
    (1, 136, 3, 6, 7, True, False),     # channels past Cout left out of the LayerNorm statistics
]


@pytest.mark.parametrize("case", RESBLOCK_CASES)
def test_packed_resblock_equals_unpacked(case):
    """cvt_resblock3d_packed on weights packed once equals cvt_resblock3d bit for bit (and in
    place, y = x)."""
    B, C, T, H, W, bias, inplace = case
    log(f"packed residual block {case}")
    seed = 2900 + C + T
    x = bits_to_torch(si.to_bf16_bits(si.normal((B, C, T, H, W), seed, 1.0)), channels_last=True)
    p = {"ln1_g": f32_to_torch(1.0 + si.normal((C,), seed + 1, 0.1)), "ln1_b": f32_to_torch(si.normal((C,), seed + 2, 0.1)),
         "ln2_g": f32_to_torch(1.0 + si.normal((C,), seed + 3, 0.1)), "ln2_b": f32_to_torch(si.normal((C,), seed + 4, 0.1)),
         "c1_s": _w((C, C, 1, 3, 3), seed + 5, 0.03)[0], "c1_t": _w((C, C, 3, 1, 1), seed + 6, 0.03)[0],
         "c2_s": _w((C, C, 1, 3, 3), seed + 7, 0.03)[0], "c2_t": _w((C, C, 3, 1, 1), seed + 8, 0.03)[0]}
    if bias:
        for j, k in enumerate(("c1_bs", "c1_bt", "c2_bs", "c2_bt")):
            p[k] = f32_to_torch(si.normal((C,), seed + 9 + j, 0.1))
    q = dict(p)
    for k in ("c1_s", "c1_t", "c2_s", "c2_t"):
        q[k] = cvt.conv_weights_pack(p[k])
    r = cvt.resblock3d(x, p)
    if inplace:
        y = x.clone()
        cvt.resblock3d_packed(y, q, out=y)
    else:
        y = cvt.resblock3d_packed(x, q)
    torch.cuda.synchronize()
    _same(y, r, f"residual block {case}")


def test_packed_resblock_binding_rejects_unpacked_weights():
    C = 64
    x = torch.empty((1, C, 3, 4, 4), dtype=torch.bfloat16, device="cuda", memory_format=torch.channels_last_3d)
    ones, zeros = torch.ones(C, device="cuda"), torch.zeros(C, device="cuda")
    ws, wt = _w((C, C, 1, 3, 3), 2990)[0], _w((C, C, 3, 1, 1), 2991)[0]
    p = {"ln1_g": ones, "ln1_b": zeros, "ln2_g": ones, "ln2_b": zeros, "c1_s": ws, "c1_t": wt, "c2_s": ws, "c2_t": wt}
    with pytest.raises(ValueError):
        cvt.resblock3d_packed(x, p)                                           # unpacked weights
    q = dict(p, c1_s=cvt.conv_weights_pack(wt), c1_t=cvt.conv_weights_pack(wt),
             c2_s=cvt.conv_weights_pack(ws), c2_t=cvt.conv_weights_pack(wt))
    with pytest.raises(ValueError):
        cvt.resblock3d_packed(x, q)                                           # temporal packing as spatial weights


DOWN_CASES = [
    # B, Cin, Cout, T, H, W, space, time, bias
    (1, 256, 256, 9, 12, 40, True, True, True),
    (2, 128, 128, 5, 8, 18, True, True, False),    # 128-channel tiles
    (1, 192, 192, 7, 10, 14, True, False, True),   # spatial part only
    (1, 256, 256, 9, 6, 10, False, True, True),    # temporal part only (Cin == Cout)
    (1, 128, 256, 5, 8, 12, True, True, True),     # channels widened by the spatial part
]


@pytest.mark.parametrize("case", DOWN_CASES)
def test_packed_downsample_equals_unpacked(case):
    B, Cin, Cout, T, H, W, space, time, bias = case
    log(f"packed downsampling block {case}")
    seed = 3000 + Cin + T + H
    x = bits_to_torch(si.to_bf16_bits(si.normal((B, Cin, T, H, W), seed, 1.0)), channels_last=True)
    w_s = _w((Cout, Cin, 1, 3, 3), seed + 1)[0] if space else None
    w_t = _w((Cout, Cout if space else Cin, 3, 1, 1), seed + 2)[0] if time else None
    b_s = f32_to_torch(si.normal((Cout,), seed + 3, 0.1)) if bias and space else None
    b_t = f32_to_torch(si.normal((Cout,), seed + 4, 0.1)) if bias and time else None
    pw_s = cvt.conv_weights_pack(w_s) if space else None
    pw_t = cvt.conv_weights_pack(w_t) if time else None
    y = cvt.downsample3d_packed(x, pw_s, pw_t, b_s, b_t)
    r = cvt.downsample3d(x, w_s, w_t, b_s, b_t)
    torch.cuda.synchronize()
    _same(y, r, f"downsampling {case}")


UP_CASES = [
    # B, Cin, Cout, T, H, W, space, time, bias
    (1, 256, 256, 4, 6, 20, True, True, True),
    (1, 128, 192, 3, 5, 9, True, False, False),    # 192-channel tiles, spatial repetition only
    (2, 64, 64, 3, 4, 6, False, True, True),       # temporal repetition only
]


@pytest.mark.parametrize("case", UP_CASES)
def test_packed_upsample_equals_unpacked(case):
    B, Cin, Cout, T, H, W, space, time, bias = case
    log(f"packed upsampling block {case}")
    seed = 3100 + Cin + Cout + T
    x = bits_to_torch(si.to_bf16_bits(si.normal((B, Cin, T, H, W), seed, 1.0)), channels_last=True)
    w_s, w_t = _w((Cout, Cin, 1, 3, 3), seed + 1)[0], _w((Cout, Cout, 3, 1, 1), seed + 2)[0]
    b_s = f32_to_torch(si.normal((Cout,), seed + 3, 0.1)) if bias else None
    b_t = f32_to_torch(si.normal((Cout,), seed + 4, 0.1)) if bias else None
    pw_s, pw_t = cvt.conv_weights_pack(w_s), cvt.conv_weights_pack(w_t)
    y = cvt.upsample3d_packed(x, pw_s, pw_t, b_s, b_t, space=space, time=time)
    r = cvt.upsample3d(x, w_s, w_t, b_s, b_t, space=space, time=time)
    torch.cuda.synchronize()
    _same(y, r, f"upsampling {case}")
