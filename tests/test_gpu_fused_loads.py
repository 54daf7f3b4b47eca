"""Cross-stage fusions inside the convolution's operand loads, on the GPU.

* The Haar patcher inside the first conv (haar3d_conv3d_fact): the spatial conv computes the
  192 coefficient channels from the pixel clip while staging them.  Checked against the
  float64 oracle (Haar of the pixels, rounded to bf16 as the coefficients the conv stages,
  then the factorized conv), |g - o| <= 2e-2 (|o| + rms(o)), and against the unfused GPU
  route (haar3d_fwd then causal_conv3d_fact): the staged coefficients come from a different
  order of the same additions, so outputs agree to a bf16 rounding step.
* FSQ dequantize + the 1x1 projection inside the decoder's first conv
  (fsq_dequantize_conv3d_fact): bit for bit against fsq_dequantize_proj followed by
  causal_conv3d_fact (NaN of invalid indices included), and against the oracle (dequantize,
  the projection rounded to bf16, the conv).
"""

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import bf16 as obf16
from oracle import conv as oconv
from oracle import fsq as ofsq
from oracle import haar as ohaar
from tests.gpu_helpers import assert_rel, bits_to_torch, f32_to_torch, log, rel_report, to_bits, to_f64

pytestmark = pytest.mark.gpu

cvt = pytest.importorskip("causal_video_tokenizer_amd")
TOL = 2e-2
LEVELS = (8, 8, 8, 5, 5, 5)


def bf16_dev(shape, seed, std, cl=False):
    bits = si.to_bf16_bits(si.normal(shape, seed, std))
    return bits_to_torch(bits, channels_last=cl), obf16.decode(bits)


HAAR_CASES = [
    # B, T, H, W, Cout, temporal, bias: ragged 32-column tiles and row tiles, T' = 1, 2 clips
    (1, 5, 32, 48, 64, False, False),
    (1, 9, 40, 136, 256, True, True),
    (2, 17, 24, 40, 192, True, False),
    (1, 1, 16, 16, 128, True, True),
    (1, 13, 20, 260, 256, False, True),
]


@pytest.mark.parametrize("case", HAAR_CASES)
def test_haar_conv_fused_vs_oracle_and_unfused(case):
    B, T, H, W, Cout, temporal, bias = case
    log(f"haar-fused conv {case}")
    seed = 1200 + T + H + Cout
    xb = si.to_bf16_bits(si.video_sin((B, 3, T, H, W), seed))
    x = bits_to_torch(xb)
    ws, ws64 = bf16_dev((Cout, 192, 1, 3, 3), seed + 1, 0.02)
    wt, wt64 = bf16_dev((Cout, Cout, 3, 1, 1), seed + 2, 0.02) if temporal else (None, None)
    bs = si.normal((Cout,), seed + 3, 0.1) if bias else None
    bt = si.normal((Cout,), seed + 4, 0.1) if (bias and temporal) else None
    dbs = f32_to_torch(bs) if bs is not None else None
    dbt = f32_to_torch(bt) if bt is not None else None
    y = cvt.haar3d_conv3d_fact(x, ws, wt, dbs, dbt)
    y_ref = cvt.causal_conv3d_fact(cvt.haar3d_fwd(x), ws, wt, dbs, dbt)
    torch.cuda.synchronize()
    assert y.shape == (B, Cout, 1 + (T - 1) // 4, H // 4, W // 4)
    h64 = obf16.round_to_bf16(ohaar.haar3d_fwd(obf16.decode(xb), 2))
    o = oconv.causal_conv3d_fact(h64, ws64, wt64, bs, bt)
    assert_rel(to_f64(y), o, TOL, "fused vs oracle")
    g, r = to_bits(y), to_bits(y_ref)
    same = float(np.mean(g == r))
    nbad, worst, rel = rel_report(to_f64(y), to_f64(y_ref), 1e-2)
    log(f"  fused vs unfused: identical {same:.4f}, relL2 {rel:.2e}, beyond 1e-2: {nbad}")
    assert nbad == 0 and same > 0.9


def test_haar_conv_fused_dv8x16x16_720p_frames():
    """The 49-frame 720p clip through the fused spatial conv 192 -> 256 (the route the
    benchmark times as the fused alternative): latent frames 0, 5 and 12 in full against the
    oracle, and the whole output against the unfused route."""
    cid = 4
    wl = si.WORKLOADS["c4_dv8x16x16_720p_49f"]
    xb = si.to_bf16_bits(si.video_trans(wl["x"], wl["seed"]))
    x = bits_to_torch(xb)
    ws, ws64 = bf16_dev((256, 192, 1, 3, 3), si.weight_seed(cid, 0), 0.02)
    y = cvt.haar3d_conv3d_fact(x, ws)
    y_ref = cvt.causal_conv3d_fact(cvt.haar3d_fwd(x), ws)
    torch.cuda.synchronize()
    diff = (y.float() - y_ref.float()).abs()
    tol = 1e-2 * (y_ref.float().abs() + y_ref.float().pow(2).mean().sqrt())
    nbad = int((diff > tol).sum().item())
    same = float((y.view(torch.int16) == y_ref.view(torch.int16)).float().mean().item())
    log(f"  whole clip fused vs unfused: identical {same:.4f}, beyond 1e-2: {nbad}")
    assert nbad == 0
    for tq in (0, 5, 12):
        f0 = 0 if tq == 0 else 4 * tq - 3
        px = obf16.decode(xb[:, :, f0:4 * tq + 1])
        h = ohaar.haar3d_fwd(px, 2 if tq == 0 else 3)
        o = oconv.spatial_conv(obf16.round_to_bf16(h), ws64)
        assert_rel(to_f64(y[:, :, tq:tq + 1]), o, TOL, f"frame {tq}")
    del x, y, y_ref
    torch.cuda.empty_cache()


FSQ_CASES = [
    # B, T, H, W, Cmid, Cout, temporal, bias, levels
    (1, 3, 9, 13, 64, 64, False, False, LEVELS),
    (2, 5, 12, 40, 192, 192, True, True, LEVELS),   # 3-wave tiles of 3 rows (4 row tiles)
    (1, 3, 10, 35, 160, 136, True, False, LEVELS),  # Cout 136 of 192, ragged row and column tiles
    (1, 4, 7, 70, 256, 256, True, False, LEVELS),
    (1, 2, 8, 8, 96, 128, True, True, (8, 5, 5, 5)),
    (1, 1, 10, 33, 192, 64, False, True, (7, 5, 5, 5, 3)),
]


def _fsq_case(B, T, H, W, Cmid, Cout, temporal, bias, levels, seed):
    D = len(levels)
    n = int(np.prod(levels))
    idx_np = si.uniform_indices((B, T, H, W), seed, n)
    idx = torch.from_numpy(idx_np).cuda()
    wl, wl64 = bf16_dev((Cmid, D, 1, 1, 1), seed + 1, 0.3)
    ws, ws64 = bf16_dev((Cout, Cmid, 1, 3, 3), seed + 2, 0.02)
    wt, wt64 = bf16_dev((Cout, Cout, 3, 1, 1), seed + 3, 0.02) if temporal else (None, None)
    bl = si.normal((Cmid,), seed + 4, 0.1) if bias else None
    bs = si.normal((Cout,), seed + 5, 0.1) if bias else None
    bt = si.normal((Cout,), seed + 6, 0.1) if (bias and temporal) else None
    dev = dict(idx=idx, wl=wl, ws=ws, wt=wt, bl=f32_to_torch(bl) if bias else None,
               bs=f32_to_torch(bs) if bias else None, bt=f32_to_torch(bt) if bt is not None else None)
    ref = dict(idx=idx_np, wl=wl64, ws=ws64, wt=wt64, bl=bl, bs=bs, bt=bt)
    return dev, ref


@pytest.mark.parametrize("case", FSQ_CASES)
def test_fsq_conv_fused_equals_unfused_and_oracle(case):
    B, T, H, W, Cmid, Cout, temporal, bias, levels = case
    log(f"fsq-fused conv {case}")
    dev, ref = _fsq_case(*case, seed=1300 + Cmid + Cout + T)
    y = cvt.fsq_dequantize_conv3d_fact(dev["idx"], dev["wl"], dev["ws"], dev["wt"], dev["bl"], dev["bs"], dev["bt"],
                                       levels=levels)
    z = cvt.fsq_dequantize_proj(dev["idx"], dev["wl"], dev["bl"], levels=levels)
    y_ref = cvt.causal_conv3d_fact(z, dev["ws"], dev["wt"], dev["bs"], dev["bt"])
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(y), to_bits(y_ref)), "fused differs from dequantize_proj + conv"
    codes, _ = ofsq.dequantize(ref["idx"], levels)
    z64 = obf16.round_to_bf16(oconv.pointwise(codes, ref["wl"], ref["bl"]))
    o = oconv.causal_conv3d_fact(z64, ref["ws"], ref["wt"], ref["bs"], ref["bt"])
    assert_rel(to_f64(y), o, TOL, "fused vs oracle")


def test_fsq_conv_fused_invalid_indices_bit_exact():
    dev, _ = _fsq_case(1, 3, 6, 9, 64, 64, True, False, LEVELS, seed=1401)
    idx = dev["idx"].clone()
    idx[0, 1, 2, 3] = -5
    idx[0, 2, 5, 8] = 64000
    y = cvt.fsq_dequantize_conv3d_fact(idx, dev["wl"], dev["ws"], dev["wt"])
    y_ref = cvt.causal_conv3d_fact(cvt.fsq_dequantize_proj(idx, dev["wl"]), dev["ws"], dev["wt"])
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(y), to_bits(y_ref))
    assert bool(torch.isnan(y[0, :, 1, 2, 3]).all()), "an invalid index poisons its neighbourhood"
    assert not bool(torch.isnan(y[0, :, 0]).any()), "frames before the invalid one stay finite (causal)"


def test_fsq_conv_fused_dv4x8x8_360p_decode():
    """The batched DV4x8x8-360p decode's first layers: 8 x 13 x 90 x 160 indices -> the 6 -> 192
    projection inside the conv 192 -> 192 (spatial + temporal), bit for bit against the
    unfused route on the whole output."""
    cid = 5
    wl_ = si.WORKLOADS["c5_dv4x8x8_360p_decode"]
    idx = torch.from_numpy(si.uniform_indices(wl_["indices"], wl_["seed"])).cuda()
    lift = bf16_dev((192, 6, 1, 1, 1), si.weight_seed(cid, 0), 0.02)[0]
    ws = bf16_dev((192, 192, 1, 3, 3), si.weight_seed(cid, 1), 0.02)[0]
    wt = bf16_dev((192, 192, 3, 1, 1), si.weight_seed(cid, 2), 0.02)[0]
    y = cvt.fsq_dequantize_conv3d_fact(idx, lift, ws, wt)
    y_ref = cvt.causal_conv3d_fact(cvt.fsq_dequantize_proj(idx, lift), ws, wt)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    del y, y_ref
    torch.cuda.empty_cache()
