"""Cross-stage fusions on the GPU: FSQ computed in the epilogue of the conv's fused 1x1
projection, and FSQ dequantize fused with the decoder's 1x1 projection.  Each is checked
bit for bit against the unfused kernels it replaces (whose parity with the oracle the other
GPU tests establish) and against the oracle directly: the indices against the oracle's FSQ
of the GPU's bf16 latent (bit-exact away from rounding boundaries), the dequantized
projection against the oracle's codes times the weights."""

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import bf16 as obf16
from oracle import conv as oconv
from oracle import fsq as ofsq
from tests.gpu_helpers import assert_rel, bits_to_torch, f32_to_torch, log, to_bits, to_f64

pytestmark = pytest.mark.gpu

cvt = pytest.importorskip("causal_video_tokenizer_amd")
LEVELS = (8, 8, 8, 5, 5, 5)


def bf16_dev(shape, seed, std, cl=False):
    bits = si.to_bf16_bits(si.normal(shape, seed, std))
    return bits_to_torch(bits, channels_last=cl), obf16.decode(bits)


FSQ_CASES = [
    # B, Cin, Cout, T, H, W, k, spatial, bias, levels: fused in the 256-channel temporal
    # epilogue, on the 128-channel tiles, temporal only, two clips; then the unfused routes
    # (no temporal part; Cout above 256)
    (1, 192, 256, 5, 12, 20, 3, True, False, LEVELS),
    (1, 64, 128, 3, 9, 13, 3, True, True, LEVELS),
    (2, 256, 256, 4, 6, 11, 3, False, True, LEVELS),
    (1, 128, 256, 3, 8, 8, 3, True, False, (8, 5, 5, 5)),
    (1, 256, 256, 2, 8, 8, 1, True, False, LEVELS),
    (1, 64, 320, 3, 5, 7, 3, True, False, LEVELS),
]


@pytest.mark.parametrize("case", FSQ_CASES)
def test_conv_proj_fsq_equals_unfused_and_oracle(case):
    B, Cin, Cout, T, H, W, k, spatial, bias, levels = case
    log(f"conv+proj+fsq {case}")
    D = len(levels)
    x, _ = bf16_dev((B, Cin, T, H, W), 900 + Cin, 1.0, cl=True)
    ws = bf16_dev((Cout, Cin, 1, k, k), 901, 0.02)[0] if spatial else None
    wt = bf16_dev((Cout, Cout, k, 1, 1), 902, 0.02)[0] if k == 3 else None
    wp = bf16_dev((D, Cout, 1, 1, 1), 903, 0.15)[0]
    bt = f32_to_torch(si.normal((Cout,), 904, 0.1)) if (bias and wt is not None) else None
    bp = f32_to_torch(si.normal((D,), 905, 0.3)) if bias else None
    lat_ref = cvt.causal_conv3d_fact_proj(x, ws, wt, wp, b_t=bt, b_p=bp)
    idx_ref = cvt.fsq_quantize(lat_ref, levels=levels)
    idx, lat = cvt.causal_conv3d_fact_proj_fsq(x, ws, wt, wp, b_t=bt, b_p=bp, levels=levels, return_latent=True)
    idx2 = cvt.causal_conv3d_fact_proj_fsq(x, ws, wt, wp, b_t=bt, b_p=bp, levels=levels)  # no latent written
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(lat), to_bits(lat_ref))
    gi = idx.cpu().numpy()
    assert np.array_equal(gi, idx_ref.cpu().numpy())
    assert np.array_equal(idx2.cpu().numpy(), gi)
    oi, _, dist = ofsq.quantize(obf16.decode(to_bits(lat)), levels)
    off = dist >= 1e-6
    log(f"  positions={gi.size} spread of indices={len(np.unique(gi))} boundary={int((~off).sum())}")
    assert np.array_equal(gi[off], oi[off])
    assert len(np.unique(gi)) > min(gi.size // 10, 200)  # the latent spans many codes


def test_conv_proj_fsq_nan_latent_gives_minus_one():
    B, C, T, H, W = 1, 128, 3, 4, 8
    x, _ = bf16_dev((B, C, T, H, W), 910, 1.0, cl=True)
    x[0, :, 1, 2, 3] = float("nan")  # poisons frames 1 and 2 of position (2, 3) through the causal taps
    wt = bf16_dev((C, C, 3, 1, 1), 911, 0.02)[0]
    wp = bf16_dev((6, C, 1, 1, 1), 912, 0.15)[0]
    idx = cvt.causal_conv3d_fact_proj_fsq(x, None, wt, wp)
    ref = cvt.fsq_quantize(cvt.causal_conv3d_fact_proj(x, None, wt, wp))
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    assert np.array_equal(gi, ref.cpu().numpy())
    assert gi[0, 1, 2, 3] == -1 and gi[0, 2, 2, 3] == -1 and gi[0, 0, 2, 3] >= 0


DQ_CASES = [
    # B, T, H, W, Cout, bias, levels
    (1, 13, 9, 16, 192, True, LEVELS),     # the DV4x8x8-360p latent grid, cut down
    (2, 3, 5, 7, 64, False, LEVELS),
    (1, 2, 4, 4, 20, True, LEVELS),        # Cout not a multiple of 8
    (1, 3, 4, 5, 48, False, (7, 6, 5)),    # codes not exact in bf16 (halves 3)
    (1, 5, 7, 11, 72, True, LEVELS),       # 9 channel groups per position
    (2, 3, 6, 9, 256, False, (7, 6, 5, 9)),  # four levels, halves 3 and 4
]


@pytest.mark.parametrize("case", DQ_CASES)
def test_dequantize_proj_equals_unfused_and_oracle(case):
    B, T, H, W, Cout, bias, levels = case
    log(f"dequant+proj {case}")
    D = len(levels)
    n = int(np.prod(levels))
    idx_np = si.uniform_indices((B, T, H, W), 920 + Cout, high=n)
    idx = torch.from_numpy(idx_np).cuda()
    wp, wp64 = bf16_dev((Cout, D, 1, 1, 1), 921, 0.2)
    bp = f32_to_torch(si.normal((Cout,), 922, 0.1)) if bias else None
    y = cvt.fsq_dequantize_proj(idx, wp, bp, levels=levels)
    codes = cvt.fsq_dequantize(idx, levels=levels)  # bf16 NTHWC
    y2 = cvt.causal_conv3d_fact(codes, wp, None, b_s=bp)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(y), to_bits(y2))
    oc, bad = ofsq.dequantize(idx_np, levels)
    assert bad == 0
    ref = oconv.pointwise(oc, wp64[:, :, 0, 0, 0], bp.cpu().double().numpy() if bias else None)
    assert_rel(to_f64(y), ref, 1e-2, "dequant+proj")


@pytest.mark.parametrize("Cout", [64, 192])
def test_dequantize_proj_invalid_indices(Cout):
    idx_np = si.uniform_indices((1, 2, 4, 8), 930)
    idx_np[0, 0, 0, :3] = [-1, 64000, 2 ** 31 - 1]
    idx = torch.from_numpy(idx_np).cuda()
    wp, _ = bf16_dev((Cout, 6, 1, 1, 1), 931, 0.2)
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = cvt.fsq_dequantize_proj(idx, wp, invalid_count=cnt)
    torch.cuda.synchronize()
    assert int(cnt.item()) == 3
    g = to_f64(y)
    assert np.isnan(g[0, :, 0, 0, :3]).all() and not np.isnan(g[0, :, 0, 0, 3:]).any()
    assert not np.isnan(g[0, :, 1]).any()
