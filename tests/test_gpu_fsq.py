"""GPU parity of cvt_fsq_quantize / cvt_fsq_dequantize against the oracle:
indices bit-exact, codes bit-exact, boundary positions reported."""

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import bf16 as obf16
from oracle import fsq as ofsq
from tests.gpu_helpers import bits_to_torch, f32_to_torch, log, to_f64

pytestmark = pytest.mark.gpu

cvt = pytest.importorskip("causal_video_tokenizer_amd")
LEVELS = (8, 8, 8, 5, 5, 5)


def check_quantize(z_t, z64, levels=LEVELS, what=""):
    idx, codes = cvt.fsq_quantize(z_t, levels=levels, return_codes=True)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy().astype(np.int64)
    oi, oc, dist = ofsq.quantize(z64, levels)
    boundary = dist < 1e-6
    mism = gi != oi
    nb = int(boundary.sum())
    log(f"  {what}: positions={oi.size} boundary(<1e-6)={nb} mismatches: off-boundary="
        f"{int((mism & ~boundary).sum())} on-boundary={int((mism & boundary).sum())}")
    assert not np.any(mism & ~boundary), "FSQ index mismatch away from a rounding boundary"
    gc = to_f64(codes)
    if z_t.dtype == torch.float32:
        oc = oc.astype(np.float32).astype(np.float64)
    else:
        oc = obf16.round_to_bf16(oc)
    same = (gc == oc) | (np.isnan(gc) & np.isnan(oc))
    ok_codes = same | np.broadcast_to(boundary[:, None], same.shape)
    assert ok_codes.all(), "FSQ codes mismatch"
    return gi, oi, boundary


@pytest.mark.parametrize("layout", ["NCTHW", "NTHWC"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_c4_latent(layout, dtype):
    """The N(0, 1.5) latent of shape 1 x 6 x 13 x 180 x 320 (748,800 positions)."""
    wl = si.WORKLOADS["c4_dv8x16x16_720p_49f"]
    z = si.normal(wl["latent"], wl["latent_seed"], wl["latent_std"])
    if dtype == "bf16":
        bits = si.to_bf16_bits(z)
        zt, z64 = bits_to_torch(bits, channels_last=(layout == "NTHWC")), obf16.decode(bits)
    else:
        zt, z64 = f32_to_torch(z, channels_last=(layout == "NTHWC")), z.astype(np.float64)
    gi, oi, boundary = check_quantize(zt, z64, what=f"c4 latent {dtype} {layout}")
    assert np.array_equal(gi, oi), "the exact breakpoint decision should also agree on boundary positions"
    assert len(np.unique(gi)) > 60000


@pytest.mark.parametrize("shape", [(1, 6, 3, 5, 7), (3, 6, 1, 1, 13), (2, 6, 2, 4, 4), (1, 6, 1, 1, 1)])
@pytest.mark.parametrize("layout", ["NCTHW", "NTHWC"])
def test_quantize_ragged_shapes(shape, layout):
    z = si.normal(shape, 21, 1.5)
    bits = si.to_bf16_bits(z)
    check_quantize(bits_to_torch(bits, channels_last=(layout == "NTHWC")), obf16.decode(bits),
                   what=f"ragged {shape} {layout}")


def test_quantize_special_values_and_breakpoint_neighbours():
    """NaN -> -1, +-inf saturate, and float32 values adjacent to every
    breakpoint (where the bound crosses a half-integer) take the float64
    definition's decision."""
    vals = [0.0, -0.0, np.inf, -np.inf, 50.0, -50.0, 1e-30, -1e-30]
    for L in sorted(set(LEVELS)):
        h, o, s = ofsq.constants(L)
        half = L // 2
        for j in range(-half, L - half - 1):
            zb = np.arctanh((j + 0.5 + o) / h) - s
            f = np.float32(zb)
            up = dn = f
            vals.append(float(f))
            for _ in range(3):
                up = np.nextafter(up, np.float32(np.inf))
                dn = np.nextafter(dn, np.float32(-np.inf))
                vals += [float(up), float(dn)]
    vals = np.array(vals, dtype=np.float32)
    n = len(vals)
    z = np.zeros((1, 6, 1, 1, n * 6), dtype=np.float32)
    for i in range(6):
        z[0, i, 0, 0, :] = np.roll(np.tile(vals, 6), 7 * i)
    z[0, 3, 0, 0, 5] = np.nan
    gi, oi, _ = check_quantize(f32_to_torch(z), z.astype(np.float64), what="breakpoint neighbours")
    assert np.array_equal(gi, oi)
    assert gi[0, 0, 0, 5] == -1


@pytest.mark.parametrize("levels", [(7, 5, 3, 16), (2, 2, 2), (8, 8, 8, 5, 5, 5, 4, 3), (11,)])
def test_other_level_sets(levels):
    D = len(levels)
    z = si.normal((2, D, 3, 4, 8), 31, 1.5)
    gi, oi, _ = check_quantize(f32_to_torch(z), z.astype(np.float64), levels=levels, what=f"levels {levels}")
    assert np.array_equal(gi, oi)
    codes = cvt.fsq_dequantize(torch.from_numpy(oi.astype(np.int32)).cuda(), levels=levels, dtype=torch.float32,
                               layout="NCTHW")
    torch.cuda.synchronize()
    oc, bad = ofsq.dequantize(oi, levels)
    assert bad == 0
    assert np.array_equal(to_f64(codes), oc.astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("layout", ["NCTHW", "NTHWC"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_dequantize_all_indices_and_invalid(layout, dtype):
    idx = np.concatenate([np.arange(64000), [-1, 64000, 2**31 - 1, -2**31, 123, 63999, 0, 64001]]).astype(np.int32)
    idx = idx.reshape(1, 1, 1, -1)
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    codes = cvt.fsq_dequantize(torch.from_numpy(idx).cuda(), dtype=dtype, layout=layout, invalid_count=cnt)
    torch.cuda.synchronize()
    oc, bad = ofsq.dequantize(idx, LEVELS)
    gc = to_f64(codes)
    same = (gc == oc) | (np.isnan(gc) & np.isnan(oc))
    assert same.all()
    assert int(cnt.item()) == bad == 5
    # every valid index survives quantize(lattice centre of its codes): the latent
    # whose bound is exactly the integer q = code * floor(L/2), via the inverse of tanh
    valid = idx[..., :64000]
    zc = np.empty_like(oc[..., :64000])
    for i, L in enumerate(LEVELS):
        h, o, s = ofsq.constants(L)
        q = oc[:, i, ..., :64000] * (L // 2)
        zc[:, i] = np.arctanh((q + o) / h) - s
    z = torch.from_numpy(zc.astype(np.float32)).cuda()
    assert np.array_equal(cvt.fsq_quantize(z).cpu().numpy(), valid)


def test_dequantize_c5_grid():
    """Uniform indices on the 8 x 13 x 90 x 160 decode-side grid, NTHWC bf16 codes."""
    wl = si.WORKLOADS["c5_dv4x8x8_360p_decode"]
    idx = si.uniform_indices(wl["indices"], wl["seed"])
    codes = cvt.fsq_dequantize(torch.from_numpy(idx).cuda(), dtype=torch.bfloat16, layout="NTHWC")
    torch.cuda.synchronize()
    assert codes.is_contiguous(memory_format=torch.channels_last_3d)
    oc, bad = ofsq.dequantize(idx, LEVELS)
    assert bad == 0
    assert np.array_equal(to_f64(codes), oc)


def test_bandwidth_size_sampled():
    """The 64 x 6 x 13 x 180 x 320 latent used for bandwidth: checked on sampled batches."""
    shape = (64, 6, 13, 180, 320)
    z = si.normal(shape, 1015, 1.5)
    bits = si.to_bf16_bits(z)
    del z
    zt = bits_to_torch(bits)
    idx = cvt.fsq_quantize(zt)
    codes = cvt.fsq_dequantize(idx, dtype=torch.bfloat16, layout="NCTHW")
    torch.cuda.synchronize()
    for b in (0, 31, 63):
        zb = obf16.decode(bits[b:b + 1])
        oi, _, dist = ofsq.quantize(zb, LEVELS)
        gi = idx[b:b + 1].cpu().numpy()
        assert np.array_equal(gi, oi), b
        oc, _ = ofsq.dequantize(oi, LEVELS)
        assert np.array_equal(to_f64(codes[b:b + 1]), oc)
    del zt, idx, codes
    torch.cuda.empty_cache()
