"""cvt_causal_conv3d_fact_noalloc (the factorized conv with the library's preallocated
scratch in place of a workspace) against cvt_causal_conv3d_fact with a caller workspace:
bit-identical outputs on two calls in a row, the second with a smaller input (the
scratch keeps the first call's contents), for both parts, spatial only and temporal
only; the first also against the float64 oracle, |g - o| <= 2e-2 (|o| + rms(o)).  A
call that would need more than the preallocated scratch returns CVT_E_WORKSPACE and
writes nothing."""

import ctypes

import numpy as np
import pytest
import torch

import synthetic_inputs as si
from oracle import bf16 as obf16
from oracle import conv as oconv
from tests.gpu_helpers import assert_rel, bits_to_torch, f32_to_torch, log, to_bits, to_f64

pytestmark = pytest.mark.gpu

cvt = pytest.importorskip("causal_video_tokenizer_amd")
E_WORKSPACE = 7


def _case(B, Cin, Cout, T, H, W, bias, seed):
    xb = si.to_bf16_bits(si.normal((B, Cin, T, H, W), seed, 1.0))
    wsb = si.to_bf16_bits(si.normal((Cout, Cin, 1, 3, 3), seed + 1, 0.02))
    wtb = si.to_bf16_bits(si.normal((Cout, Cout, 3, 1, 1), seed + 2, 0.02))
    bs = si.normal((Cout,), seed + 3, 0.1) if bias else None
    bt = si.normal((Cout,), seed + 4, 0.1) if bias else None
    dev = dict(x=bits_to_torch(xb, channels_last=True), w_s=bits_to_torch(wsb), w_t=bits_to_torch(wtb),
               b_s=f32_to_torch(bs) if bias else None, b_t=f32_to_torch(bt) if bias else None)
    ref = dict(x=obf16.decode(xb), ws=obf16.decode(wsb), wt=obf16.decode(wtb), bs=bs, bt=bt)
    return dev, ref


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _noalloc(x, w_s, w_t, b_s, b_t, y):
    """One call through the C ABI; returns the status."""
    B, Cin, T, H, W = x.shape
    Cout = y.shape[1]
    st = cvt.lib.cvt_causal_conv3d_fact_noalloc(_p(x), _p(w_s), _p(w_t), _p(b_s), _p(b_t), _p(y), B, Cin, Cout, T, H,
                                                W, 3, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def _out(x, Cout):
    B, _, T, H, W = x.shape
    return torch.full((B, Cout, T, H, W), 7.0, dtype=torch.bfloat16, device=x.device).to(
        memory_format=torch.channels_last_3d)


@pytest.mark.parametrize("parts", ["both", "spatial", "temporal"])
def test_noalloc_equals_workspace_call_twice(parts):
    cases = [(1, 192, 256, 5, 64, 64, True, 901), (2, 64, 64, 3, 8, 12, False, 902)]  # second call smaller
    for i, (B, Cin, Cout, T, H, W, bias, seed) in enumerate(cases):
        if parts == "temporal":
            Cin = Cout
        log(f"no-alloc call {i}: parts={parts} B={B} Cin={Cin} Cout={Cout} T={T} H={H} W={W} bias={bias}")
        dev, ref = _case(B, Cin, Cout, T, H, W, bias, seed)
        w_s = dev["w_s"] if parts != "temporal" else None
        w_t = dev["w_t"] if parts != "spatial" else None
        b_s = dev["b_s"] if parts != "temporal" else None
        b_t = dev["b_t"] if parts != "spatial" else None
        need = cvt.conv_workspace_bytes(dev["x"].shape, Cout, 3, w_s is not None, w_t is not None)
        assert need <= cvt.NOALLOC_SCRATCH_BYTES
        y = _out(dev["x"], Cout)
        assert _noalloc(dev["x"], w_s, w_t, b_s, b_t, y) == 0, cvt.lib.cvt_last_error()
        y_ref = cvt.causal_conv3d_fact(dev["x"], w_s, w_t, b_s, b_t)
        torch.cuda.synchronize()
        g, r = to_bits(y), to_bits(y_ref)
        log(f"  identical to the workspace call: {int(np.sum(g == r))}/{g.size}")
        assert np.array_equal(g, r)
        if i == 0:
            if parts == "both":
                o = oconv.causal_conv3d_fact(ref["x"], ref["ws"], ref["wt"], ref["bs"], ref["bt"])
            elif parts == "spatial":
                o = oconv.spatial_conv(ref["x"], ref["ws"], ref["bs"])
            else:
                o = oconv.temporal_conv(ref["x"], ref["wt"], ref["bt"])
            assert_rel(to_f64(y), o, 2e-2, "no-alloc conv vs oracle")


def test_noalloc_rejects_calls_beyond_the_scratch():
    # both parts at 256 channels on 160,000 positions: the bf16 intermediate alone is 82 MB
    x = torch.zeros((1, 256, 10, 100, 160), dtype=torch.bfloat16, device="cuda").to(
        memory_format=torch.channels_last_3d)
    w_s = torch.zeros((256, 256, 1, 3, 3), dtype=torch.bfloat16, device="cuda")
    w_t = torch.zeros((256, 256, 3, 1, 1), dtype=torch.bfloat16, device="cuda")
    assert cvt.conv_workspace_bytes(x.shape, 256, 3) > cvt.NOALLOC_SCRATCH_BYTES
    y = _out(x, 256)
    assert _noalloc(x, w_s, w_t, None, None, y) == E_WORKSPACE
    assert b"preallocated scratch" in cvt.lib.cvt_last_error()
    torch.cuda.synchronize()
    assert bool(torch.all(y == 7.0)), "nothing may be written on an error"
    # the same shape without the temporal part needs only the packed weights
    assert _noalloc(x, w_s, None, None, None, y) == 0
    torch.cuda.synchronize()
    assert bool(torch.all(y == 0.0))
