"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol include/cvt.h declares, and rejects invalid arguments before any
launch with the documented status codes."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cvt.h")

cvt = pytest.importorskip("causal_video_tokenizer_amd", reason="libcvt.so not built")
lib = cvt.lib

OK, E_NULL, E_SHAPE, E_DTYPE, E_LAYOUT, E_ALIGN, E_LEVELS, E_WORKSPACE = range(8)
# Fake, 256-byte aligned "device" addresses: every call below fails validation,
# so nothing is ever dereferenced or launched.
A, B_, C_ = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), ctypes.c_void_p(0x300000)
MIS = ctypes.c_void_p(0x100008)


def header_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(cvt_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound():
    names = header_symbols()
    assert len(names) == 46
    for n in names:
        assert hasattr(lib, n), n
        assert n in cvt.SIGNATURES, n


def test_version_and_status_strings():
    assert lib.cvt_abi_version() == 1
    assert lib.cvt_status_string(0) == b"CVT_OK"
    for s in range(1, 9):
        assert lib.cvt_status_string(s).startswith(b"CVT_E_")
    assert lib.cvt_status_string(99) == b"unknown cvt status"


def fwd(*, x=A, xdt=1, y=B_, ydt=1, lay=1, B=1, C=3, T=5, H=8, W=8, tl=2):
    return lib.cvt_haar3d_fwd(x, xdt, y, ydt, lay, B, C, T, H, W, tl, None)


def test_haar_validation():
    assert fwd(x=None) == E_NULL
    assert fwd(xdt=7) == E_DTYPE
    assert fwd(lay=5) == E_LAYOUT
    assert fwd(T=4) == E_SHAPE            # T != 1 + 4k
    assert fwd(H=6) == E_SHAPE
    assert fwd(W=10) == E_SHAPE
    assert fwd(tl=1) == E_SHAPE
    assert fwd(B=0) == E_SHAPE
    assert fwd(x=MIS) == E_ALIGN
    assert fwd(T=4) == E_SHAPE and b"T = 1 + 4k" in lib.cvt_last_error()
    assert fwd(x=MIS) == E_ALIGN and b"aligned" in lib.cvt_last_error()
    assert lib.cvt_haar3d_inv(A, 1, 1, B_, 1, 1, 3, 6, 8, 8, 2, None) == E_SHAPE
    assert lib.cvt_haar3d_inv(None, 1, 1, B_, 1, 1, 3, 5, 8, 8, 2, None) == E_NULL


def levels(*ls):
    return (ctypes.c_int32 * len(ls))(*ls)


def test_fsq_validation():
    L = levels(8, 8, 8, 5, 5, 5)
    q = lambda **kw: lib.cvt_fsq_quantize(kw.get("z", A), kw.get("dt", 1), kw.get("lay", 0), kw.get("idx", B_),
                                          None, kw.get("lv", L), kw.get("D", 6), 1, 2, 4, 4, None)
    assert q(z=None) == E_NULL
    assert q(idx=None) == E_NULL
    assert q(dt=3) == E_DTYPE
    assert q(lay=2) == E_LAYOUT
    assert q(lv=None) == E_NULL
    assert q(D=0) == E_LEVELS
    assert q(D=9) == E_LEVELS
    assert q(lv=levels(8, 1, 8, 5, 5, 5)) == E_LEVELS
    assert q(lv=levels(8, 17, 8, 5, 5, 5)) == E_LEVELS
    assert q(lv=levels(16, 16, 16, 16, 16, 16, 16, 16), D=8) == E_LEVELS   # 2^32 codes
    assert q(z=MIS) == E_ALIGN
    dq = lambda **kw: lib.cvt_fsq_dequantize(kw.get("idx", A), kw.get("c", B_), 1, 1, L, 6, 1, 2, 4, 4,
                                             kw.get("cnt", None), None)
    assert dq(idx=None) == E_NULL
    assert dq(c=MIS) == E_ALIGN
    assert dq(cnt=ctypes.c_void_p(0x100002)) == E_ALIGN


def test_conv_validation_and_workspace():
    ws = lib.cvt_causal_conv3d_fact_workspace(1, 192, 256, 5, 8, 8, 3, 3)
    P = 5 * 8 * 8
    assert ws >= 256 * 192 * 9 * 2 + 256 * 256 * 3 * 2 + P * 256 * 2
    assert lib.cvt_causal_conv3d_fact_workspace(1, 192, 256, 5, 8, 8, 2, 3) == 0
    assert lib.cvt_causal_conv3d_fact_workspace(1, 192, 256, 5, 8, 8, 3, 1) < ws
    assert lib.cvt_causal_conv3d_fact_workspace(1, 256, 256, 5, 8, 8, 3, 2) == 256 * 256 * 3 * 2
    assert lib.cvt_causal_conv3d_fact_workspace(1, 192, 256, 5, 8, 8, 3, 0) == 0

    def call(**kw):
        return lib.cvt_causal_conv3d_fact(kw.get("x", A), kw.get("ws", B_), kw.get("wt", C_), None, None,
                                          kw.get("y", ctypes.c_void_p(0x400000)), 1, kw.get("Cin", 192),
                                          kw.get("Cout", 256), 5, 8, 8, kw.get("k", 3),
                                          kw.get("work", ctypes.c_void_p(0x500000)), kw.get("wsb", ws), None)
    assert call(x=None) == E_NULL
    assert call(ws=None, wt=None) == E_NULL
    assert call(ws=None) == E_SHAPE           # temporal-only needs Cin == Cout
    assert call(k=2) == E_SHAPE
    assert call(Cin=12) == E_SHAPE            # not a multiple of 8 with k = 3
    assert call(Cout=12) == E_SHAPE           # temporal part needs Cout % 8 == 0
    assert call(Cout=5000) == E_SHAPE
    assert call(x=MIS) == E_ALIGN
    assert call(wsb=ws - 1) == E_WORKSPACE
    assert call(work=None) == E_WORKSPACE


def test_conv_proj_validation_and_workspace():
    """The fused conv + 1x1 entry point: workspace query (fused path: no Cout-channel
    intermediate for a temporal-only call; fallback path: it is included) and argument
    checks before any launch."""
    P = 5 * 8 * 8
    fused = lib.cvt_causal_conv3d_fact_proj_workspace(1, 256, 256, 6, 5, 8, 8, 3, 2)
    assert 256 * 256 * 3 * 2 <= fused < 256 * 256 * 3 * 2 + P * 256 * 2
    both = lib.cvt_causal_conv3d_fact_proj_workspace(1, 192, 256, 6, 5, 8, 8, 3, 3)
    assert both >= 256 * 192 * 9 * 2 + 256 * 256 * 3 * 2 + P * 256 * 2
    wide = lib.cvt_causal_conv3d_fact_proj_workspace(1, 256, 256, 24, 5, 8, 8, 3, 2)  # Cp > 16: two passes
    assert wide >= 256 * 256 * 3 * 2 + P * 256 * 2
    assert lib.cvt_causal_conv3d_fact_proj_workspace(1, 256, 256, 0, 5, 8, 8, 3, 2) == 0
    assert lib.cvt_causal_conv3d_fact_proj_workspace(1, 256, 256, 6, 5, 8, 8, 2, 2) == 0

    def call(**kw):
        return lib.cvt_causal_conv3d_fact_proj(kw.get("x", A), kw.get("ws", B_), kw.get("wt", C_), None, None,
                                               kw.get("wp", ctypes.c_void_p(0x600000)), None,
                                               kw.get("y", ctypes.c_void_p(0x400000)), 1, kw.get("Cin", 192),
                                               kw.get("Cout", 256), kw.get("Cp", 6), 5, 8, 8, kw.get("k", 3),
                                               kw.get("work", ctypes.c_void_p(0x500000)), kw.get("wsb", both), None)
    assert call(wp=None) == E_NULL
    assert call(y=None) == E_NULL
    assert call(ws=None, wt=None) == E_NULL
    assert call(Cp=0) == E_SHAPE
    assert call(Cp=5000) == E_SHAPE
    assert call(Cin=12) == E_SHAPE
    assert call(Cout=12) == E_SHAPE
    assert call(ws=None) == E_SHAPE           # temporal-only needs Cin == Cout
    assert call(wp=ctypes.c_void_p(0x600001)) == E_ALIGN
    assert call(wsb=both - 1) == E_WORKSPACE


def test_binding_rejects_mismatched_outputs():
    """A caller-provided output must have the shape, dtype and memory layout the kernel
    writes (an NCTHW buffer for an NTHWC result would be filled in the wrong order)."""
    import torch
    import causal_video_tokenizer_amd as cvt
    shape = (1, 6, 3, 4, 8)
    good = torch.empty(shape, dtype=torch.bfloat16, memory_format=torch.channels_last_3d)
    assert cvt._check_out(good, shape, torch.bfloat16, good.device, cvt.CVT_NTHWC) is good
    planar = torch.empty(shape, dtype=torch.bfloat16)
    assert cvt._check_out(planar, shape, torch.bfloat16, planar.device, cvt.CVT_NCTHW) is planar
    with pytest.raises(ValueError, match="channels_last_3d"):
        cvt._check_out(planar, shape, torch.bfloat16, planar.device, cvt.CVT_NTHWC)
    with pytest.raises(ValueError, match="contiguous"):
        cvt._check_out(good, shape, torch.bfloat16, good.device, cvt.CVT_NCTHW)
    with pytest.raises(ValueError, match="dtype"):
        cvt._check_out(good, shape, torch.float32, good.device, cvt.CVT_NTHWC)
    with pytest.raises(ValueError, match="shape"):
        cvt._check_out(good, (1, 6, 3, 4, 4), torch.bfloat16, good.device, cvt.CVT_NTHWC)


def test_attention_validation():
    """cvt_attention3d rejects bad arguments before any launch."""
    def call(**kw):
        return lib.cvt_attention3d(kw.get("q", A), kw.get("k", B_), kw.get("v", C_), kw.get("o", ctypes.c_void_p(0x400000)),
                                   kw.get("B", 1), kw.get("C", 256), kw.get("T", 16), kw.get("H", 9), kw.get("W", 10),
                                   kw.get("heads", 4), kw.get("axis", 0), None)
    assert call(q=None) == E_NULL
    assert call(o=None) == E_NULL
    assert call(axis=2) == E_LAYOUT
    assert call(heads=3) == E_SHAPE           # does not divide 256
    assert call(heads=64) == E_SHAPE          # head dim 4: not a multiple of 8
    assert call(C=512, heads=1) == E_SHAPE    # head dim 512 above 256
    assert call(C=260, heads=4) == E_SHAPE    # C not a multiple of 8
    assert call(H=0) == E_SHAPE
    assert call(H=4096, W=1024) == E_SHAPE    # a frame of 2^30 elements
    assert call(q=MIS) == E_ALIGN
    assert call(o=ctypes.c_void_p(0x400008)) == E_ALIGN
    assert b"head dim" in (call(heads=64) and lib.cvt_last_error())


def test_temporal_stream_validation():
    ws = lib.cvt_causal_conv3d_temporal_stream_workspace(256, 6)
    assert ws >= 256 * 256 * 3 * 2 and lib.cvt_causal_conv3d_temporal_stream_workspace(256, 0) < ws
    assert lib.cvt_causal_conv3d_temporal_stream_workspace(0, 0) == 0

    def call(**kw):
        return lib.cvt_causal_conv3d_temporal_stream(kw.get("x", A), kw.get("hist", None), kw.get("wt", B_), None,
                                                     kw.get("wp", None), None, kw.get("y", C_), 1, kw.get("C", 256),
                                                     kw.get("Cp", 0), 5, 8, 8, kw.get("work", ctypes.c_void_p(0x500000)),
                                                     kw.get("wsb", ws), None)
    assert call(x=None) == E_NULL
    assert call(wt=None) == E_NULL
    assert call(C=48) == E_SHAPE                                     # below 64 channels
    assert call(C=260) == E_SHAPE                                    # not a multiple of 8
    assert call(wp=ctypes.c_void_p(0x600000), Cp=17) == E_SHAPE     # projection wider than 16
    assert call(wp=ctypes.c_void_p(0x600000), Cp=6, C=512) == E_SHAPE
    assert call(hist=MIS) == E_ALIGN
    assert call(wsb=10) == E_WORKSPACE
    assert call(work=None) == E_WORKSPACE



def test_video_window_geometry_matches_the_oracle():
    from oracle import window as ow
    for T, H, W, win, ta, sa in [(40, 720, 1280, 17, 4, 16), (121, 1080, 1919, 17, 8, 16), (5, 3, 5, 2, 4, 4),
                                 (1, 7, 9, 17, 4, 8), (33, 36, 64, 16, 4, 4)]:
        bounds = ow.window_bounds(T, win)
        got = cvt.video_windows(T, H, W, win, ta, sa)
        assert got == [(t0, nt) + ow.aligned_size(nt, H, W, ta, sa) for t0, nt in bounds]
        assert cvt.video_window(T, H, W, win, ta, sa)[0] == len(bounds)
    n = ctypes.c_int(0)
    assert lib.cvt_video_window(40, 8, 8, 17, 4, 4, 3, ctypes.byref(n), None, None, None, None, None) == E_SHAPE
    assert lib.cvt_video_window(40, 8, 8, 0, 4, 4, 0, None, None, None, None, None, None) == E_SHAPE
    assert lib.cvt_video_window(40, 8, 8, 17, 4, 4, 2, ctypes.byref(n), None, None, None, None, None) == OK
    assert n.value == 3


def test_video_pad_validation():
    def pad(**kw):
        a = dict(x=A, y=B_, dt=1, B=1, C=3, T=40, H=30, W=50, t0=34, nt=6, Tp=9, Hp=32, Wp=56)
        a.update(kw)
        return lib.cvt_video_pad(a["x"], a["y"], a["dt"], a["B"], a["C"], a["T"], a["H"], a["W"], a["t0"], a["nt"],
                                 a["Tp"], a["Hp"], a["Wp"], None)
    assert pad(x=None) == E_NULL
    assert pad(dt=5) == E_DTYPE
    assert pad(nt=7) == E_SHAPE            # past the clip's end
    assert pad(t0=-1) == E_SHAPE
    assert pad(Tp=5) == E_SHAPE            # shorter than the window
    assert pad(Hp=29) == E_SHAPE
    assert pad(Wp=49) == E_SHAPE
    assert pad(Hp=32768, Wp=32768) == E_SHAPE
    assert pad(y=MIS) == E_ALIGN
    assert lib.cvt_video_unpad(A, B_, 1, 1, 3, 40, 30, 50, 34, 7, 9, 32, 56, None) == E_SHAPE
    assert lib.cvt_video_unpad(MIS, B_, 1, 1, 3, 40, 30, 50, 34, 6, 9, 32, 56, None) == E_ALIGN


def test_haar_window_validation():
    # every call below fails validation (no call may pass it: the pointers are not device memory)
    def hw(fn, **kw):
        a = dict(p=A, pdt=1, c=B_, cdt=1, lay=1, B=1, C=3, T=40, H=30, W=50, t0=34, nt=6, Tp=9, Hp=32, Wp=52, tl=2)
        a.update(kw)
        if fn == "fwd":
            return lib.cvt_haar3d_fwd_window(a["p"], a["pdt"], a["c"], a["cdt"], a["lay"], a["B"], a["C"], a["T"],
                                             a["H"], a["W"], a["t0"], a["nt"], a["Tp"], a["Hp"], a["Wp"], a["tl"], None)
        return lib.cvt_haar3d_inv_window(a["c"], a["cdt"], a["lay"], a["p"], a["pdt"], a["B"], a["C"], a["T"],
                                         a["H"], a["W"], a["t0"], a["nt"], a["Tp"], a["Hp"], a["Wp"], a["tl"], None)
    for fn in ("fwd", "inv"):
        assert hw(fn, p=None) == E_NULL
        assert hw(fn, c=None) == E_NULL
        assert hw(fn, pdt=7) == E_DTYPE
        assert hw(fn, cdt=7) == E_DTYPE
        assert hw(fn, lay=9) == E_LAYOUT
        assert hw(fn, tl=3, Tp=8) == E_SHAPE      # a window is not a continuation chunk
        assert hw(fn, Tp=8) == E_SHAPE            # not 1 + 4k
        assert hw(fn, Hp=30) == E_SHAPE           # padded height not a multiple of 4
        assert hw(fn, Wp=48) == E_SHAPE           # below the clip's width
        assert hw(fn, nt=7) == E_SHAPE            # past the clip's end
        assert hw(fn, t0=-1) == E_SHAPE
        assert hw(fn, Tp=5, nt=6) == E_SHAPE      # shorter than the window
        assert hw(fn, tl=0, Tp=5) == E_SHAPE
        assert hw(fn, p=MIS) == E_ALIGN
        assert hw(fn, c=MIS) == E_ALIGN


def test_block_validation():
    F = ctypes.c_void_p(0x700000)
    assert lib.cvt_layernorm3d(None, F, F, B_, 1, 256, 2, 4, 4, 1e-6, 1, None) == E_NULL
    assert lib.cvt_layernorm3d(A, F, F, B_, 1, 252, 2, 4, 4, 1e-6, 1, None) == E_SHAPE
    assert lib.cvt_layernorm3d(A, ctypes.c_void_p(0x700004), F, B_, 1, 256, 2, 4, 4, 1e-6, 1, None) == E_ALIGN

    w = cvt.ResblockWeights(*([0x700000] * 12))
    need = lib.cvt_resblock3d_workspace(1, 256, 5, 8, 8)
    assert need >= 2 * 256 * 256 * 12 * 2
    wk = ctypes.c_void_p(0x800000)

    def rb(**kw):
        return lib.cvt_resblock3d(kw.get("x", A), ctypes.byref(kw.get("w", w)), B_, 1, kw.get("C", 256), 5, 8, 8,
                                  1e-6, kw.get("work", wk), kw.get("wsb", need), None)
    bad = cvt.ResblockWeights(*([0x700000] * 12))
    bad.c2_t = None
    assert rb(w=bad) == E_NULL
    assert rb(C=48) == E_SHAPE
    assert rb(C=260) == E_SHAPE
    assert rb(wsb=need - 1) == E_WORKSPACE
    assert rb(x=MIS) == E_ALIGN
    odd = cvt.ResblockWeights(*([0x700000] * 12))
    odd.ln2_b = 0x700004
    assert rb(w=odd) == E_ALIGN

    # the packed-weight block: only the two intermediates in its workspace, 16-byte aligned packed weights
    need_p = lib.cvt_resblock3d_packed_workspace(1, 256, 5, 8, 8)
    assert need_p == 2 * 5 * 8 * 8 * 256 * 2 and need - need_p >= 2 * 256 * 256 * 12 * 2
    assert lib.cvt_resblock3d_packed_workspace(1, 256, 0, 8, 8) == 0

    def rbp(**kw):
        return lib.cvt_resblock3d_packed(kw.get("x", A), ctypes.byref(kw.get("w", w)), B_, 1, kw.get("C", 256), 5, 8,
                                         8, 1e-6, kw.get("work", wk), kw.get("wsb", need_p), None)
    assert rbp(w=bad) == E_NULL
    assert rbp(C=48) == E_SHAPE
    assert rbp(wsb=need_p - 1) == E_WORKSPACE
    assert rbp(x=MIS) == E_ALIGN
    odd_w = cvt.ResblockWeights(*([0x700000] * 12))
    odd_w.c1_t = 0x700008                      # 2-byte aligned (enough unpacked), not 16-byte
    assert rbp(w=odd_w) == E_ALIGN

    def ds(**kw):
        return lib.cvt_downsample3d(A, kw.get("ws", C_), kw.get("wt", C_), None, None, B_, 1, kw.get("Cin", 64), 64,
                                    kw.get("T", 5), kw.get("H", 8), 8, wk, kw.get("wsb", 1 << 30), None)
    assert ds(ws=None, wt=None) == E_NULL
    assert ds(T=4) == E_SHAPE                # not 1 + 2k
    assert ds(H=7) == E_SHAPE                # odd height with the spatial part
    assert ds(Cin=60) == E_SHAPE
    assert ds(wsb=10) == E_WORKSPACE
    assert lib.cvt_downsample3d_workspace(1, 64, 64, 5, 8, 8, 0) == 0

    def us(**kw):
        return lib.cvt_upsample3d(A, kw.get("ws", C_), C_, None, None, B_, 1, 64, kw.get("Cout", 64), 3, 4, 4, 1, 1,
                                  wk, kw.get("wsb", 1 << 30), None)
    assert us(ws=None) == E_NULL
    assert us(Cout=32) == E_SHAPE
    assert us(wsb=10) == E_WORKSPACE
    assert lib.cvt_upsample3d_workspace(1, 64, 128, 3, 4, 4, 1, 1) > lib.cvt_upsample3d_workspace(1, 64, 128, 3, 4,
                                                                                                   4, 0, 1)

    # the packed-weight blocks: only the intermediates in their workspaces, 16-byte aligned packed weights, and
    # (downsampling) every part on the row-tiled kernels
    P16, P8 = ctypes.c_void_p(0x300000), ctypes.c_void_p(0x300008)
    assert lib.cvt_downsample3d_packed_workspace(1, 64, 64, 5, 8, 8, 3) == 5 * 4 * 4 * 64 * 2   # the 5 x 4 x 4 intermediate
    assert lib.cvt_downsample3d_packed_workspace(1, 64, 64, 5, 8, 8, 1) == 0
    assert lib.cvt_downsample3d_packed_workspace(1, 64, 64, 5, 8, 8, 2) == 0

    def dsp(**kw):
        return lib.cvt_downsample3d_packed(A, kw.get("ws", P16), kw.get("wt", P16), None, None, B_, 1,
                                           kw.get("Cin", 64), kw.get("Cout", 64), kw.get("T", 5), 8, 8, wk,
                                           kw.get("wsb", 10), None)
    assert dsp(ws=None, wt=None) == E_NULL
    assert dsp(T=4) == E_SHAPE
    assert dsp(Cout=32) == E_SHAPE                    # below the row kernels' 64 output channels
    assert dsp(ws=None, Cin=128) == E_SHAPE           # temporal part alone with Cin != Cout
    assert dsp(wt=P8) == E_ALIGN
    assert dsp() == E_WORKSPACE                       # two parts: the intermediate

    need_up = lib.cvt_upsample3d_packed_workspace(1, 64, 64, 3, 4, 4, 1, 1)
    assert need_up == 3 * 8 * 8 * 64 * 2 and lib.cvt_upsample3d_workspace(1, 64, 64, 3, 4, 4, 1, 1) > need_up

    def usp(**kw):
        return lib.cvt_upsample3d_packed(A, kw.get("ws", P16), P16, None, None, B_, 1, 64, kw.get("Cout", 64), 3, 4,
                                         4, 1, 1, wk, kw.get("wsb", need_up - 1), None)
    assert usp(ws=None) == E_NULL
    assert usp(Cout=32) == E_SHAPE
    assert usp(ws=P8) == E_ALIGN
    assert usp() == E_WORKSPACE


def test_fused_fsq_validation():
    lv = (ctypes.c_int32 * 6)(8, 8, 8, 5, 5, 5)
    bad_lv = (ctypes.c_int32 * 6)(8, 8, 8, 5, 5, 1)
    need = lib.cvt_causal_conv3d_fact_proj_fsq_workspace(1, 192, 256, 6, 5, 8, 8, 3, 3)
    assert need > lib.cvt_causal_conv3d_fact_proj_workspace(1, 192, 256, 6, 5, 8, 8, 3, 3)
    wk = ctypes.c_void_p(0x800000)

    def call(**kw):
        return lib.cvt_causal_conv3d_fact_proj_fsq(A, B_, C_, None, None, kw.get("wp", ctypes.c_void_p(0x600000)),
                                                   None, kw.get("lv", lv), 6, None, kw.get("idx", C_), 1,
                                                   kw.get("Cin", 192), 256, 5, 8, 8, 3, wk, kw.get("wsb", need), None)
    assert call(wp=None) == E_NULL
    assert call(idx=None) == E_NULL
    assert call(lv=bad_lv) == E_LEVELS
    assert call(Cin=190) == E_SHAPE
    assert call(idx=MIS) == E_ALIGN
    assert call(wsb=need - 1) == E_WORKSPACE

    def dq(**kw):
        return lib.cvt_fsq_dequantize_proj(kw.get("idx", A), kw.get("lv", lv), 6, kw.get("wp", B_), None,
                                           kw.get("y", C_), 1, kw.get("Cout", 192), 5, 8, 8, None, None)
    assert dq(idx=None) == E_NULL
    assert dq(wp=None) == E_NULL
    assert dq(lv=bad_lv) == E_LEVELS
    assert dq(Cout=0) == E_SHAPE
    assert dq(y=MIS) == E_ALIGN


def test_conv_bindings_reject_non_bf16_inputs():
    """The ABI receives no dtype for x, and its kernels size their buffer resources at 2
    bytes per element, so the bindings must refuse any other dtype (or layout) before a
    launch: float32 would be read as garbage, a 1-byte dtype past its allocation."""
    import torch

    cl = torch.channels_last_3d
    w_s = torch.zeros((64, 64, 1, 3, 3), dtype=torch.bfloat16)
    w_t = torch.zeros((64, 64, 3, 1, 1), dtype=torch.bfloat16)
    w_p = torch.zeros((6, 64, 1, 1, 1), dtype=torch.bfloat16)
    for dt in (torch.float32, torch.uint8, torch.int8, torch.bool, torch.float16):
        x = torch.zeros((1, 64, 5, 8, 8), dtype=dt).to(memory_format=cl)
        calls = [
            lambda: cvt.causal_conv3d_fact(x, w_s, w_t),
            lambda: cvt.causal_conv3d_fact_proj(x, None, w_t, w_p),
            lambda: cvt.causal_conv3d_fact_proj_fsq(x, w_s, w_t, w_p),
            lambda: cvt.causal_conv3d_temporal_stream(x, w_t),
            lambda: cvt.resblock3d(x, {}),
            lambda: cvt.downsample3d(x, w_s, w_t),
            lambda: cvt.upsample3d(x, w_s, w_t),
        ]
        for fn in calls:
            with pytest.raises(ValueError, match="bfloat16"):
                fn()
    # bf16 in the wrong memory layout is refused as well
    x = torch.zeros((1, 64, 5, 8, 8), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="channels_last_3d"):
        cvt.causal_conv3d_fact(x, w_s, w_t)
    with pytest.raises(ValueError, match="channels_last_3d"):
        cvt.causal_conv3d_fact_proj(x, None, w_t, w_p)


def test_conv_noalloc_validation():
    """The no-alloc conv validates like cvt_causal_conv3d_fact and refuses, before touching
    any device, a call whose packed weights and intermediate exceed the preallocated
    scratch."""
    def call(**kw):
        return lib.cvt_causal_conv3d_fact_noalloc(kw.get("x", A), kw.get("ws", B_), kw.get("wt", C_), None, None,
                                                  kw.get("y", ctypes.c_void_p(0x400000)), 1, kw.get("Cin", 256),
                                                  kw.get("Cout", 256), kw.get("T", 10), kw.get("H", 100), 160, 3,
                                                  None)
    assert call(x=None) == E_NULL
    assert call(ws=None, wt=None) == E_NULL
    assert call(Cin=12) == E_SHAPE
    assert call(x=MIS) == E_ALIGN
    assert call() == E_WORKSPACE                      # 160,000 positions x 256 channels of intermediate
    assert b"preallocated scratch" in lib.cvt_last_error()
    assert lib.cvt_causal_conv3d_fact_workspace(1, 256, 256, 10, 100, 160, 3, 3) > cvt.NOALLOC_SCRATCH_BYTES
    assert cvt.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_conv_packed_validation_and_workspace():
    """Packing and the packed-weight convs: sizes of the packed form, workspace queries (only
    the bf16 intermediate), and every argument check before any launch."""
    assert lib.cvt_conv_weights_packed_bytes(256, 192, 9) == 12 * 9 * 8 * 1024  # Cin/16 x taps x Cout/32 fragments
    assert lib.cvt_conv_weights_packed_bytes(256, 256, 3) == 48 * 8 * 1024
    assert lib.cvt_conv_weights_packed_bytes(6, 256, 1) == 16 * 1024             # rows past Cp padded to 32
    assert lib.cvt_conv_weights_packed_bytes(256, 256, 2) == 0
    assert lib.cvt_conv_weights_packed_bytes(0, 256, 3) == 0
    assert lib.cvt_conv_weights_pack(None, B_, 256, 256, 3, None) == E_NULL
    assert lib.cvt_conv_weights_pack(A, None, 256, 256, 3, None) == E_NULL
    assert lib.cvt_conv_weights_pack(A, B_, 256, 256, 5, None) == E_SHAPE
    assert lib.cvt_conv_weights_pack(A, B_, 5000, 256, 3, None) == E_SHAPE
    assert lib.cvt_conv_weights_pack(ctypes.c_void_p(0x100001), B_, 256, 256, 3, None) == E_ALIGN
    assert lib.cvt_conv_weights_pack(A, MIS, 256, 256, 3, None) == E_ALIGN

    P = 5 * 8 * 8
    assert lib.cvt_causal_conv3d_fact_packed_workspace(1, 256, 5, 8, 8, 3) == P * 256 * 2
    assert lib.cvt_causal_conv3d_fact_packed_workspace(1, 256, 5, 8, 8, 1) == 0
    assert lib.cvt_causal_conv3d_fact_packed_workspace(1, 256, 5, 8, 8, 2) == 0
    assert lib.cvt_causal_conv3d_fact_packed_workspace(1, 256, 5, 8, 8, 0) == 0
    assert lib.cvt_causal_conv3d_fact_proj_packed_workspace(1, 256, 5, 8, 8, 3) == P * 256 * 2
    assert lib.cvt_causal_conv3d_fact_proj_packed_workspace(1, 256, 5, 8, 8, 2) == 0
    assert lib.cvt_causal_conv3d_fact_proj_packed_workspace(1, 256, 5, 8, 8, 1) == 0  # the temporal part is required

    W8 = ctypes.c_void_p(0x500000)

    def call(**kw):
        return lib.cvt_causal_conv3d_fact_packed(kw.get("x", A), kw.get("ws", B_), kw.get("wt", C_), None, None,
                                                 kw.get("y", ctypes.c_void_p(0x400000)), 1, kw.get("Cin", 192),
                                                 kw.get("Cout", 256), 5, 8, kw.get("W", 8), kw.get("work", W8),
                                                 kw.get("wsb", P * 256 * 2), None)
    assert call(x=None) == E_NULL
    assert call(ws=None, wt=None) == E_NULL
    assert call(ws=None) == E_SHAPE           # temporal-only needs Cin == Cout
    assert call(Cin=12) == E_SHAPE
    assert call(Cout=12) == E_SHAPE
    assert call(Cout=32) == E_SHAPE           # the row-tiled kernels need Cout >= 64
    assert b"row-tiled" in lib.cvt_last_error()
    assert call(Cout=5000) == E_SHAPE
    assert call(x=MIS) == E_ALIGN
    assert call(ws=MIS) == E_ALIGN
    assert call(wsb=P * 256 * 2 - 1) == E_WORKSPACE
    assert call(work=None) == E_WORKSPACE
    assert call(wt=None, work=None, wsb=0, W=1 << 23) == E_SHAPE   # 10 image rows of 2^23 x 192 x 2 bytes > 2 GiB

    def pcall(**kw):
        return lib.cvt_causal_conv3d_fact_proj_packed(kw.get("x", A), kw.get("ws", B_), kw.get("wt", C_), None, None,
                                                      kw.get("wp", ctypes.c_void_p(0x600000)), None,
                                                      kw.get("y", ctypes.c_void_p(0x400000)), 1, kw.get("Cin", 192),
                                                      kw.get("Cout", 256), kw.get("Cp", 6), 5, 8, 8,
                                                      kw.get("work", W8), kw.get("wsb", P * 256 * 2), None)
    assert pcall(wt=None) == E_NULL
    assert pcall(wp=None) == E_NULL
    assert pcall(y=None) == E_NULL
    assert pcall(Cp=0) == E_SHAPE
    assert pcall(Cp=17) == E_SHAPE
    assert pcall(Cout=320, Cin=320) == E_SHAPE   # the fused projection needs Cout <= 256
    assert pcall(ws=None) == E_SHAPE             # temporal-only needs Cin == Cout
    assert pcall(wp=ctypes.c_void_p(0x600008)) == E_ALIGN
    assert pcall(wsb=P * 256 * 2 - 1) == E_WORKSPACE
