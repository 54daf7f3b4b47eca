"""Causal video tokenizer hot path on AMD MI355X: Python binding of libcvt.

The work is done by the HIP kernels in ``libcvt.so`` behind the C ABI declared
in ``include/cvt.h``.  This module only marshals arguments: it allocates
outputs with torch on the input's device, passes raw device pointers, sizes and
torch's current HIP stream, and raises ``CvtError`` on a non-OK status.  There
is no fallback: if the library is missing, importing this module fails.

Tensor conventions
------------------
* Pixel videos are [B, C, T, H, W] contiguous (NCTHW), float32 or bfloat16.
* Latents / Haar coefficients default to NTHWC, exposed as torch tensors of
  logical shape [B, C, T, H, W] in ``torch.channels_last_3d`` memory format.
* FSQ indices are int32 [B, T, H, W].

Entry points (same names as the C functions without the ``cvt_`` prefix):
``haar3d_fwd``, ``haar3d_inv``, ``causal_conv3d_fact``,
``causal_conv3d_fact_noalloc``, ``causal_conv3d_fact_proj``, ``conv_weights_pack``,
``causal_conv3d_fact_packed``, ``causal_conv3d_fact_proj_packed``, ``causal_conv3d_temporal_stream``, ``attention3d``,
``fsq_quantize``, ``fsq_dequantize``, ``video_window``, ``video_pad``,
``video_unpad``, ``layernorm3d``, ``resblock3d``, ``downsample3d``, ``upsample3d``.  ``lib`` is the loaded ctypes library with the raw C
functions.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcvt.so")

CVT_F32, CVT_BF16 = 0, 1
CVT_NCTHW, CVT_NTHWC = 0, 1
DEFAULT_LEVELS = (8, 8, 8, 5, 5, 5)

# Every symbol include/cvt.h declares, with its ctypes signature.
_vp, _ci, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_pi = ctypes.POINTER(_ci)
SIGNATURES = {
    "cvt_abi_version": (_ci, []),
    "cvt_status_string": (ctypes.c_char_p, [_ci]),
    "cvt_last_error": (ctypes.c_char_p, []),
    "cvt_haar3d_fwd": (_ci, [_vp, _ci, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _vp]),
    "cvt_haar3d_inv": (_ci, [_vp, _ci, _ci, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _vp]),
    "cvt_causal_conv3d_fact_workspace": (_sz, [_ci, _ci, _ci, _ci, _ci, _ci, _ci, _ci]),
    "cvt_causal_conv3d_fact": (_ci, [_vp, _vp, _vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _vp, _sz, _vp]),
    "cvt_causal_conv3d_fact_noalloc": (_ci, [_vp, _vp, _vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _vp]),
    "cvt_conv_weights_packed_bytes": (_sz, [_ci, _ci, _ci]),
    "cvt_conv_weights_pack": (_ci, [_vp, _vp, _ci, _ci, _ci, _vp]),
    "cvt_causal_conv3d_fact_packed_workspace": (_sz, [_ci] * 6),
    "cvt_causal_conv3d_fact_packed": (_ci, [_vp] * 6 + [_ci] * 6 + [_vp, _sz, _vp]),
    "cvt_causal_conv3d_fact_proj_packed_workspace": (_sz, [_ci] * 6),
    "cvt_causal_conv3d_fact_proj_packed": (_ci, [_vp] * 8 + [_ci] * 7 + [_vp, _sz, _vp]),
    "cvt_causal_conv3d_fact_proj_workspace": (_sz, [_ci, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _ci]),
    "cvt_causal_conv3d_fact_proj": (_ci, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _ci,
                                          _ci, _vp, _sz, _vp]),
    "cvt_causal_conv3d_temporal_stream_workspace": (_sz, [_ci, _ci]),
    "cvt_causal_conv3d_temporal_stream": (_ci, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci,
                                                _vp, _sz, _vp]),
    "cvt_attention3d": (_ci, [_vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _ci, _vp]),
    "cvt_fsq_quantize": (_ci, [_vp, _ci, _ci, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _vp]),
    "cvt_fsq_dequantize": (_ci, [_vp, _vp, _ci, _ci, _vp, _ci, _ci, _ci, _ci, _ci, _vp, _vp]),
    "cvt_video_window": (_ci, [_ci] * 7 + [_pi] * 6),
    "cvt_video_pad": (_ci, [_vp, _vp] + [_ci] * 11 + [_vp]),
    "cvt_video_unpad": (_ci, [_vp, _vp] + [_ci] * 11 + [_vp]),
    "cvt_haar3d_fwd_window": (_ci, [_vp, _ci, _vp, _ci, _ci] + [_ci] * 11 + [_vp]),
    "cvt_haar3d_inv_window": (_ci, [_vp, _ci, _ci, _vp, _ci] + [_ci] * 11 + [_vp]),
    "cvt_causal_conv3d_fact_proj_fsq_workspace": (_sz, [_ci] * 9),
    "cvt_causal_conv3d_fact_proj_fsq": (_ci, [_vp] * 7 + [_vp, _ci, _vp, _vp] + [_ci] * 7 + [_vp, _sz, _vp]),
    "cvt_fsq_dequantize_proj": (_ci, [_vp, _vp, _ci, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _vp, _vp]),
    "cvt_haar3d_conv3d_fact_workspace": (_sz, [_ci] * 6),
    "cvt_haar3d_conv3d_fact": (_ci, [_vp] * 6 + [_ci] * 5 + [_vp, _sz, _vp]),
    "cvt_fsq_dequantize_conv3d_fact_workspace": (_sz, [_ci] * 7),
    "cvt_fsq_dequantize_conv3d_fact": (_ci, [_vp, _vp, _ci] + [_vp] * 7 + [_ci] * 6 + [_vp, _sz, _vp]),
    "cvt_layernorm3d": (_ci, [_vp, _vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, ctypes.c_float, _ci, _vp]),
    "cvt_resblock3d_workspace": (_sz, [_ci] * 5),
    "cvt_resblock3d": (_ci, [_vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, ctypes.c_float, _vp, _sz, _vp]),
    "cvt_resblock3d_packed_workspace": (_sz, [_ci] * 5),
    "cvt_resblock3d_packed": (_ci, [_vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, ctypes.c_float, _vp, _sz, _vp]),
    "cvt_downsample3d_workspace": (_sz, [_ci] * 7),
    "cvt_downsample3d": (_ci, [_vp] * 6 + [_ci] * 6 + [_vp, _sz, _vp]),
    "cvt_upsample3d_workspace": (_sz, [_ci] * 8),
    "cvt_upsample3d": (_ci, [_vp] * 6 + [_ci] * 8 + [_vp, _sz, _vp]),
    "cvt_downsample3d_packed_workspace": (_sz, [_ci] * 7),
    "cvt_downsample3d_packed": (_ci, [_vp] * 6 + [_ci] * 6 + [_vp, _sz, _vp]),
    "cvt_upsample3d_packed_workspace": (_sz, [_ci] * 8),
    "cvt_upsample3d_packed": (_ci, [_vp] * 6 + [_ci] * 8 + [_vp, _sz, _vp]),
}


class ResblockWeights(ctypes.Structure):
    """cvt_resblock_weights: device pointers of one residual block's parameters."""
    _fields_ = [(n, ctypes.c_void_p) for n in ("ln1_g", "ln1_b", "c1_s", "c1_t", "c1_bs", "c1_bt",
                                               "ln2_g", "ln2_b", "c2_s", "c2_t", "c2_bs", "c2_bt")]


class CvtError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        detail = lib.cvt_last_error().decode(errors="replace")
        super().__init__(f"{where}: {lib.cvt_status_string(status).decode()} ({detail})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python causal_video_tokenizer_amd/build.py` "
            "(hipcc for gfx950); there is no fallback implementation")
    handle = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


lib = _load()


def _check(status, where):
    if status != 0:
        raise CvtError(status, where)


def _dtype_code(t):
    if t == torch.float32:
        return CVT_F32
    if t == torch.bfloat16:
        return CVT_BF16
    raise TypeError(f"unsupported dtype {t}; use float32 or bfloat16")


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _require_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on a ROCm GPU device")


def _same_device(x, *ts):
    """Every tensor given (weights, biases, workspace) lives on x's device: the kernels
    dereference their pointers on that device."""
    for t in ts:
        if t is not None and t.device != x.device:
            raise ValueError(f"a tensor is on {t.device}, expected {x.device} (the device of x)")


def _workspace_arg(workspace, need, x):
    """The caller's workspace (uint8, contiguous, on x's device) or a new one of `need` bytes."""
    if workspace is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    return workspace


def _layout_of(t):
    """Physical layout code of a 5-D tensor (NCTHW contiguous or NTHWC)."""
    if t.is_contiguous():
        return CVT_NCTHW
    if t.is_contiguous(memory_format=torch.channels_last_3d):
        return CVT_NTHWC
    raise ValueError("5-D tensors must be contiguous (NCTHW) or channels_last_3d (NTHWC)")


def _check_out(t, shape, dtype, device, layout=None, what="out"):
    """A caller-provided output must match what the kernel writes: logical shape, dtype,
    device and memory layout (NTHWC = channels_last_3d, else C-contiguous)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{what} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{what} is on {t.device}, expected {device}")
    fmt = torch.channels_last_3d if layout == CVT_NTHWC else torch.contiguous_format
    if not t.is_contiguous(memory_format=fmt):
        raise ValueError(f"{what} must be {'channels_last_3d (NTHWC)' if layout == CVT_NTHWC else 'contiguous'}")
    return t


def _empty5(shape, dtype, device, layout):
    mf = torch.channels_last_3d if layout == CVT_NTHWC else torch.contiguous_format
    return torch.empty(shape, dtype=dtype, device=device, memory_format=mf)


def haar3d_fwd(x, temporal_levels=2, out_dtype=None, layout="NTHWC", out=None):
    """Forward Haar patcher: x [B, C, T, H, W] NCTHW -> [B, 64C, T', H/4, W/4]
    (16C and T with temporal_levels=0; T' = T/4 for a continuation chunk,
    temporal_levels=3) in ``layout``."""
    _require_gpu(x)
    if not x.is_contiguous():
        raise ValueError("x must be NCTHW-contiguous")
    B, C, T, H, W = x.shape
    lay = CVT_NTHWC if layout == "NTHWC" else CVT_NCTHW
    odt = out_dtype or (out.dtype if out is not None else x.dtype)
    if temporal_levels == 2:
        shape = (B, 64 * C, 1 + max(T - 1, 0) // 4, H // 4, W // 4)
    elif temporal_levels == 3:  # continuation chunk of 4k frames
        shape = (B, 64 * C, T // 4, H // 4, W // 4)
    else:
        shape = (B, 16 * C, T, H // 4, W // 4)
    y = _check_out(out, shape, odt, x.device, lay) if out is not None else _empty5(shape, odt, x.device, lay)
    _check(lib.cvt_haar3d_fwd(_ptr(x), _dtype_code(x.dtype), _ptr(y), _dtype_code(y.dtype), lay,
                              B, C, T, H, W, temporal_levels, _stream(x.device)), "haar3d_fwd")
    return y


def haar3d_inv(y, temporal_levels=2, out_dtype=None, out=None):
    """Inverse Haar patcher: coefficients [B, 64C, T', H', W'] (either layout)
    -> pixels [B, C, 4T'-3, 4H', 4W'] NCTHW (T' frames with temporal_levels=0)."""
    _require_gpu(y)
    lay = _layout_of(y)
    B, NCH, Tq, Hq, Wq = y.shape
    G = 64 if temporal_levels in (2, 3) else 16
    if NCH % G:
        raise ValueError(f"coefficient channels must be a multiple of {G}")
    C = NCH // G
    T = {2: 4 * Tq - 3, 3: 4 * Tq}.get(temporal_levels, Tq)
    odt = out_dtype or (out.dtype if out is not None else y.dtype)
    shape = (B, C, T, 4 * Hq, 4 * Wq)
    x = _check_out(out, shape, odt, y.device) if out is not None else torch.empty(shape, dtype=odt, device=y.device)
    _check(lib.cvt_haar3d_inv(_ptr(y), _dtype_code(y.dtype), lay, _ptr(x), _dtype_code(x.dtype),
                              B, C, T, 4 * Hq, 4 * Wq, temporal_levels, _stream(y.device)), "haar3d_inv")
    return x


CVT_CONV_SPATIAL, CVT_CONV_TEMPORAL = 1, 2


def conv_workspace_bytes(x_shape, Cout, k, spatial=True, temporal=True):
    B, Cin, T, H, W = x_shape
    parts = (CVT_CONV_SPATIAL if spatial else 0) | (CVT_CONV_TEMPORAL if temporal else 0)
    return int(lib.cvt_causal_conv3d_fact_workspace(B, Cin, Cout, T, H, W, k, parts))


def causal_conv3d_fact(x, w_s, w_t=None, b_s=None, b_t=None, workspace=None, out=None):
    """Factorized causal convolution on a bf16 NTHWC tensor.

    x: [B, Cin, T, H, W] bf16 channels_last_3d; w_s: [Cout, Cin, 1, k, k] bf16
    or None (temporal part only); w_t: [Cout, Cout, k, 1, 1] bf16 or None
    (spatial part only); b_s, b_t: float32 [Cout] or None.
    Returns y [B, Cout, T, H, W] bf16 channels_last_3d.
    """
    _nthwc_bf16(x, "x")
    _require_gpu(x, w_s, w_t, b_s, b_t, workspace)
    _same_device(x, w_s, w_t, b_s, b_t, workspace)
    B, Cin, T, H, W = x.shape
    if w_s is not None:
        Cout, Cin_w, kt, k, k2 = w_s.shape
        if Cin_w != Cin or kt != 1 or k != k2:
            raise ValueError("w_s must be [Cout, Cin, 1, k, k]")
    elif w_t is not None:
        Cout, k = w_t.shape[0], w_t.shape[2]
    else:
        raise ValueError("at least one of w_s and w_t is needed")
    if w_t is not None and tuple(w_t.shape) != (Cout, Cout, k, 1, 1):
        raise ValueError("w_t must be [Cout, Cout, k, 1, 1]")
    for w in (w_s, w_t):
        if w is not None and (w.dtype != torch.bfloat16 or not w.is_contiguous()):
            raise ValueError("weights must be contiguous bfloat16")
    for b in (b_s, b_t):
        if b is not None and (b.dtype != torch.float32 or not b.is_contiguous() or b.numel() != Cout):
            raise ValueError("biases must be contiguous float32 [Cout]")
    need = conv_workspace_bytes(x.shape, Cout, k, w_s is not None, w_t is not None)
    workspace = _workspace_arg(workspace, need, x)
    shape = (B, Cout, T, H, W)
    y = (_check_out(out, shape, torch.bfloat16, x.device, CVT_NTHWC) if out is not None
         else _empty5(shape, torch.bfloat16, x.device, CVT_NTHWC))
    _check(lib.cvt_causal_conv3d_fact(_ptr(x), _ptr(w_s), _ptr(w_t), _ptr(b_s), _ptr(b_t), _ptr(y),
                                      B, Cin, Cout, T, H, W, k, _ptr(workspace), workspace.numel(),
                                      _stream(x.device)), "causal_conv3d_fact")
    return y


NOALLOC_SCRATCH_BYTES = 64 << 20  # CVT_NOALLOC_SCRATCH_BYTES


def causal_conv3d_fact_noalloc(x, w_s, w_t=None, b_s=None, b_t=None, out=None):
    """causal_conv3d_fact with the library's preallocated scratch in place of a workspace
    (cvt_causal_conv3d_fact_noalloc): nothing is allocated but the output, and nothing at
    all with ``out`` given.  Calls that overlap on one GPU share that scratch and race."""
    _nthwc_bf16(x, "x")
    _require_gpu(x, w_s, w_t, b_s, b_t)
    _same_device(x, w_s, w_t, b_s, b_t)
    B, Cin, T, H, W = x.shape
    w0 = w_s if w_s is not None else w_t
    if w0 is None:
        raise ValueError("at least one of w_s and w_t is needed")
    Cout, k = w0.shape[0], w0.shape[3] if w_s is not None else w0.shape[2]
    if w_s is not None and tuple(w_s.shape) != (Cout, Cin, 1, k, k):
        raise ValueError("w_s must be [Cout, Cin, 1, k, k]")
    if w_t is not None and tuple(w_t.shape) != (Cout, Cout, k, 1, 1):
        raise ValueError("w_t must be [Cout, Cout, k, 1, 1]")
    for w in (w_s, w_t):
        if w is not None and (w.dtype != torch.bfloat16 or not w.is_contiguous()):
            raise ValueError("weights must be contiguous bfloat16")
    for b in (b_s, b_t):
        _f32_vec(b, Cout, "bias")
    shape = (B, Cout, T, H, W)
    y = (_check_out(out, shape, torch.bfloat16, x.device, CVT_NTHWC) if out is not None
         else _empty5(shape, torch.bfloat16, x.device, CVT_NTHWC))
    _check(lib.cvt_causal_conv3d_fact_noalloc(_ptr(x), _ptr(w_s), _ptr(w_t), _ptr(b_s), _ptr(b_t), _ptr(y),
                                              B, Cin, Cout, T, H, W, k, _stream(x.device)),
           "causal_conv3d_fact_noalloc")
    return y


class PackedWeights:
    """Conv weights in the order the row-tiled kernels read them (conv_weights_pack):
    ``data`` is a uint8 device tensor; Cout, Cin and taps (9 spatial 1x3x3, 3 temporal
    3x1x1, 1 projection) record the tensor it was packed from."""

    def __init__(self, data, Cout, Cin, taps):
        self.data, self.Cout, self.Cin, self.taps = data, Cout, Cin, taps


def conv_weights_pack(w):
    """Pack bf16 conv weights [Cout, Cin, kt, kh, kw] (torch order; 1x3x3, 3x1x1 or 1x1x1)
    once, for repeated packed calls (causal_conv3d_fact_packed and
    causal_conv3d_fact_proj_packed) on fixed weights."""
    _require_gpu(w)
    if w.dim() != 5 or w.dtype != torch.bfloat16 or not w.is_contiguous():
        raise ValueError("w must be contiguous bfloat16 [Cout, Cin, kt, kh, kw]")
    Cout, Cin, kt, kh, kw = w.shape
    taps = {(1, 3, 3): 9, (3, 1, 1): 3, (1, 1, 1): 1}.get((kt, kh, kw))
    if taps is None:
        raise ValueError("w must be a 1x3x3, 3x1x1 or 1x1x1 kernel")
    n = int(lib.cvt_conv_weights_packed_bytes(Cout, Cin, taps))
    if n == 0:
        raise ValueError(f"unsupported weight shape {tuple(w.shape)}")
    data = torch.empty(n, dtype=torch.uint8, device=w.device)
    _check(lib.cvt_conv_weights_pack(_ptr(w), _ptr(data), Cout, Cin, taps, _stream(w.device)), "conv_weights_pack")
    return PackedWeights(data, Cout, Cin, taps)


def _packed(pw, taps, what):
    if pw is None:
        return None
    if not isinstance(pw, PackedWeights) or pw.taps != taps:
        raise ValueError(f"{what} must be PackedWeights of a {'1x3x3' if taps == 9 else '3x1x1' if taps == 3 else '1x1x1'}"
                         " kernel (conv_weights_pack)")
    return pw


def conv_packed_workspace_bytes(x_shape, Cout, spatial=True, temporal=True):
    B, _, T, H, W = x_shape
    parts = (CVT_CONV_SPATIAL if spatial else 0) | (CVT_CONV_TEMPORAL if temporal else 0)
    return int(lib.cvt_causal_conv3d_fact_packed_workspace(B, Cout, T, H, W, parts))


def causal_conv3d_fact_packed(x, pw_s, pw_t=None, b_s=None, b_t=None, workspace=None, out=None):
    """causal_conv3d_fact (k = 3) on weights packed once by conv_weights_pack: the same
    kernels and result bit for bit, without the per-call weight repack.  The workspace holds
    only the spatial->temporal intermediate (none for one part)."""
    _nthwc_bf16(x, "x")
    pw_s, pw_t = _packed(pw_s, 9, "pw_s"), _packed(pw_t, 3, "pw_t")
    if pw_s is None and pw_t is None:
        raise ValueError("at least one of pw_s and pw_t is needed")
    B, Cin, T, H, W = x.shape
    Cout = (pw_s or pw_t).Cout
    if pw_s is not None and pw_s.Cin != Cin:
        raise ValueError(f"pw_s was packed for Cin={pw_s.Cin}, x has {Cin} channels")
    if pw_t is not None and (pw_t.Cout != Cout or pw_t.Cin != Cout):
        raise ValueError("pw_t must be packed from [Cout, Cout, 3, 1, 1] weights")
    ds = [t.data if t is not None else None for t in (pw_s, pw_t)]
    _require_gpu(x, *ds, b_s, b_t, workspace)
    _same_device(x, *ds, b_s, b_t, workspace)
    for b in (b_s, b_t):
        _f32_vec(b, Cout, "bias")
    need = conv_packed_workspace_bytes(x.shape, Cout, pw_s is not None, pw_t is not None)
    workspace = _workspace_arg(workspace, need, x) if need else workspace
    shape = (B, Cout, T, H, W)
    y = (_check_out(out, shape, torch.bfloat16, x.device, CVT_NTHWC) if out is not None
         else _empty5(shape, torch.bfloat16, x.device, CVT_NTHWC))
    _check(lib.cvt_causal_conv3d_fact_packed(_ptr(x), _ptr(ds[0]), _ptr(ds[1]), _ptr(b_s), _ptr(b_t), _ptr(y),
                                             B, Cin, Cout, T, H, W, _ptr(workspace),
                                             workspace.numel() if workspace is not None else 0, _stream(x.device)),
           "causal_conv3d_fact_packed")
    return y


def conv_proj_packed_workspace_bytes(x_shape, Cout, spatial=True):
    B, _, T, H, W = x_shape
    parts = CVT_CONV_TEMPORAL | (CVT_CONV_SPATIAL if spatial else 0)
    return int(lib.cvt_causal_conv3d_fact_proj_packed_workspace(B, Cout, T, H, W, parts))


def causal_conv3d_fact_proj_packed(x, pw_s, pw_t, pw_p, b_s=None, b_t=None, b_p=None, workspace=None, out=None):
    """causal_conv3d_fact_proj (k = 3, the projection in the temporal conv's epilogue) on
    weights packed once by conv_weights_pack; bit for bit the unpacked call's result."""
    _nthwc_bf16(x, "x")
    pw_s, pw_t, pw_p = _packed(pw_s, 9, "pw_s"), _packed(pw_t, 3, "pw_t"), _packed(pw_p, 1, "pw_p")
    if pw_t is None or pw_p is None:
        raise ValueError("pw_t and pw_p are needed")
    B, Cin, T, H, W = x.shape
    Cout, Cp = pw_t.Cout, pw_p.Cout
    if pw_t.Cin != Cout or pw_p.Cin != Cout or (pw_s is not None and (pw_s.Cout != Cout or pw_s.Cin != Cin)):
        raise ValueError("packed weights do not chain: pw_s [Cout, Cin], pw_t [Cout, Cout], pw_p [Cp, Cout]")
    ds = [t.data if t is not None else None for t in (pw_s, pw_t, pw_p)]
    _require_gpu(x, *ds, b_s, b_t, b_p, workspace)
    _same_device(x, *ds, b_s, b_t, b_p, workspace)
    for bias, n in ((b_s, Cout), (b_t, Cout), (b_p, Cp)):
        _f32_vec(bias, n, "bias")
    need = conv_proj_packed_workspace_bytes(x.shape, Cout, pw_s is not None)
    workspace = _workspace_arg(workspace, need, x) if need else workspace
    shape = (B, Cp, T, H, W)
    y = (_check_out(out, shape, torch.bfloat16, x.device, CVT_NTHWC) if out is not None
         else _empty5(shape, torch.bfloat16, x.device, CVT_NTHWC))
    _check(lib.cvt_causal_conv3d_fact_proj_packed(_ptr(x), _ptr(ds[0]), _ptr(ds[1]), _ptr(b_s), _ptr(b_t), _ptr(ds[2]),
                                                  _ptr(b_p), _ptr(y), B, Cin, Cout, Cp, T, H, W, _ptr(workspace),
                                                  workspace.numel() if workspace is not None else 0,
                                                  _stream(x.device)), "causal_conv3d_fact_proj_packed")
    return y


def conv_proj_workspace_bytes(x_shape, Cout, Cp, k, spatial=True, temporal=True):
    B, Cin, T, H, W = x_shape
    parts = (CVT_CONV_SPATIAL if spatial else 0) | (CVT_CONV_TEMPORAL if temporal else 0)
    return int(lib.cvt_causal_conv3d_fact_proj_workspace(B, Cin, Cout, Cp, T, H, W, k, parts))


def conv_proj_fsq_workspace_bytes(x_shape, Cout, D, k, spatial=True, temporal=True):
    B, Cin, T, H, W = x_shape
    parts = (CVT_CONV_SPATIAL if spatial else 0) | (CVT_CONV_TEMPORAL if temporal else 0)
    return int(lib.cvt_causal_conv3d_fact_proj_fsq_workspace(B, Cin, Cout, D, T, H, W, k, parts))


def causal_conv3d_fact_proj(x, w_s, w_t, w_p, b_s=None, b_t=None, b_p=None, workspace=None, out=None):
    """Factorized causal convolution followed by a 1x1x1 projection, without
    materialising the Cout-channel result.

    x, w_s, w_t, b_s, b_t: as causal_conv3d_fact; w_p: [Cp, Cout, 1, 1, 1] bf16;
    b_p: float32 [Cp] or None.  Returns [B, Cp, T, H, W] bf16 channels_last_3d.
    """
    _nthwc_bf16(x, "x")
    _require_gpu(x, w_s, w_t, w_p, b_s, b_t, b_p, workspace)
    _same_device(x, w_s, w_t, w_p, b_s, b_t, b_p, workspace)
    B, Cin, T, H, W = x.shape
    if w_s is not None:
        Cout, k = w_s.shape[0], w_s.shape[3]
        if tuple(w_s.shape) != (Cout, Cin, 1, k, k):
            raise ValueError("w_s must be [Cout, Cin, 1, k, k]")
    elif w_t is not None:
        Cout, k = w_t.shape[0], w_t.shape[2]
    else:
        raise ValueError("at least one of w_s and w_t is needed")
    if w_t is not None and tuple(w_t.shape) != (Cout, Cout, k, 1, 1):
        raise ValueError("w_t must be [Cout, Cout, k, 1, 1]")
    Cp = w_p.shape[0]
    if tuple(w_p.shape) != (Cp, Cout, 1, 1, 1):
        raise ValueError("w_p must be [Cp, Cout, 1, 1, 1]")
    for w in (w_s, w_t, w_p):
        if w is not None and (w.dtype != torch.bfloat16 or not w.is_contiguous()):
            raise ValueError("weights must be contiguous bfloat16")
    for bias, n in ((b_s, Cout), (b_t, Cout), (b_p, Cp)):
        if bias is not None and (bias.dtype != torch.float32 or not bias.is_contiguous() or bias.numel() != n):
            raise ValueError("biases must be contiguous float32 of their output width")
    need = conv_proj_workspace_bytes(x.shape, Cout, Cp, k, w_s is not None, w_t is not None)
    workspace = _workspace_arg(workspace, need, x)
    shape = (B, Cp, T, H, W)
    y = (_check_out(out, shape, torch.bfloat16, x.device, CVT_NTHWC) if out is not None
         else _empty5(shape, torch.bfloat16, x.device, CVT_NTHWC))
    _check(lib.cvt_causal_conv3d_fact_proj(_ptr(x), _ptr(w_s), _ptr(w_t), _ptr(b_s), _ptr(b_t), _ptr(w_p), _ptr(b_p),
                                           _ptr(y), B, Cin, Cout, Cp, T, H, W, k, _ptr(workspace), workspace.numel(),
                                           _stream(x.device)), "causal_conv3d_fact_proj")
    return y


def temporal_stream_workspace_bytes(C, Cp=0):
    return int(lib.cvt_causal_conv3d_temporal_stream_workspace(C, Cp))


def causal_conv3d_temporal_stream(x, w_t, hist=None, w_p=None, b_t=None, b_p=None, workspace=None, out=None):
    """Causal temporal convolution (k = 3) of one chunk of a stream, optionally with the
    fused 1x1 projection w_p [Cp, C, 1, 1, 1].  x: [B, C, T, H, W] bf16 channels_last_3d;
    hist: None (start of a stream: zero padding) or the two frames before x,
    [B, C, 2, H, W] bf16 channels_last_3d (for B = 1 a view of the previous chunk's last
    two frames).  Chunk by chunk this equals one call over the whole clip, bit for bit."""
    _nthwc_bf16(x, "x")
    _require_gpu(x, w_t, hist, w_p, b_t, b_p, workspace)
    _same_device(x, w_t, hist, w_p, b_t, b_p, workspace)
    B, C, T, H, W = x.shape
    if hist is not None:
        if (tuple(hist.shape) != (B, C, 2, H, W) or hist.dtype != torch.bfloat16
                or not hist.is_contiguous(memory_format=torch.channels_last_3d)):
            raise ValueError("hist must be bfloat16 channels_last_3d [B, C, 2, H, W]")
    if tuple(w_t.shape) != (C, C, 3, 1, 1) or w_t.dtype != torch.bfloat16 or not w_t.is_contiguous():
        raise ValueError("w_t must be contiguous bfloat16 [C, C, 3, 1, 1]")
    Cp = 0
    if w_p is not None:
        Cp = w_p.shape[0]
        if tuple(w_p.shape) != (Cp, C, 1, 1, 1) or w_p.dtype != torch.bfloat16 or not w_p.is_contiguous():
            raise ValueError("w_p must be contiguous bfloat16 [Cp, C, 1, 1, 1]")
    for bias, n in ((b_t, C), (b_p, Cp)):
        if bias is not None and (bias.dtype != torch.float32 or not bias.is_contiguous() or bias.numel() != n):
            raise ValueError("biases must be contiguous float32 of their output width")
    need = temporal_stream_workspace_bytes(C, Cp)
    workspace = _workspace_arg(workspace, need, x)
    shape = (B, Cp if w_p is not None else C, T, H, W)
    y = (_check_out(out, shape, torch.bfloat16, x.device, CVT_NTHWC) if out is not None
         else _empty5(shape, torch.bfloat16, x.device, CVT_NTHWC))
    _check(lib.cvt_causal_conv3d_temporal_stream(_ptr(x), _ptr(hist), _ptr(w_t), _ptr(b_t), _ptr(w_p), _ptr(b_p),
                                                 _ptr(y), B, C, Cp, T, H, W, _ptr(workspace), workspace.numel(),
                                                 _stream(x.device)), "causal_conv3d_temporal_stream")
    return y


CVT_ATTN_SPATIAL, CVT_ATTN_TEMPORAL_CAUSAL = 0, 1


def attention3d(q, k, v, heads, axis="spatial", out=None):
    """Factorized self-attention core on bf16 NTHWC tensors [B, C, T, H, W]:
    softmax(q k^T / sqrt(d)) v per head of d = C / heads consecutive channels,
    over the H*W positions of each frame (axis="spatial") or, causally, over the
    T frames of each position (axis="temporal").  Returns out (channels_last_3d)."""
    _require_gpu(q, k, v)
    codes = {"spatial": CVT_ATTN_SPATIAL, "temporal": CVT_ATTN_TEMPORAL_CAUSAL}
    if axis not in codes:
        raise ValueError('axis must be "spatial" or "temporal"')
    for t in (q, k, v):
        if t.dtype != torch.bfloat16 or not t.is_contiguous(memory_format=torch.channels_last_3d):
            raise ValueError("q, k and v must be bfloat16 channels_last_3d (NTHWC)")
        if tuple(t.shape) != tuple(q.shape) or t.device != q.device:
            raise ValueError("q, k and v must have one shape and device")
    B, C, T, H, W = q.shape
    o = (_check_out(out, q.shape, torch.bfloat16, q.device, CVT_NTHWC) if out is not None
         else _empty5(q.shape, torch.bfloat16, q.device, CVT_NTHWC))
    _check(lib.cvt_attention3d(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, C, T, H, W, heads, codes[axis],
                               _stream(q.device)), "attention3d")
    return o


def _levels_arg(levels):
    arr = (ctypes.c_int32 * len(levels))(*levels)
    return arr, len(levels)


def fsq_quantize(z, levels=DEFAULT_LEVELS, return_codes=False, indices=None, codes=None):
    """FSQ: z [B, D, T, H, W] (NCTHW or NTHWC, f32/bf16) -> int32 indices [B, T, H, W]
    (and the quantized codes, shaped and laid out like z, when return_codes)."""
    _require_gpu(z)
    lay = _layout_of(z)
    B, D, T, H, W = z.shape
    arr, n = _levels_arg(levels)
    if indices is not None:
        idx = _check_out(indices, (B, T, H, W), torch.int32, z.device, what="indices")
    else:
        idx = torch.empty((B, T, H, W), dtype=torch.int32, device=z.device)
    if return_codes:
        codes = (_check_out(codes, tuple(z.shape), z.dtype, z.device, lay, what="codes") if codes is not None
                 else _empty5(tuple(z.shape), z.dtype, z.device, lay))
    _check(lib.cvt_fsq_quantize(_ptr(z), _dtype_code(z.dtype), lay, _ptr(idx), _ptr(codes) if return_codes else None,
                                arr, n, B, T, H, W, _stream(z.device)), "fsq_quantize")
    return (idx, codes) if return_codes else idx


def fsq_dequantize(indices, levels=DEFAULT_LEVELS, dtype=torch.bfloat16, layout="NTHWC", invalid_count=None,
                   out=None):
    """FSQ dequantize: int32 indices [B, T, H, W] -> codes [B, D, T, H, W] in
    ``layout``.  ``invalid_count``: optional int32 device tensor of one element
    to which the number of out-of-range indices is added."""
    _require_gpu(indices)
    if indices.dtype != torch.int32 or not indices.is_contiguous():
        raise ValueError("indices must be contiguous int32")
    B, T, H, W = indices.shape
    lay = CVT_NTHWC if layout == "NTHWC" else CVT_NCTHW
    arr, n = _levels_arg(levels)
    shape = (B, n, T, H, W)
    codes = (_check_out(out, shape, dtype, indices.device, lay) if out is not None
             else _empty5(shape, dtype, indices.device, lay))
    _check(lib.cvt_fsq_dequantize(_ptr(indices), _ptr(codes), _dtype_code(codes.dtype), lay, arr, n,
                                  B, T, H, W, _ptr(invalid_count), _stream(indices.device)), "fsq_dequantize")
    return codes


def video_window(T, H, W, window=17, t_align=4, s_align=4, index=0):
    """Window ``index`` of a T-frame H x W clip cut into windows of ``window`` frames:
    (n_windows, t0, nt, Tp, Hp, Wp), the padded sizes being the smallest
    1 + k*t_align >= nt and multiples of s_align >= H, W (host arithmetic in the library)."""
    out = [ctypes.c_int(0) for _ in range(6)]
    _check(lib.cvt_video_window(T, H, W, window, t_align, s_align, index, *[ctypes.byref(o) for o in out]),
           "video_window")
    return tuple(o.value for o in out)


def video_windows(T, H, W, window=17, t_align=4, s_align=4):
    """[(t0, nt, Tp, Hp, Wp), ...] for every window of the clip."""
    n = video_window(T, H, W, window, t_align, s_align, 0)[0]
    return [video_window(T, H, W, window, t_align, s_align, i)[1:] for i in range(n)]


def video_pad(x, t0, nt, Tp, Hp, Wp, out=None):
    """Frames t0 .. t0+nt-1 of the clip x [B, C, T, H, W] (contiguous, f32/bf16) padded to
    [B, C, Tp, Hp, Wp]: frames mirrored about the window's last frame, zero rows and
    columns after the content."""
    _require_gpu(x)
    if not x.is_contiguous():
        raise ValueError("x must be contiguous (NCTHW)")
    B, C, T, H, W = x.shape
    shape = (B, C, Tp, Hp, Wp)
    y = (_check_out(out, shape, x.dtype, x.device) if out is not None
         else torch.empty(shape, dtype=x.dtype, device=x.device))
    _check(lib.cvt_video_pad(_ptr(x), _ptr(y), _dtype_code(x.dtype), B, C, T, H, W, t0, nt, Tp, Hp, Wp,
                             _stream(x.device)), "video_pad")
    return y


def video_unpad(y, clip, t0, nt):
    """Crop the padded window y [B, C, Tp, Hp, Wp] to nt frames and the clip's H x W and
    write it at frames t0 .. t0+nt-1 of ``clip`` [B, C, T, H, W] (contiguous, same
    dtype), in place.  Returns clip."""
    _require_gpu(y, clip)
    if not y.is_contiguous() or not clip.is_contiguous():
        raise ValueError("y and clip must be contiguous (NCTHW)")
    if y.dtype != clip.dtype or y.device != clip.device:
        raise ValueError("y and clip must share dtype and device")
    B, C, T, H, W = clip.shape
    By, Cy, Tp, Hp, Wp = y.shape
    if (By, Cy) != (B, C):
        raise ValueError("y and clip must have the same batch and channels")
    _check(lib.cvt_video_unpad(_ptr(y), _ptr(clip), _dtype_code(clip.dtype), B, C, T, H, W, t0, nt, Tp, Hp, Wp,
                               _stream(clip.device)), "video_unpad")
    return clip


def haar3d_fwd_window(x, t0, nt, Tp, Hp, Wp, temporal_levels=2, out_dtype=None, layout="NTHWC", out=None):
    """Forward Haar patcher of window (t0, nt) of the clip x [B, C, T, H, W] (NCTHW) padded to
    Tp x Hp x Wp as video_pad pads it: the coefficients haar3d_fwd(video_pad(x, ...)) gives,
    computed without writing the padded window."""
    _require_gpu(x)
    if not x.is_contiguous():
        raise ValueError("x must be NCTHW-contiguous")
    B, C, T, H, W = x.shape
    lay = CVT_NTHWC if layout == "NTHWC" else CVT_NCTHW
    odt = out_dtype or (out.dtype if out is not None else x.dtype)
    if temporal_levels == 2:
        shape = (B, 64 * C, 1 + max(Tp - 1, 0) // 4, Hp // 4, Wp // 4)
    else:
        shape = (B, 16 * C, Tp, Hp // 4, Wp // 4)
    y = _check_out(out, shape, odt, x.device, lay) if out is not None else _empty5(shape, odt, x.device, lay)
    _check(lib.cvt_haar3d_fwd_window(_ptr(x), _dtype_code(x.dtype), _ptr(y), _dtype_code(y.dtype), lay, B, C, T, H, W,
                                     t0, nt, Tp, Hp, Wp, temporal_levels, _stream(x.device)), "haar3d_fwd_window")
    return y


def haar3d_inv_window(y, clip, t0, nt, temporal_levels=2):
    """Inverse Haar patcher of a padded window's coefficients y (either layout) written
    straight into frames t0 .. t0+nt-1 of ``clip`` [B, C, T, H, W] (NCTHW, in place), cropped
    to the clip's H x W: what video_unpad(haar3d_inv(y), clip, t0, nt) gives.  Returns clip."""
    _require_gpu(y, clip)
    if not clip.is_contiguous():
        raise ValueError("clip must be NCTHW-contiguous")
    lay = _layout_of(y)
    B, NCH, Tq, Hq, Wq = y.shape
    G = 64 if temporal_levels == 2 else 16
    if NCH % G:
        raise ValueError(f"coefficient channels must be a multiple of {G}")
    Bc, C, T, H, W = clip.shape
    if (Bc, C) != (B, NCH // G):
        raise ValueError("y and clip must have the same batch and pixel channels")
    Tp = 4 * Tq - 3 if temporal_levels == 2 else Tq
    _check(lib.cvt_haar3d_inv_window(_ptr(y), _dtype_code(y.dtype), lay, _ptr(clip), _dtype_code(clip.dtype), B, C, T,
                                     H, W, t0, nt, Tp, 4 * Hq, 4 * Wq, temporal_levels, _stream(y.device)),
           "haar3d_inv_window")
    return clip


LN_EPS = 1e-6


def _nthwc_bf16(t, what):
    if t.dtype != torch.bfloat16 or not t.is_contiguous(memory_format=torch.channels_last_3d):
        raise ValueError(f"{what} must be bfloat16 channels_last_3d (NTHWC)")


def _f32_vec(t, n, what):
    if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != n):
        raise ValueError(f"{what} must be contiguous float32 of {n} elements")


def _bf16_w(t, shape, what):
    if t is None or tuple(t.shape) != tuple(shape) or t.dtype != torch.bfloat16 or not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous bfloat16 {list(shape)}")


def layernorm3d(x, gamma, beta, eps=LN_EPS, swish=False, out=None):
    """LayerNorm over the channels of each position of a bf16 NTHWC tensor [B, C, T, H, W],
    per-channel float32 scale and shift, then Swish if ``swish``.  ``out`` may be x."""
    _require_gpu(x, gamma, beta)
    _nthwc_bf16(x, "x")
    B, C, T, H, W = x.shape
    _f32_vec(gamma, C, "gamma")
    _f32_vec(beta, C, "beta")
    y = _check_out(out, x.shape, torch.bfloat16, x.device, CVT_NTHWC) if out is not None else torch.empty_like(x)
    _check(lib.cvt_layernorm3d(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), B, C, T, H, W, eps, int(bool(swish)),
                               _stream(x.device)), "layernorm3d")
    return y


RESBLOCK_KEYS = ("ln1_g", "ln1_b", "c1_s", "c1_t", "c1_bs", "c1_bt", "ln2_g", "ln2_b", "c2_s", "c2_t", "c2_bs",
                 "c2_bt")


def resblock3d(x, p, eps=LN_EPS, workspace=None, out=None):
    """Residual block y = x + conv2(swish(LN2(conv1(swish(LN1(x)))))) on a bf16 NTHWC tensor.
    p: dict with ln1_g, ln1_b, ln2_g, ln2_b (float32 [C]), c1_s, c2_s (bf16 [C, C, 1, 3, 3]),
    c1_t, c2_t (bf16 [C, C, 3, 1, 1]) and optional biases c1_bs, c1_bt, c2_bs, c2_bt."""
    _nthwc_bf16(x, "x")
    _require_gpu(x, workspace, *[p.get(k) for k in RESBLOCK_KEYS])
    _same_device(x, workspace, *[p.get(k) for k in RESBLOCK_KEYS])
    B, C, T, H, W = x.shape
    for k in ("ln1_g", "ln1_b", "ln2_g", "ln2_b"):
        if p.get(k) is None:
            raise ValueError(f"{k} is required")
        _f32_vec(p[k], C, k)
    for k in ("c1_bs", "c1_bt", "c2_bs", "c2_bt"):
        _f32_vec(p.get(k), C, k)
    for c in ("c1", "c2"):
        _bf16_w(p.get(c + "_s"), (C, C, 1, 3, 3), c + "_s")
        _bf16_w(p.get(c + "_t"), (C, C, 3, 1, 1), c + "_t")
    w = ResblockWeights(*[p[k].data_ptr() if p.get(k) is not None else None for k in RESBLOCK_KEYS])
    need = int(lib.cvt_resblock3d_workspace(B, C, T, H, W))
    workspace = _workspace_arg(workspace, need, x)
    y = _check_out(out, x.shape, torch.bfloat16, x.device, CVT_NTHWC) if out is not None else torch.empty_like(x)
    _check(lib.cvt_resblock3d(_ptr(x), ctypes.byref(w), _ptr(y), B, C, T, H, W, eps, _ptr(workspace),
                              workspace.numel(), _stream(x.device)), "resblock3d")
    return y


def resblock3d_packed(x, p, eps=LN_EPS, workspace=None, out=None):
    """resblock3d on conv weights packed once by conv_weights_pack: p as for resblock3d, with
    c1_s, c2_s the PackedWeights of the [C, C, 1, 3, 3] and c1_t, c2_t those of the
    [C, C, 3, 1, 1] weights; bit for bit resblock3d's result, without its four repacks."""
    _nthwc_bf16(x, "x")
    B, C, T, H, W = x.shape
    q = dict(p)
    for k, taps in (("c1_s", 9), ("c1_t", 3), ("c2_s", 9), ("c2_t", 3)):
        pw = _packed(p.get(k), taps, k)
        if pw is None:
            raise ValueError(f"{k} is required")
        if pw.Cout != C or pw.Cin != C:
            raise ValueError(f"{k} was packed for [{pw.Cout}, {pw.Cin}], x has {C} channels")
        q[k] = pw.data
    _require_gpu(x, workspace, *[q.get(k) for k in RESBLOCK_KEYS])
    _same_device(x, workspace, *[q.get(k) for k in RESBLOCK_KEYS])
    for k in ("ln1_g", "ln1_b", "ln2_g", "ln2_b"):
        if q.get(k) is None:
            raise ValueError(f"{k} is required")
        _f32_vec(q[k], C, k)
    for k in ("c1_bs", "c1_bt", "c2_bs", "c2_bt"):
        _f32_vec(q.get(k), C, k)
    w = ResblockWeights(*[q[k].data_ptr() if q.get(k) is not None else None for k in RESBLOCK_KEYS])
    need = int(lib.cvt_resblock3d_packed_workspace(B, C, T, H, W))
    workspace = _workspace_arg(workspace, need, x)
    y = _check_out(out, x.shape, torch.bfloat16, x.device, CVT_NTHWC) if out is not None else torch.empty_like(x)
    _check(lib.cvt_resblock3d_packed(_ptr(x), ctypes.byref(w), _ptr(y), B, C, T, H, W, eps, _ptr(workspace),
                                     workspace.numel(), _stream(x.device)), "resblock3d_packed")
    return y


def downsample3d(x, w_s=None, w_t=None, b_s=None, b_t=None, workspace=None, out=None):
    """Downsampling block on a bf16 NTHWC tensor: 1x3x3 conv at stride 2 in H and W (w_s
    [Cout, Cin, 1, 3, 3]) and/or causal 3x1x1 conv at stride 2 in time (w_t [Cout, C, 3, 1, 1],
    T = 1 + 2k -> 1 + k)."""
    _nthwc_bf16(x, "x")
    _require_gpu(x, w_s, w_t, b_s, b_t, workspace)
    _same_device(x, w_s, w_t, b_s, b_t, workspace)
    B, Cin, T, H, W = x.shape
    if w_s is None and w_t is None:
        raise ValueError("at least one of w_s and w_t is needed")
    Cout = (w_s if w_s is not None else w_t).shape[0]
    if w_s is not None:
        _bf16_w(w_s, (Cout, Cin, 1, 3, 3), "w_s")
    if w_t is not None:
        _bf16_w(w_t, (Cout, Cout if w_s is not None else Cin, 3, 1, 1), "w_t")
    _f32_vec(b_s, Cout, "b_s")
    _f32_vec(b_t, Cout, "b_t")
    parts = (CVT_CONV_SPATIAL if w_s is not None else 0) | (CVT_CONV_TEMPORAL if w_t is not None else 0)
    need = int(lib.cvt_downsample3d_workspace(B, Cin, Cout, T, H, W, parts))
    workspace = _workspace_arg(workspace, need, x)
    shape = (B, Cout, 1 + (T - 1) // 2 if w_t is not None else T, H // 2 if w_s is not None else H,
             W // 2 if w_s is not None else W)
    y = (_check_out(out, shape, torch.bfloat16, x.device, CVT_NTHWC) if out is not None
         else _empty5(shape, torch.bfloat16, x.device, CVT_NTHWC))
    _check(lib.cvt_downsample3d(_ptr(x), _ptr(w_s), _ptr(w_t), _ptr(b_s), _ptr(b_t), _ptr(y), B, Cin, Cout, T, H, W,
                                _ptr(workspace), workspace.numel(), _stream(x.device)), "downsample3d")
    return y


def upsample3d(x, w_s, w_t, b_s=None, b_t=None, space=True, time=True, workspace=None, out=None):
    """Upsampling block on a bf16 NTHWC tensor: nearest-neighbour repetition x2 in H and W
    (space) and/or causal x2 in time (time: T -> 2T - 1), then the factorized conv
    (w_s [Cout, Cin, 1, 3, 3], w_t [Cout, Cout, 3, 1, 1])."""
    _nthwc_bf16(x, "x")
    _require_gpu(x, w_s, w_t, b_s, b_t, workspace)
    _same_device(x, w_s, w_t, b_s, b_t, workspace)
    B, Cin, T, H, W = x.shape
    Cout = w_s.shape[0]
    _bf16_w(w_s, (Cout, Cin, 1, 3, 3), "w_s")
    _bf16_w(w_t, (Cout, Cout, 3, 1, 1), "w_t")
    _f32_vec(b_s, Cout, "b_s")
    _f32_vec(b_t, Cout, "b_t")
    need = int(lib.cvt_upsample3d_workspace(B, Cin, Cout, T, H, W, int(space), int(time)))
    workspace = _workspace_arg(workspace, need, x)
    f = 2 if space else 1
    shape = (B, Cout, 2 * T - 1 if time else T, f * H, f * W)
    y = (_check_out(out, shape, torch.bfloat16, x.device, CVT_NTHWC) if out is not None
         else _empty5(shape, torch.bfloat16, x.device, CVT_NTHWC))
    _check(lib.cvt_upsample3d(_ptr(x), _ptr(w_s), _ptr(w_t), _ptr(b_s), _ptr(b_t), _ptr(y), B, Cin, Cout, T, H, W,
                              int(space), int(time), _ptr(workspace), workspace.numel(), _stream(x.device)),
           "upsample3d")
    return y


def downsample3d_packed(x, pw_s=None, pw_t=None, b_s=None, b_t=None, workspace=None, out=None):
    """downsample3d on weights packed once by conv_weights_pack (pw_s of the [Cout, Cin, 1, 3, 3],
    pw_t of the [Cout, C, 3, 1, 1] weights, either None); bit for bit downsample3d's result."""
    _nthwc_bf16(x, "x")
    pw_s, pw_t = _packed(pw_s, 9, "pw_s"), _packed(pw_t, 3, "pw_t")
    if pw_s is None and pw_t is None:
        raise ValueError("at least one of pw_s and pw_t is needed")
    B, Cin, T, H, W = x.shape
    Cout = (pw_s or pw_t).Cout
    if pw_s is not None and pw_s.Cin != Cin:
        raise ValueError(f"pw_s was packed for Cin={pw_s.Cin}, x has {Cin} channels")
    if pw_t is not None and (pw_t.Cout != Cout or pw_t.Cin != (Cout if pw_s is not None else Cin)):
        raise ValueError("pw_t must be packed from [Cout, Cout (or Cin without pw_s), 3, 1, 1] weights")
    ds = [t.data if t is not None else None for t in (pw_s, pw_t)]
    _require_gpu(x, *ds, b_s, b_t, workspace)
    _same_device(x, *ds, b_s, b_t, workspace)
    _f32_vec(b_s, Cout, "b_s")
    _f32_vec(b_t, Cout, "b_t")
    parts = (CVT_CONV_SPATIAL if pw_s is not None else 0) | (CVT_CONV_TEMPORAL if pw_t is not None else 0)
    need = int(lib.cvt_downsample3d_packed_workspace(B, Cin, Cout, T, H, W, parts))
    workspace = _workspace_arg(workspace, need, x) if need else workspace
    shape = (B, Cout, 1 + (T - 1) // 2 if pw_t is not None else T, H // 2 if pw_s is not None else H,
             W // 2 if pw_s is not None else W)
    y = (_check_out(out, shape, torch.bfloat16, x.device, CVT_NTHWC) if out is not None
         else _empty5(shape, torch.bfloat16, x.device, CVT_NTHWC))
    _check(lib.cvt_downsample3d_packed(_ptr(x), _ptr(ds[0]), _ptr(ds[1]), _ptr(b_s), _ptr(b_t), _ptr(y), B, Cin, Cout,
                                       T, H, W, _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                       _stream(x.device)), "downsample3d_packed")
    return y


def upsample3d_packed(x, pw_s, pw_t, b_s=None, b_t=None, space=True, time=True, workspace=None, out=None):
    """upsample3d on weights packed once by conv_weights_pack (pw_s of the [Cout, Cin, 1, 3, 3],
    pw_t of the [Cout, Cout, 3, 1, 1] weights); bit for bit upsample3d's result."""
    _nthwc_bf16(x, "x")
    pw_s, pw_t = _packed(pw_s, 9, "pw_s"), _packed(pw_t, 3, "pw_t")
    if pw_s is None or pw_t is None:
        raise ValueError("pw_s and pw_t are needed")
    B, Cin, T, H, W = x.shape
    Cout = pw_s.Cout
    if pw_s.Cin != Cin or pw_t.Cout != Cout or pw_t.Cin != Cout:
        raise ValueError("packed weights do not chain: pw_s [Cout, Cin], pw_t [Cout, Cout]")
    ds = [pw_s.data, pw_t.data]
    _require_gpu(x, *ds, b_s, b_t, workspace)
    _same_device(x, *ds, b_s, b_t, workspace)
    _f32_vec(b_s, Cout, "b_s")
    _f32_vec(b_t, Cout, "b_t")
    need = int(lib.cvt_upsample3d_packed_workspace(B, Cin, Cout, T, H, W, int(space), int(time)))
    workspace = _workspace_arg(workspace, need, x)
    f = 2 if space else 1
    shape = (B, Cout, 2 * T - 1 if time else T, f * H, f * W)
    y = (_check_out(out, shape, torch.bfloat16, x.device, CVT_NTHWC) if out is not None
         else _empty5(shape, torch.bfloat16, x.device, CVT_NTHWC))
    _check(lib.cvt_upsample3d_packed(_ptr(x), _ptr(ds[0]), _ptr(ds[1]), _ptr(b_s), _ptr(b_t), _ptr(y), B, Cin, Cout, T,
                                     H, W, int(space), int(time), _ptr(workspace), workspace.numel(),
                                     _stream(x.device)), "upsample3d_packed")
    return y


def causal_conv3d_fact_proj_fsq(x, w_s, w_t, w_p, b_s=None, b_t=None, b_p=None, levels=DEFAULT_LEVELS,
                                return_latent=False, workspace=None, indices=None, latent=None):
    """causal_conv3d_fact_proj to the D = len(levels) latent, then FSQ, in one pass where
    the projection is fused: returns int32 indices [B, T, H, W] (and the bf16 NTHWC latent
    when return_latent).  Bit-identical to fsq_quantize(causal_conv3d_fact_proj(...))."""
    _nthwc_bf16(x, "x")
    _require_gpu(x, w_s, w_t, w_p, b_s, b_t, b_p, workspace, indices, latent)
    _same_device(x, w_s, w_t, w_p, b_s, b_t, b_p, workspace)
    B, Cin, T, H, W = x.shape
    if w_s is not None:
        Cout, k = w_s.shape[0], w_s.shape[3]
        if tuple(w_s.shape) != (Cout, Cin, 1, k, k):
            raise ValueError("w_s must be [Cout, Cin, 1, k, k]")
    elif w_t is not None:
        Cout, k = w_t.shape[0], w_t.shape[2]
    else:
        raise ValueError("at least one of w_s and w_t is needed")
    if w_t is not None and tuple(w_t.shape) != (Cout, Cout, k, 1, 1):
        raise ValueError("w_t must be [Cout, Cout, k, 1, 1]")
    D = len(levels)
    if tuple(w_p.shape) != (D, Cout, 1, 1, 1):
        raise ValueError("w_p must be [len(levels), Cout, 1, 1, 1]")
    for w in (w_s, w_t, w_p):
        if w is not None and (w.dtype != torch.bfloat16 or not w.is_contiguous()):
            raise ValueError("weights must be contiguous bfloat16")
    for bias, n in ((b_s, Cout), (b_t, Cout), (b_p, D)):
        _f32_vec(bias, n, "bias")
    parts = (CVT_CONV_SPATIAL if w_s is not None else 0) | (CVT_CONV_TEMPORAL if w_t is not None else 0)
    need = int(lib.cvt_causal_conv3d_fact_proj_fsq_workspace(B, Cin, Cout, D, T, H, W, k, parts))
    workspace = _workspace_arg(workspace, need, x)
    idx = (_check_out(indices, (B, T, H, W), torch.int32, x.device, what="indices") if indices is not None
           else torch.empty((B, T, H, W), dtype=torch.int32, device=x.device))
    lat = None
    if return_latent or latent is not None:
        lat = (_check_out(latent, (B, D, T, H, W), torch.bfloat16, x.device, CVT_NTHWC, what="latent")
               if latent is not None else _empty5((B, D, T, H, W), torch.bfloat16, x.device, CVT_NTHWC))
    arr, n = _levels_arg(levels)
    _check(lib.cvt_causal_conv3d_fact_proj_fsq(_ptr(x), _ptr(w_s), _ptr(w_t), _ptr(b_s), _ptr(b_t), _ptr(w_p),
                                               _ptr(b_p), arr, n, _ptr(lat), _ptr(idx), B, Cin, Cout, T, H, W, k,
                                               _ptr(workspace), workspace.numel(), _stream(x.device)),
           "causal_conv3d_fact_proj_fsq")
    return (idx, lat) if return_latent else idx


def fsq_dequantize_proj(indices, w_p, b_p=None, levels=DEFAULT_LEVELS, invalid_count=None, out=None):
    """FSQ dequantize + the 1x1 projection D -> Cout in one kernel: int32 indices
    [B, T, H, W] -> bf16 NTHWC [B, Cout, T, H, W] (w_p bf16 [Cout, D, 1, 1, 1])."""
    _require_gpu(indices, w_p, b_p, invalid_count)
    if indices.dtype != torch.int32 or not indices.is_contiguous():
        raise ValueError("indices must be contiguous int32 [B, T, H, W]")
    B, T, H, W = indices.shape
    D = len(levels)
    Cout = w_p.shape[0]
    _bf16_w(w_p, (Cout, D, 1, 1, 1), "w_p")
    _f32_vec(b_p, Cout, "b_p")
    shape = (B, Cout, T, H, W)
    y = (_check_out(out, shape, torch.bfloat16, indices.device, CVT_NTHWC) if out is not None
         else _empty5(shape, torch.bfloat16, indices.device, CVT_NTHWC))
    arr, n = _levels_arg(levels)
    _check(lib.cvt_fsq_dequantize_proj(_ptr(indices), arr, n, _ptr(w_p), _ptr(b_p), _ptr(y), B, Cout, T, H, W,
                                       _ptr(invalid_count), _stream(indices.device)), "fsq_dequantize_proj")
    return y


def haar3d_conv3d_fact_workspace_bytes(x_shape, Cout, temporal=True):
    B, C, T, H, W = x_shape
    parts = CVT_CONV_SPATIAL | (CVT_CONV_TEMPORAL if temporal else 0)
    return int(lib.cvt_haar3d_conv3d_fact_workspace(B, Cout, T, H, W, parts))


def haar3d_conv3d_fact(x, w_s, w_t=None, b_s=None, b_t=None, workspace=None, out=None):
    """causal_conv3d_fact(haar3d_fwd(x), w_s, w_t) for a 3-channel bf16 clip x [B, 3, T, H, W]
    (NCTHW), the Haar coefficients computed inside the spatial conv's loads and never written.
    w_s: bf16 [Cout, 192, 1, 3, 3]; w_t: bf16 [Cout, Cout, 3, 1, 1] or None.  Returns
    [B, Cout, 1 + (T-1)/4, H/4, W/4] bf16 channels_last_3d."""
    if x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise ValueError("x must be a contiguous (NCTHW) bfloat16 clip")
    _require_gpu(x, w_s, w_t, b_s, b_t, workspace)
    _same_device(x, w_s, w_t, b_s, b_t, workspace)
    B, C, T, H, W = x.shape
    if C != 3:
        raise ValueError("the fused Haar conv takes 3-channel clips")
    Cout = w_s.shape[0]
    _bf16_w(w_s, (Cout, 192, 1, 3, 3), "w_s")
    if w_t is not None:
        _bf16_w(w_t, (Cout, Cout, 3, 1, 1), "w_t")
    _f32_vec(b_s, Cout, "b_s")
    _f32_vec(b_t, Cout, "b_t")
    need = haar3d_conv3d_fact_workspace_bytes(x.shape, Cout, w_t is not None)
    workspace = _workspace_arg(workspace, need, x)
    shape = (B, Cout, 1 + max(T - 1, 0) // 4, H // 4, W // 4)
    y = (_check_out(out, shape, torch.bfloat16, x.device, CVT_NTHWC) if out is not None
         else _empty5(shape, torch.bfloat16, x.device, CVT_NTHWC))
    _check(lib.cvt_haar3d_conv3d_fact(_ptr(x), _ptr(w_s), _ptr(w_t), _ptr(b_s), _ptr(b_t), _ptr(y), B, Cout, T, H, W,
                                      _ptr(workspace), workspace.numel(), _stream(x.device)), "haar3d_conv3d_fact")
    return y


def fsq_dequantize_conv3d_fact_workspace_bytes(idx_shape, Cmid, Cout, temporal=True):
    B, T, H, W = idx_shape
    parts = CVT_CONV_SPATIAL | (CVT_CONV_TEMPORAL if temporal else 0)
    return int(lib.cvt_fsq_dequantize_conv3d_fact_workspace(B, Cmid, Cout, T, H, W, parts))


def fsq_dequantize_conv3d_fact(indices, w_lift, w_s, w_t=None, b_lift=None, b_s=None, b_t=None,
                               levels=DEFAULT_LEVELS, workspace=None, out=None):
    """causal_conv3d_fact(fsq_dequantize_proj(indices, w_lift, b_lift), w_s, w_t) with the
    projection computed inside the spatial conv's loads and never written; equal to the
    unfused route bit for bit.  indices: int32 [B, T, H, W]; w_lift: bf16 [Cmid, D, 1, 1, 1];
    w_s: bf16 [Cout, Cmid, 1, 3, 3]; w_t: bf16 [Cout, Cout, 3, 1, 1] or None."""
    if indices.dtype != torch.int32 or not indices.is_contiguous():
        raise ValueError("indices must be contiguous int32 [B, T, H, W]")
    _require_gpu(indices, w_lift, w_s, w_t, b_lift, b_s, b_t, workspace)
    _same_device(indices, w_lift, w_s, w_t, b_lift, b_s, b_t, workspace)
    B, T, H, W = indices.shape
    D = len(levels)
    Cmid, Cout = w_lift.shape[0], w_s.shape[0]
    _bf16_w(w_lift, (Cmid, D, 1, 1, 1), "w_lift")
    _bf16_w(w_s, (Cout, Cmid, 1, 3, 3), "w_s")
    if w_t is not None:
        _bf16_w(w_t, (Cout, Cout, 3, 1, 1), "w_t")
    _f32_vec(b_lift, Cmid, "b_lift")
    _f32_vec(b_s, Cout, "b_s")
    _f32_vec(b_t, Cout, "b_t")
    need = fsq_dequantize_conv3d_fact_workspace_bytes(indices.shape, Cmid, Cout, w_t is not None)
    workspace = _workspace_arg(workspace, need, indices)
    shape = (B, Cout, T, H, W)
    y = (_check_out(out, shape, torch.bfloat16, indices.device, CVT_NTHWC) if out is not None
         else _empty5(shape, torch.bfloat16, indices.device, CVT_NTHWC))
    arr, n = _levels_arg(levels)
    _check(lib.cvt_fsq_dequantize_conv3d_fact(_ptr(indices), arr, n, _ptr(w_lift), _ptr(b_lift), _ptr(w_s), _ptr(w_t),
                                              _ptr(b_s), _ptr(b_t), _ptr(y), B, Cmid, Cout, T, H, W, _ptr(workspace),
                                              workspace.numel(), _stream(indices.device)),
           "fsq_dequantize_conv3d_fact")
    return y
