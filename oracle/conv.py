"""Factorized causal 3D convolution and 1x1 projection (oracle, test infrastructure).

The passage followed: Cosmos-Predict1 summary, section "1) Cosmos Tokenizer":
the encoder uses a space-time factorized 3D convolution, first a 1 x k x k
spatial convolution, then a k x 1 x 1 temporal convolution with left padding
k - 1 so that it is causal.  The model card ("Model Architecture") and the
Cosmos Tokenizer guide (section 7.3) add that the temporal convolution is
causal: an output frame depends only on the same and earlier frames.

Readings taken where the pages are silent:

* The spatial convolution changes channels (Cin -> Cout); the temporal one
  keeps Cout -> Cout.
* Spatial: stride 1, zero padding (k-1)/2 on each side of H and W,
  cross-correlation (no kernel flip), as torch's conv3d computes.
* Temporal: zero padding of k-1 frames in front, none behind.
* Optional biases are added after each convolution; no activation or norm.

Definition, with x~ the input zero-extended in H and W, p = (k-1)/2, and S
zero-extended for frames below 0:

    S[b,m,t,h,w] = sum_{c,dy,dx} Ws[m,c,0,dy,dx] x~[b,c,t,h+dy-p,w+dx-p] (+ bs[m])
    Y[b,o,t,h,w] = sum_{m,dt}    Wt[o,m,dt,0,0]  S[b,m,t+dt-(k-1),h,w]   (+ bt[o])

Computed tap by tap as shifted-slice contractions over channels (a BLAS
tensordot per tap), in float64, with no im2col, FFT or Winograd.  Tensors are
[B, C, T, H, W]; weights are in torch's [Cout, Cin, kT, kH, kW] order.
"""

import numpy as np


def _contract(w2, xs):
    """sum_c w2[o, c] * xs[b, c, ...] -> [b, o, ...] (float64)."""
    return np.moveaxis(np.tensordot(w2, xs, axes=([1], [1])), 0, 1)


def spatial_conv(x, ws, bs=None):
    """1 x k x k convolution, zero padding (k-1)/2 in H and W.

    x: [B, Cin, T, H, W]; ws: [Cout, Cin, 1, k, k]; bs: [Cout] or None.
    """
    x = np.asarray(x, dtype=np.float64)
    ws = np.asarray(ws, dtype=np.float64)
    Cout, Cin, kt, k, k2 = ws.shape
    if kt != 1 or k != k2 or k % 2 != 1:
        raise ValueError("spatial weights must be [Cout, Cin, 1, k, k] with odd k")
    B, C, T, H, W = x.shape
    if C != Cin:
        raise ValueError("channel mismatch")
    p = (k - 1) // 2
    xp = np.pad(x, ((0, 0), (0, 0), (0, 0), (p, p), (p, p)))
    out = np.zeros((B, Cout, T, H, W), dtype=np.float64)
    for dy in range(k):
        for dx in range(k):
            out += _contract(ws[:, :, 0, dy, dx], xp[:, :, :, dy:dy + H, dx:dx + W])
    if bs is not None:
        out += np.asarray(bs, dtype=np.float64)[None, :, None, None, None]
    return out


def temporal_conv(s, wt, bt=None):
    """k x 1 x 1 causal convolution, k-1 zero frames of left padding.

    s: [B, C, T, H, W]; wt: [Cout, C, k, 1, 1]; bt: [Cout] or None.
    """
    s = np.asarray(s, dtype=np.float64)
    wt = np.asarray(wt, dtype=np.float64)
    Cout, C, k, kh, kw = wt.shape
    if kh != 1 or kw != 1:
        raise ValueError("temporal weights must be [Cout, C, k, 1, 1]")
    B, Cs, T, H, W = s.shape
    if Cs != C:
        raise ValueError("channel mismatch")
    sp = np.pad(s, ((0, 0), (0, 0), (k - 1, 0), (0, 0), (0, 0)))
    out = np.zeros((B, Cout, T, H, W), dtype=np.float64)
    for dt in range(k):
        # output frame t reads padded frame t + dt, i.e. input frame t + dt - (k-1)
        out += _contract(wt[:, :, dt, 0, 0], sp[:, :, dt:dt + T])
    if bt is not None:
        out += np.asarray(bt, dtype=np.float64)[None, :, None, None, None]
    return out


def causal_conv3d_fact(x, ws, wt=None, bs=None, bt=None):
    """Spatial 1 x k x k convolution followed by the causal k x 1 x 1 one.

    With ``wt`` None only the spatial part runs (k = 1 makes it a 1x1
    projection, see ``pointwise``).
    """
    s = spatial_conv(x, ws, bs)
    if wt is None:
        return s
    return temporal_conv(s, wt, bt)


def pointwise(x, w, b=None):
    """1x1x1 projection over channels: Y[b,o,...] = sum_c W[o,c] X[b,c,...] (+ b[o]).

    w may be [Cout, Cin] or [Cout, Cin, 1, 1, 1].
    """
    w = np.asarray(w, dtype=np.float64).reshape(np.shape(w)[0], -1)
    out = _contract(w, np.asarray(x, dtype=np.float64))
    if b is not None:
        out += np.asarray(b, dtype=np.float64)[None, :, None, None, None]
    return out
