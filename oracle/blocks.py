"""Encoder residual and downsampling blocks and the decoder's mirrored upsampling
(oracle, test infrastructure).

Passages followed:

* "Cosmos World Foundation Model Platform for Physical AI (Cosmos-Predict1)"
  summary, section "1) Cosmos Tokenizer": after the 2-level Haar transform the
  encoder is made of residual blocks and downsampling blocks built from the
  space-time factorized convolution (1 x k x k, then k x 1 x 1 with k - 1 frames
  of left padding) and factorized causal self-attention; the activation is
  Swish and the normalization LayerNorm (chosen over GroupNorm so that no local
  region of the latent takes large values).  The same section lists the video
  compression factors 4x8x8, 8x8x8 and 8x16x16 (T x H x W).
* Model card "nvidia/Cosmos-Tokenize1-CV8x8x8-720p", "Model Architecture": the
  decoder mirrors the encoder; the Haar transform gives 4x in T, H and W, the
  rest of the compression comes from the blocks after it.

Readings taken where the pages are silent (no block diagram, order, stride or
epsilon is given):

* Swish(x) = x * sigmoid(x).
* LayerNorm normalizes the C channels of each position (b, t, h, w) to zero
  mean and unit variance (biased variance, eps = 1e-6 inside the square root)
  and applies a per-channel scale gamma and shift beta.
* Residual block (the usual pre-activation form):
      y = x + conv2(swish(LN2(conv1(swish(LN1(x))))))
  with conv1, conv2 factorized causal convolutions C -> C (k = 3).
* Downsampling block: the factorized convolution with stride 2 - the spatial
  1x3x3 conv with stride 2 in H and W (zero padding 1 on each side, so H, W ->
  H/2, W/2), and/or the causal temporal 3x1x1 conv with stride 2 (two zero
  frames in front, so T = 1 + 2k -> 1 + k: output frame 0 sees only frame 0,
  output frame j the frames 2j-2 .. 2j, the causal first frame kept).  A strided
  convolution is the stride-1 convolution evaluated at every second position,
  which is how it is computed here.
* Upsampling (the decoder's mirror of a downsampling block): nearest-neighbour
  repetition by 2 in H and W, and/or causal repetition in time (frame 0 once,
  every later frame twice: T -> 2T - 1, the inverse of the temporal stride),
  followed by a factorized convolution at stride 1.

Tensors are [B, C, T, H, W] float64; weights in torch's [Cout, Cin, kT, kH, kW]
order.  The convolutions are the ones of oracle.conv.
"""

import numpy as np

from oracle import conv as oconv

LN_EPS = 1e-6


def swish(x):
    """x * sigmoid(x), written as x / (1 + exp(-x))."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def layer_norm(x, gamma=None, beta=None, eps=LN_EPS):
    """Normalize the channels (axis 1) of every position, then scale and shift per channel."""
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=1, keepdims=True)
    y = (x - mean) / np.sqrt(var + eps)
    C = x.shape[1]
    shape = (1, C) + (1,) * (x.ndim - 2)
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64).reshape(shape)
    if beta is not None:
        y = y + np.asarray(beta, dtype=np.float64).reshape(shape)
    return y


def norm_swish(x, gamma=None, beta=None, eps=LN_EPS):
    return swish(layer_norm(x, gamma, beta, eps))


def factorized_conv(x, p, prefix):
    """The factorized causal conv with weights p[prefix + '_s'], p[prefix + '_t'] and
    optional biases p[prefix + '_bs'], p[prefix + '_bt']."""
    return oconv.causal_conv3d_fact(x, p[prefix + "_s"], p[prefix + "_t"], p.get(prefix + "_bs"),
                                    p.get(prefix + "_bt"))


def resblock(x, p, eps=LN_EPS):
    """x + conv2(swish(LN2(conv1(swish(LN1(x)))))).

    p holds ln1_g, ln1_b, ln2_g, ln2_b ([C]) and c1_s, c1_t, c2_s, c2_t (and
    optional c1_bs, c1_bt, c2_bs, c2_bt) for C -> C convolutions.
    """
    x = np.asarray(x, dtype=np.float64)
    h = norm_swish(x, p["ln1_g"], p["ln1_b"], eps)
    h = factorized_conv(h, p, "c1")
    h = norm_swish(h, p["ln2_g"], p["ln2_b"], eps)
    h = factorized_conv(h, p, "c2")
    return x + h


def downsample(x, ws=None, wt=None, bs=None, bt=None):
    """Strided factorized conv: spatial 1x3x3 with stride 2 in H and W (if ws is given;
    H and W even), then causal temporal 3x1x1 with stride 2 (if wt is given; T = 1 + 2k)."""
    y = np.asarray(x, dtype=np.float64)
    if ws is not None:
        _, _, _, H, W = y.shape
        if H % 2 or W % 2:
            raise ValueError("spatial downsampling needs even H and W")
        y = oconv.spatial_conv(y, ws, bs)[:, :, :, ::2, ::2]
    if wt is not None:
        T = y.shape[2]
        if (T - 1) % 2:
            raise ValueError("temporal downsampling needs T = 1 + 2k")
        y = oconv.temporal_conv(y, wt, bt)[:, :, ::2]
    return y


def upsample_repeat(x, space=True, time=True):
    """Nearest-neighbour repetition: x2 in H and W; causal x2 in time (frame 0 once,
    frames j >= 1 twice, T -> 2T - 1)."""
    y = np.asarray(x, dtype=np.float64)
    if space:
        y = np.repeat(np.repeat(y, 2, axis=3), 2, axis=4)
    if time:
        y = np.concatenate([y[:, :, :1], np.repeat(y[:, :, 1:], 2, axis=2)], axis=2)
    return y


def upsample(x, ws, wt, bs=None, bt=None, space=True, time=True):
    """Decoder upsampling block: repetition (upsample_repeat), then the factorized conv."""
    return oconv.causal_conv3d_fact(upsample_repeat(x, space, time), ws, wt, bs, bt)
