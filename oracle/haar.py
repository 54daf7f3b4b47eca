"""2-level Haar wavelet patching with the causal first frame, and its inverse.

Oracle (test infrastructure).  Plain float64 NumPy, level by level, in the
order the pages describe:

* Cosmos Tokenizer guide, section 7.1 (Haar wavelet patching): the 2D patcher
  uses the Haar filter pair (0.7071, 0.7071); each DWT multiplies the channel
  count by 4 and halves H and W, e.g. [3,256,256] -> [12,128,128] ->
  [48,64,64]; the 3D patcher multiplies channels by 8 per DWT, halves T, H
  and W, and repeats the first frame so the first latent frame stays aligned
  with the first input frame; patch size 4 means two DWT levels; the inverse
  ("UnPatcher") undoes it at the end of the decoder.
* Cosmos Tokenizer guide, sections 6.1 and 7.3: T input frames give
  1 + (T-1)/4 latent frames, latent frame 0 representing frame 0 alone.
* Cosmos-Tokenize1-CV8x8x8-720p model card, "Model Architecture": the encoder
  starts with a 2-level Haar wavelet transform that downsamples T, H and W by
  4; the decoder ends with the inverse transform.
* Cosmos-Predict1 summary, section "1) Cosmos Tokenizer": 2-level 3D Haar
  along x, y and t, each by 4.

Readings taken where the pages are silent (each one a free convention that the
GPU library matches):

* Filter taps are exactly 1/sqrt(2) (orthonormal); 0.7071 is that value
  printed to four digits.
* For a pair (e, o) of neighbours along one axis, e being the earlier /
  upper / left sample: Lo = (e + o)/sqrt(2), Hi = (e - o)/sqrt(2).
* One level transforms every axis it covers (t, h, w; or h, w for images)
  and concatenates the 8 (or 4) subbands subband-major along channels:
  channel' = s*C + c with s = 4*b_t + 2*b_h + b_w (s = 2*b_h + b_w in 2D),
  b = 0 for Lo and 1 for Hi.  The second level transforms every subband of
  the first (a full packet; only a packet gives one tensor of 48 or 192
  channels), so the final channel is s2*8C + s1*C + c (s2*4C + s1*C + c in 2D).
* The causal first frame: the sequence is extended in front with three extra
  copies of frame 0, P[p] = x[max(p - 3, 0)], which gives T + 3 = 4*T' frames.
* The inverse keeps reconstructed padded frame t + 3 as output frame t, i.e.
  drops the three leading padded frames.
"""

import numpy as np

R = 1.0 / np.sqrt(2.0)


def latent_frames(T):
    """Latent frame count 1 + (T-1)/4 of a T-frame input (guide, sections 6.1 and 7.3)."""
    if T < 1 or (T - 1) % 4 != 0:
        raise ValueError(f"temporal Haar needs T = 1 + 4k frames, got T={T}")
    return 1 + (T - 1) // 4


def causal_pad(x):
    """Prepend three copies of frame 0 along T: P[p] = x[max(p-3, 0)]."""
    first = x[:, :, :1]
    return np.concatenate([first, first, first, x], axis=2)


def _split(X, axis):
    """One Haar analysis step along ``axis``: returns (Lo, Hi)."""
    n = X.shape[axis]
    even = np.take(X, np.arange(0, n, 2), axis=axis)
    odd = np.take(X, np.arange(1, n, 2), axis=axis)
    return (even + odd) * R, (even - odd) * R


def _merge(lo, hi, axis):
    """One Haar synthesis step along ``axis`` (the transpose of ``_split``)."""
    even = (lo + hi) * R
    odd = (lo - hi) * R
    shape = list(lo.shape)
    shape[axis] *= 2
    out = np.empty(shape, dtype=np.float64)
    sl_e = [slice(None)] * lo.ndim
    sl_o = [slice(None)] * lo.ndim
    sl_e[axis] = slice(0, None, 2)
    sl_o[axis] = slice(1, None, 2)
    out[tuple(sl_e)] = even
    out[tuple(sl_o)] = odd
    return out


def haar_level(X, axes):
    """One DWT level on [B, C, T, H, W] over ``axes``; channels become
    (2**len(axes)) * C, subband-major, the first listed axis most significant."""
    bands = {(): X}
    for ax in axes:
        nxt = {}
        for key, arr in bands.items():
            lo, hi = _split(arr, ax)
            nxt[key + (0,)] = lo
            nxt[key + (1,)] = hi
        bands = nxt
    # sorted tuples (b_t, b_h, b_w) enumerate s = 4 b_t + 2 b_h + b_w in order
    return np.concatenate([bands[k] for k in sorted(bands)], axis=1)


def haar_level_inv(Y, axes):
    """Inverse of ``haar_level``."""
    nb = 2 ** len(axes)
    C = Y.shape[1] // nb
    keys = sorted(np.ndindex(*([2] * len(axes))))
    bands = {tuple(k): Y[:, i * C:(i + 1) * C] for i, k in enumerate(keys)}
    for depth in range(len(axes) - 1, -1, -1):
        ax = axes[depth]
        nxt = {}
        for key in {k[:depth] for k in bands}:
            nxt[key] = _merge(bands[key + (0,)], bands[key + (1,)], ax)
        bands = nxt
    return bands[()]


def _check_spatial(H, W):
    if H % 4 != 0 or W % 4 != 0:
        raise ValueError(f"2-level Haar needs H and W divisible by 4, got {H}x{W}")


def haar3d_fwd(x, temporal_levels=2):
    """Forward patcher on x [B, C, T, H, W] (float64).

    temporal_levels=2: 3D, output [B, 64C, 1+(T-1)/4, H/4, W/4].
    temporal_levels=3: 3D continuation chunk of a stream (T = 4k, no leading
    copies of frame 0), output [B, 64C, T/4, H/4, W/4].
    temporal_levels=0: 2D per frame, output [B, 16C, T, H/4, W/4].
    """
    x = np.asarray(x, dtype=np.float64)
    B, C, T, H, W = x.shape
    _check_spatial(H, W)
    if temporal_levels == 2:
        latent_frames(T)
        X = causal_pad(x)
        axes = (2, 3, 4)
    elif temporal_levels == 3:  # continuation chunk: frames 4j .. 4j+3 form latent frame j
        if T % 4 != 0:
            raise ValueError(f"a continuation chunk needs T = 4k frames, got T={T}")
        X = x
        axes = (2, 3, 4)
    elif temporal_levels == 0:
        X = x
        axes = (3, 4)
    else:
        raise ValueError("temporal_levels must be 0, 2 or 3")
    X = haar_level(X, axes)
    X = haar_level(X, axes)
    return X


def haar3d_inv(y, temporal_levels=2):
    """Inverse patcher: y [B, 64C, T', H', W'] -> x [B, C, 4T'-3, 4H', 4W']
    (temporal_levels=2), [B, C, 4T', 4H', 4W'] for a continuation chunk (3), or
    [B, 16C, T, H', W'] -> [B, C, T, 4H', 4W'] (0)."""
    y = np.asarray(y, dtype=np.float64)
    if temporal_levels in (2, 3):
        axes = (2, 3, 4)
        if y.shape[1] % 64:
            raise ValueError("3D inverse needs 64*C channels")
    elif temporal_levels == 0:
        axes = (3, 4)
        if y.shape[1] % 16:
            raise ValueError("2D inverse needs 16*C channels")
    else:
        raise ValueError("temporal_levels must be 0, 2 or 3")
    X = haar_level_inv(y, axes)
    X = haar_level_inv(X, axes)
    if temporal_levels == 2:
        X = X[:, :, 3:]
    return X

