"""Sliding-window processing of videos of any length and size (oracle, test infrastructure).

Passage followed: the Cosmos Tokenizer guide, section 6.3 (end-to-end
reconstruction and videos of any length).  The tokenizer's forward pass takes a
``temporal_window`` (17 frames in the guide) and works through the video one
window at a time; each window is first padded up to sizes the network accepts,
with zeros in space and by reflection at the edge in time, is reconstructed,
cropped back to its own size, and the windows are concatenated.  Sections 6.1
and 7.3 fix what an aligned length is for a causal video tokenizer: 1 + k*f
frames for a temporal compression f (the first frame on its own, then groups
of f).

Readings taken where the passage is silent:

* Windows are consecutive and do not overlap: window i holds frames
  [i*win, min((i+1)*win, T)); the last one may be shorter.
* Each window is a clip of its own: it restarts the causal first frame.
* Padding goes after the content (frames after the window's last frame, rows
  below, columns to the right), so that the crop keeps indices unchanged.
* Aligned sizes: the time length becomes the smallest 1 + k*t_align >= nt, the
  height and width the smallest multiples of s_align (the spatial compression)
  that are >= H and >= W.
* "Reflection at the edge" is the mirror about the last frame, without
  repeating it: frames nt-2, nt-3, ... follow frame nt-1, and the mirror
  bounces back and forth if the pad is longer than the window (NumPy's
  ``reflect`` mode); a one-frame window repeats its frame.

The only library step is numpy.pad; the window list and the aligned sizes are
integer arithmetic written out.
"""

import numpy as np


def window_bounds(T, window):
    """[(t0, nt), ...]: the consecutive windows of at most ``window`` frames that
    cover frames 0 .. T-1."""
    if T < 1 or window < 1:
        raise ValueError("T and window must be positive")
    out, t0 = [], 0
    while t0 < T:
        nt = min(window, T - t0)
        out.append((t0, nt))
        t0 += nt
    return out


def aligned_size(nt, H, W, t_align, s_align):
    """(Tp, Hp, Wp): the smallest 1 + k*t_align >= nt and the smallest multiples of
    s_align >= H and >= W."""
    if min(nt, H, W, t_align, s_align) < 1:
        raise ValueError("sizes and alignments must be positive")
    k = -(-(nt - 1) // t_align)
    Tp = 1 + k * t_align
    Hp = -(-H // s_align) * s_align
    Wp = -(-W // s_align) * s_align
    return Tp, Hp, Wp


def pad_window(x, t0, nt, Tp, Hp, Wp):
    """Frames t0 .. t0+nt-1 of x [B, C, T, H, W], padded to [B, C, Tp, Hp, Wp]:
    mirrored frames after the last one, zero rows and columns after the content."""
    x = np.asarray(x)
    B, C, T, H, W = x.shape
    if not (0 <= t0 and nt >= 1 and t0 + nt <= T and Tp >= nt and Hp >= H and Wp >= W):
        raise ValueError("window outside the clip or padded size too small")
    win = x[:, :, t0:t0 + nt]
    win = np.pad(win, ((0, 0), (0, 0), (0, Tp - nt), (0, 0), (0, 0)), mode="reflect" if nt > 1 else "edge")
    return np.pad(win, ((0, 0), (0, 0), (0, 0), (0, Hp - H), (0, Wp - W)), mode="constant")


def unpad_window(y, out, t0, nt):
    """Crop a processed padded window y [B, C, Tp, Hp, Wp] back to nt frames and
    out's H x W, and place it at frames t0 .. t0+nt-1 of out [B, C, T, H, W] (in place)."""
    B, C, T, H, W = out.shape
    if not (0 <= t0 and nt >= 1 and t0 + nt <= T):
        raise ValueError("window outside the clip")
    if y.shape[2] < nt or y.shape[3] < H or y.shape[4] < W:
        raise ValueError("padded window smaller than its crop")
    out[:, :, t0:t0 + nt] = y[:, :, :nt, :H, :W]
    return out


def windowed(x, process, window, t_align, s_align):
    """Run ``process`` (a function from a padded window [B, C, Tp, Hp, Wp] to an
    array of the same shape, e.g. encode then decode) window by window over
    x [B, C, T, H, W] and return the cropped, concatenated result."""
    x = np.asarray(x)
    B, C, T, H, W = x.shape
    out = np.zeros(x.shape, dtype=np.float64)
    for t0, nt in window_bounds(T, window):
        Tp, Hp, Wp = aligned_size(nt, H, W, t_align, s_align)
        y = process(pad_window(x, t0, nt, Tp, Hp, Wp))
        unpad_window(np.asarray(y), out, t0, nt)
    return out
