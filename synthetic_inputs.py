"""Seeded synthetic inputs and the workload shapes they are drawn for.

This module is shared by the tests, the smoke check and the benchmark; it holds
none of the tokenizer's arithmetic (no Haar, convolution or FSQ step), only
random draws and the bf16 rounding of those draws, so both the CPU oracle and
the HIP library consume byte-identical inputs.

The shapes follow the pages' workloads: 121-frame 720p clips (the
Cosmos-Tokenize1-CV8x8x8-720p context), 49-frame clips at 720p and 360p
(the DV8x16x16-720p and DV4x8x8-360p contexts), and a single image; pixels are
RGB in [-1, 1].  These stand in for the DAVIS / TokenBench clips the pages
evaluate on, which are not used.

Generators (NumPy PCG64, parameters drawn first, then the noise, C order):

* ``video_sin``: per (batch, channel) three sinusoids with amplitude
  U(0.15, 0.30), spatial frequencies U(0.5, 3) cycles per frame width /
  height, temporal frequency U(0, 2) cycles per clip and phase U(0, 2 pi),
  plus N(0, 0.05) noise, clipped to [-1, 1].
* ``video_trans``: the same spatial field with no temporal frequency,
  translated by a seeded velocity U(-4, 4) px/frame in x and y (a smooth
  moving scene), plus N(0, 0.05) noise, clipped to [-1, 1].
* ``normal``: N(0, std) draws (weights with std 0.02, FSQ latents with std 1.5).
* ``uniform_indices``: int32 indices uniform in [0, high).
"""

import numpy as np

TWO_PI = 2.0 * np.pi


def _field(rng, B, C, T, H, W, moving):
    x = np.zeros((B, C, T, H, W), dtype=np.float32)
    t = np.arange(T, dtype=np.float64)
    h = np.arange(H, dtype=np.float64)
    w = np.arange(W, dtype=np.float64)
    params = []
    for b in range(B):
        for c in range(C):
            comps = []
            for _ in range(3):
                a = rng.uniform(0.15, 0.30)
                fx = rng.uniform(0.5, 3.0)
                fy = rng.uniform(0.5, 3.0)
                ft = 0.0 if moving else rng.uniform(0.0, 2.0)
                phi = rng.uniform(0.0, TWO_PI)
                comps.append((a, fx, fy, ft, phi))
            vel = (rng.uniform(-4.0, 4.0), rng.uniform(-4.0, 4.0)) if moving else (0.0, 0.0)
            params.append((b, c, comps, vel))
    for b, c, comps, (vy, vx) in params:
        acc = np.zeros((T, H, W), dtype=np.float32)
        for a, fx, fy, ft, phi in comps:
            # phase = 2 pi (fx (w - vx t)/W + fy (h - vy t)/H + ft t/T) + phi,
            # split as P(w) + Q(t, h) and evaluated with the angle-sum identity.
            P = TWO_PI * fx * w / W
            Q = (TWO_PI * (fy * h[None, :] / H
                           - (fx * vx / W + fy * vy / H) * t[:, None]
                           + ft * t[:, None] / T) + phi)
            sP, cP = np.sin(P).astype(np.float32), np.cos(P).astype(np.float32)
            sQ, cQ = np.sin(Q).astype(np.float32), np.cos(Q).astype(np.float32)
            acc += np.float32(a) * (sQ[:, :, None] * cP[None, None, :] + cQ[:, :, None] * sP[None, None, :])
        x[b, c] = acc
    return x


def _add_noise_clip(rng, x, sigma=0.05):
    noise = rng.standard_normal(x.shape, dtype=np.float32)
    noise *= np.float32(sigma)
    x += noise
    np.clip(x, -1.0, 1.0, out=x)
    return x


def video_sin(shape, seed):
    """[B, C, T, H, W] float32 sinusoid video in [-1, 1]."""
    rng = np.random.default_rng(seed)
    x = _field(rng, *shape, moving=False)
    return _add_noise_clip(rng, x)


def video_trans(shape, seed):
    """[B, C, T, H, W] float32 translating-field video in [-1, 1]."""
    rng = np.random.default_rng(seed)
    x = _field(rng, *shape, moving=True)
    return _add_noise_clip(rng, x)


def normal(shape, seed, std):
    """float32 N(0, std) draws."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return a


def uniform_indices(shape, seed, high=64000):
    rng = np.random.default_rng(seed)
    return rng.integers(0, high, size=shape, dtype=np.int32)


def to_bf16_bits(a):
    """float32 array -> uint16 bf16 bit patterns (round to nearest even, torch CPU cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def weight_seed(config, layer):
    return 2000 + 10 * config + layer


# Workload shapes.  "x" is the pixel input [B, C, T, H, W]; the post-Haar grid
# is [B, 64C, 1+(T-1)/4, H/4, W/4] (16C and T for the 2D image patcher).
WORKLOADS = {
    "c1_image_64": dict(
        x=(1, 3, 1, 64, 64), dtype="f32", gen="sin", seed=1001, temporal_levels=0,
        convs=[(48, 64, 3), (64, 6, 1)], fsq=True),
    "c2_video_17x256": dict(
        x=(1, 3, 17, 256, 256), dtype="bf16", gen="sin", seed=1002, temporal_levels=2,
        convs=[(192, 256, 3), (256, 16, 1)], fsq=False),
    "c3_cv8x8x8_720p_121f": dict(
        x=(1, 3, 121, 720, 1280), dtype="bf16", gen="trans", seed=1003, temporal_levels=2,
        convs=[(192, 256, 3), (256, 256, 3), (256, 16, 1)], fsq=False),
    "c4_dv8x16x16_720p_49f": dict(
        x=(1, 3, 49, 720, 1280), dtype="bf16", gen="trans", seed=1004, temporal_levels=2,
        convs=[(192, 256, 3), (256, 6, 1)], fsq=True,
        latent=(1, 6, 13, 180, 320), latent_seed=1014, latent_std=1.5),
    "c5_dv4x8x8_360p_decode": dict(
        indices=(8, 13, 90, 160), seed=1005,
        convs=[(6, 192, 1), (192, 192, 3)], out_x=(8, 3, 49, 360, 640)),
    # FSQ at a bandwidth-meaningful size: 64 latents of the 49-frame 720p grid
    "fsq_bw": dict(latent=(64, 6, 13, 180, 320), latent_seed=1015, latent_std=1.5),
    # factorized attention on the CV8x8x8-720p token grid of a 121-frame clip (16 x 90 x 160),
    # 256 channels in 4 heads of 64; q, k, v ~ N(0, 1), seeds seed, seed + 1, seed + 2
    "attn_cv8x8x8_720p_tokens": dict(x=(1, 256, 16, 90, 160), heads=4, seed=1006, std=1.0),
    # encoder / decoder blocks on the CV8x8x8-720p grids of a 121-frame clip: a residual block
    # and the stride-2 downsampling block at the post-Haar grid 31 x 180 x 320 (-> 16 x 90 x
    # 160), the mirrored upsampling block back; 256 channels, x ~ N(0, 1), conv weights
    # N(0, 0.02), LayerNorm scales 1 and shifts 0 (seeds seed .. seed + 9)
    "blocks_cv8x8x8_720p": dict(x=(1, 256, 31, 180, 320), low=(1, 256, 16, 90, 160), seed=1030, w_std=0.02),
    # a 1080p clip whose length and height the tokenizer does not accept as they are: 50
    # frames (not 1 + 4k) of 1080 rows (not a multiple of 16), worked through in windows of
    # 17 frames padded to 1 + 4k frames and 1088 x 1920; pixels N(0, 0.5)
    "window_1080p_50f": dict(x=(1, 3, 50, 1080, 1920), seed=1020, std=0.5, window=17, t_align=4,
                             s_align=16),
    # activations of 2 GiB or more: a 256-channel tensor on 40 frames of a 1080p clip's post-Haar
    # grid (270 x 480), 2.65 GB in bf16; x ~ N(0, 1), conv weights N(0, 0.02)
    "large_256x40x270x480": dict(x=(1, 256, 40, 270, 480), seed=1040, w_std=0.02),
    # a 129-frame 1080p clip (the model card's longest one-pass 1080p input is 8 s): Haar ->
    # conv 192 -> 256 (its output, 2.19 GB, is the temporal conv's input) -> temporal conv with
    # the 1x1 -> 16 fused; G_trans pixels
    "clip_1080p_129f": dict(x=(1, 3, 129, 1080, 1920), seed=1041),
}
