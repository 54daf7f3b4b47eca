"""Finite scalar quantization (FSQ): quantize to a mixed-radix index and back.

Oracle (test infrastructure).  Passages followed:

* Cosmos Tokenizer guide, section 7.2 (FSQ): each of the latent's 6 channels
  is quantized on its own to levels [8,8,8,5,5,5]; the range is bounded with
  tanh before rounding; the implicit codebook size is the product of the
  levels, 64000; ``codes_to_indices`` turns the digits into one integer with a
  mixed-radix basis and ``indices_to_codes`` turns it back; no codebook table
  is looked up.
* Cosmos Tokenizer guide, section 6.2: indices have shape [B, T', H', W'] and
  codes [B, 6, T', H', W'].
* Cosmos-Predict1 summary, section "1) Cosmos Tokenizer": FSQ with a 6-dim
  latent and levels (8,8,8,5,5,5), vocabulary 64,000.
* The bound function is the one of the published FSQ method (Mentzer et al.
  2023, "Finite Scalar Quantization: VQ-VAE Made Simple"), restated here.

Per channel i with L = L_i levels and eps = 1e-3:

    h = (L - 1)(1 + eps)/2          half-width
    o = 1/2 if L is even else 0     offset that centres even level counts
    s = atanh(o / h)                shift, so that bound(0) = 0
    bound(z) = tanh(z + s) * h - o
    q = round_half_even(bound(z))   in [-floor(L/2), ceil(L/2) - 1]
    d = q + floor(L/2)              digit in [0, L)
    index = sum_i d_i * beta_i,     beta = (1, L_0, L_0 L_1, ...) = (1,8,64,512,2560,12800)
    code_i = q_i / floor(L/2)       normalised code in [-1, 1]

Readings taken where the pages are silent: eps = 1e-3 applied as (1+eps);
channel 0 is the least significant digit; indices are 0-based int32 in
[0, 64000) (the guide's "[1..64K]" is the README's rounding of the same
product it computes as 64000); a NaN input gives index -1 and NaN codes;
+-inf saturate to the last / first digit; an index outside [0, prod L) is
invalid and dequantizes to NaN codes.
"""

import numpy as np

DEFAULT_LEVELS = (8, 8, 8, 5, 5, 5)
EPS = 1e-3


def basis(levels=DEFAULT_LEVELS):
    """Mixed-radix place values (1, L0, L0*L1, ...)."""
    b = [1]
    for L in levels[:-1]:
        b.append(b[-1] * L)
    return np.array(b, dtype=np.int64)


def codebook_size(levels=DEFAULT_LEVELS):
    return int(np.prod(np.array(levels, dtype=np.int64)))


def constants(L, eps=EPS):
    """(h, o, s) for one channel with L levels, in float64."""
    h = (L - 1) * (1.0 + eps) / 2.0
    o = 0.5 if L % 2 == 0 else 0.0
    s = np.arctanh(o / h)
    return h, o, s


def bound(z, L, eps=EPS):
    """tanh bound of one channel (float64)."""
    h, o, s = constants(L, eps)
    return np.tanh(np.asarray(z, dtype=np.float64) + s) * h - o


def quantize(z, levels=DEFAULT_LEVELS, eps=EPS):
    """z [B, D, ...] -> (indices [B, ...] int64, codes [B, D, ...] float64, dist [B, ...]).

    ``dist`` is, per position, the smallest distance of any channel's bound
    value to a rounding boundary (a half-integer); positions with dist below
    1e-6 are the ones where two neighbouring indices are both defensible in
    floating point.
    """
    z = np.asarray(z, dtype=np.float64)
    D = z.shape[1]
    if D != len(levels):
        raise ValueError(f"latent has {D} channels but {len(levels)} levels")
    beta = basis(levels)
    idx = np.zeros(z.shape[:1] + z.shape[2:], dtype=np.int64)
    codes = np.empty_like(z)
    dist = np.full(idx.shape, np.inf)
    nan_pos = np.zeros(idx.shape, dtype=bool)
    for i, L in enumerate(levels):
        zi = z[:, i]
        nan_pos |= np.isnan(zi)
        b = bound(np.where(np.isnan(zi), 0.0, zi), L, eps)
        q = np.rint(b)                       # round half to even
        half = L // 2
        d = (q + half).astype(np.int64)
        idx += d * beta[i]
        codes[:, i] = q / half
        dist = np.minimum(dist, np.abs(b - (np.floor(b) + 0.5)))
    idx[nan_pos] = -1
    codes[np.broadcast_to(nan_pos[:, None], codes.shape)] = np.nan
    return idx, codes, dist


def quantize_f32(z, levels=DEFAULT_LEVELS, eps=EPS):
    """The same steps with every intermediate rounded to float32 (NumPy's float32
    tanh).  Used only to report how often a float32 evaluation of the bound
    would take a different decision than the float64 definition."""
    z = np.asarray(z, dtype=np.float32)
    beta = basis(levels)
    idx = np.zeros(z.shape[:1] + z.shape[2:], dtype=np.int64)
    nan_pos = np.zeros(idx.shape, dtype=bool)
    for i, L in enumerate(levels):
        h, o, s = constants(L, eps)
        zi = z[:, i]
        nan_pos |= np.isnan(zi)
        a = (np.where(np.isnan(zi), np.float32(0), zi) + np.float32(s)).astype(np.float32)
        b = (np.tanh(a).astype(np.float32) * np.float32(h)).astype(np.float32) - np.float32(o)
        q = np.rint(b.astype(np.float32))
        idx += (q.astype(np.int64) + L // 2) * beta[i]
    idx[nan_pos] = -1
    return idx


def digits(indices, levels=DEFAULT_LEVELS):
    """index -> digits [D, ...] via d_i = floor(idx / beta_i) mod L_i."""
    idx = np.asarray(indices, dtype=np.int64)
    beta = basis(levels)
    return np.stack([(idx // beta[i]) % L for i, L in enumerate(levels)])


def dequantize(indices, levels=DEFAULT_LEVELS):
    """indices [B, ...] -> (codes [B, D, ...] float64, invalid_count).

    code_i = (d_i - floor(L_i/2)) / floor(L_i/2); indices outside
    [0, prod L) give NaN codes and are counted.
    """
    idx = np.asarray(indices, dtype=np.int64)
    n = codebook_size(levels)
    bad = (idx < 0) | (idx >= n)
    d = digits(np.where(bad, 0, idx), levels)
    codes = np.empty((idx.shape[0], len(levels)) + idx.shape[1:], dtype=np.float64)
    for i, L in enumerate(levels):
        half = L // 2
        ci = (d[i] - half) / half
        codes[:, i] = np.where(bad, np.nan, ci)
    return codes, int(bad.sum())
