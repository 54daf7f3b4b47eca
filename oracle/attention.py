"""Factorized causal self-attention over a video feature map (oracle, test infrastructure).

Passages followed:

* "Cosmos World Foundation Model Platform for Physical AI (Cosmos-Predict1)",
  section "1) Cosmos Tokenizer": the encoder's blocks pair the space-time
  factorized convolution with space-time factorized causal self-attention.
* "nvidia/Cosmos-Tokenize1-CV8x8x8-720p" (model card), "Model Architecture":
  causal temporal attention layers keep the frames' temporal order, so tokens
  of a frame depend only on the same and earlier frames.
* The Cosmos Tokenizer guide's overview: the causal encoder holds causal
  convolution and causal attention along time.

Readings taken where the pages are silent (they give no formula, head count or
width):

* "Factorized" means two attentions over a [B, C, T, H, W] feature map:
  SPATIAL, over the H*W positions of one frame, where every position attends to
  every position of the same frame (no mask: space has no causal order); and
  TEMPORAL, over the T frames of one position, causal: frame t attends to the
  frames s <= t only.
* Each is scaled dot-product attention, softmax(Q K^T / sqrt(d)) V, with the C
  channels split into G heads of d = C / G consecutive channels (head g holds
  channels g*d .. g*d + d - 1); heads are independent.
* Q, K and V are inputs: the linear maps that produce them (and the output
  map) are 1x1x1 convolutions, oracle.conv.pointwise.

The core is written out on [..., N, d] token matrices with NumPy's matmul as
the only library step, in float64, with the usual max subtraction before the
exponential (which leaves the softmax unchanged).
"""

import numpy as np


def attention(q, k, v, causal=False):
    """softmax(q k^T / sqrt(d) [+ causal mask]) v over the last two axes.

    q, k, v: [..., N, d] (the same leading shape).  With causal, query i sees
    keys j <= i only.  Returns [..., N, d] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape[-2], q.shape[-1]
    s = np.matmul(q, np.swapaxes(k, -1, -2)) / np.sqrt(d)
    if causal:
        s = np.where(np.tril(np.ones((n, n), dtype=bool)), s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    return np.matmul(p, v)


def attention_rows(q_rows, k, v):
    """The non-causal attention output of a few query rows against all keys:
    q_rows [R, d], k and v [N, d] -> [R, d].  Used to check single outputs of
    sequences too long for a full N x N score matrix."""
    return attention(np.asarray(q_rows, dtype=np.float64)[None], np.asarray(k)[None], np.asarray(v)[None])[0]


def _split_heads(x, heads):
    B, C, T, H, W = x.shape
    if heads < 1 or C % heads != 0:
        raise ValueError("C must be a multiple of heads")
    return np.asarray(x, dtype=np.float64).reshape(B, heads, C // heads, T, H, W)


def spatial_attention(q, k, v, heads):
    """Attention over the H*W positions of each frame and head.

    q, k, v: [B, C, T, H, W]; heads divides C.  Returns [B, C, T, H, W] float64.
    """
    B, C, T, H, W = np.shape(q)
    d = C // heads

    def tokens(x):  # [B, G, d, T, H, W] -> [B, T, G, H*W, d]
        return _split_heads(x, heads).transpose(0, 3, 1, 4, 5, 2).reshape(B, T, heads, H * W, d)

    o = attention(tokens(q), tokens(k), tokens(v), causal=False)
    return o.reshape(B, T, heads, H, W, d).transpose(0, 2, 5, 1, 3, 4).reshape(B, C, T, H, W)


def temporal_attention(q, k, v, heads):
    """Causal attention over the T frames of each position and head.

    q, k, v: [B, C, T, H, W]; heads divides C.  Returns [B, C, T, H, W] float64.
    """
    B, C, T, H, W = np.shape(q)
    d = C // heads

    def tokens(x):  # [B, G, d, T, H, W] -> [B, H, W, G, T, d]
        return _split_heads(x, heads).transpose(0, 4, 5, 1, 3, 2)

    o = attention(tokens(q), tokens(k), tokens(v), causal=True)
    return o.transpose(0, 3, 5, 4, 1, 2).reshape(B, C, T, H, W)
