"""Pins of the oracle's bf16 codec against torch's bf16 cast and the format's
tie and overflow rules."""

import numpy as np
import torch

from oracle import bf16


def torch_bits(a32):
    return torch.from_numpy(a32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_decode_exact_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16.decode(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_encode_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),       # subnormal range
        (rng.standard_normal(20000) * 3e38).astype(np.float32),        # near overflow
        rng.integers(0, 2**32, 100000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    vals = vals[np.isfinite(vals)]
    np.testing.assert_array_equal(bf16.encode(vals.astype(np.float64)), torch_bits(vals))


def test_ties_round_to_even_and_overflow():
    one = 1.0
    assert bf16.encode(np.array([one + 2.0 ** -8]))[0] == 0x3F80          # tie -> even (1.0)
    assert bf16.encode(np.array([one + 3 * 2.0 ** -8]))[0] == 0x3F82      # tie -> even (1 + 2^-6)
    assert bf16.encode(np.array([one + 2.0 ** -8 + 2.0 ** -40]))[0] == 0x3F81  # above tie -> up
    assert bf16.encode(np.array([3.5e38]))[0] == 0x7F80                   # overflow -> +inf
    assert bf16.encode(np.array([-np.inf]))[0] == 0xFF80
    assert bf16.encode(np.array([np.nan]))[0] == bf16.QNAN_BITS
    assert bf16.encode(np.array([-0.0]))[0] == 0x8000


def test_ulp():
    assert bf16.ulp(np.array([0x3F80]))[0] == 2.0 ** -7
    assert bf16.ulp(np.array([0x4000]))[0] == 2.0 ** -6
