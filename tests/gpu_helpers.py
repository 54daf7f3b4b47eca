"""Helpers shared by the GPU parity tests: moving seeded host inputs to the
device, reading results back, and the comparison criteria.

Criteria (applied element by element):
* float32 stages: |g - o| <= tol * (|o| + rms(o)), tol = 1e-5 for Haar;
* bf16 outputs of exact stages (Haar): |g - bf16(o)| <= 1 bf16 ulp of bf16(o)
  (or |g - o| <= 1e-12 rms(o), the oracle's own rounding level);
* bf16 convolution outputs: |g - o| <= 2e-2 * (|o| + rms(o));
* integer outputs (FSQ indices, digits): bit-exact.
The reference o is always the float64 oracle evaluated on the same bits.
"""

import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import bf16 as obf16  # noqa: E402

DEV = "cuda:0"


def log(msg):
    print(msg, flush=True)


def bits_to_torch(bits, device=DEV, channels_last=False):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    t = t.to(device)
    if channels_last:
        t = t.to(memory_format=torch.channels_last_3d)
    return t


def f32_to_torch(a, device=DEV, channels_last=False):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    if channels_last:
        t = t.to(memory_format=torch.channels_last_3d)
    return t


def to_f64(t):
    """Device tensor (any layout, f32/bf16) -> float64 numpy in logical order."""
    return t.detach().to("cpu").contiguous().to(torch.float64).numpy()


def to_bits(t):
    """bf16 device tensor -> uint16 bit patterns in logical order."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def rel_report(g, o, tol):
    """(number of elements outside tol*(|o|+rms(o)), worst ratio, relative L2)."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    rms = float(np.sqrt(np.mean(o * o))) if o.size else 0.0
    err = np.abs(g - o)
    bound = tol * (np.abs(o) + rms)
    ratio = err / np.where(bound > 0, bound, 1e-300)
    nbad = int(np.sum(err > bound))
    relL2 = float(np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-300))
    return nbad, float(ratio.max()) if ratio.size else 0.0, relL2


def assert_rel(g, o, tol, what):
    nbad, worst, relL2 = rel_report(g, o, tol)
    log(f"  {what}: n={np.size(o)} bad={nbad} worst/tol={worst:.3g} relL2={relL2:.3g}")
    assert nbad == 0, f"{what}: {nbad} elements outside {tol}*(|o|+rms)"
    return relL2


def assert_bf16_ulp(g_bits, o, what, max_ulp=1):
    """g_bits: GPU bf16 bits; o: float64 oracle values.  Each GPU value must be
    within max_ulp bf16 ulps of the oracle rounded to bf16, or within
    1e-12 * rms(o) of it: the oracle's own float64 rounding (it multiplies by
    1/sqrt(2) per level) leaves ~1e-16 where the exact coefficient is 0, which
    the float32 butterflies return exactly."""
    ob = obf16.encode(o)
    gv = obf16.decode(g_bits)
    ov = obf16.decode(ob)
    diff = np.abs(gv - ov)
    u = obf16.ulp(ob)
    floor = 1e-12 * float(np.sqrt(np.mean(np.square(o)))) if np.size(o) else 0.0
    nbad = int(np.sum((diff > max_ulp * u) & (np.abs(gv - o) > floor)))
    nne = int(np.sum(g_bits != ob))
    log(f"  {what}: n={o.size} not-identical={nne} ({nne / max(o.size, 1):.2e}) beyond {max_ulp} ulp={nbad}")
    assert nbad == 0, f"{what}: {nbad} elements beyond {max_ulp} bf16 ulp"
    return nne


def nthwc_to_logical(a):
    """numpy [B, T, H, W, C] -> [B, C, T, H, W]."""
    return np.moveaxis(a, -1, 1)
