"""fp64 CPU oracle of the gated RMSNorm on the Gated DeltaNet output -- TEST
INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU leg may use
it; the product path never imports it, and it imports nothing from the
product).

The pages place a gated RMSNorm right after the DeltaNet output and note that
it is scale-invariant in its input (NPU page "Qwen3.5-9B -- every component on
the Intel NPU", section "How it works", the paragraph on fp16 precision of the
DeltaNet output), with the norm epsilon of the SSM layers 1e-6, taken from the
config (Candle pull-request page, section "Bug elimination log", bug 7).
Readings taken where the pages are silent:
  * the norm runs over the value dimension of each (token, value head) row;
  * y = o / sqrt(mean(o^2) + eps) * w * silu(z), with a weight w of length dv
    shared by the heads and the gate z (same shape as o) entering through
    silu(z) = z / (1 + exp(-z));
  * eps sits inside the square root, added to the mean square.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        x = x.double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def silu(z):
    """z * sigmoid(z), in fp64."""
    z = _f64(z)
    return z / (1.0 + np.exp(-z))


def gated_rmsnorm(o, z, weight, eps: float = 1e-6):
    """Gated RMSNorm of o [..., dv] with gate z [..., dv] and weight [dv], fp64.

    Each row o[..., :] is divided by the square root of its mean square plus
    eps, then multiplied elementwise by the weight and by silu of the gate.
    """
    o, z, w = _f64(o), _f64(z), _f64(weight)
    if o.shape != z.shape or w.shape != (o.shape[-1],):
        raise ValueError("o and z must share a shape [..., dv] and weight must be [dv]")
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return o / np.sqrt(ms + float(eps)) * w * silu(z)
