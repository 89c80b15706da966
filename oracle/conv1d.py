"""fp64 CPU oracle of the depthwise causal conv1d ahead of the gated delta rule
-- TEST INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU leg
may use it; the product path never imports it, and it imports nothing from the
product).

The pages put a depthwise causal conv in the Gated DeltaNet layer ahead of the
recurrence, with a conv state kept per layer between calls next to the
recurrent state (NPU page "Qwen3.5-9B -- every component on the Intel NPU",
section "How it works": the caches hold 24 conv states and 24 recurrent
states; section "New in v2": prefix reuse keeps the recurrent/conv/KV state),
and fix its orientation to PyTorch's Conv1d with left padding: the kernel is
applied as a cross-correlation over the window that ends at the current token
(Candle pull-request page, section "Bug elimination log", bug 2).  q and k
reach the recurrence L2-normalised per head (the problem statement of the
rule).  Readings taken where the pages are silent:
  * channel c of token t: y[t, c] = sum_{i<K} w[c, i] * x[t - K + 1 + i, c], so
    w[c, K-1] multiplies the current token;
  * inputs before the first token of a sequence come from its conv state,
    state[n, c, j] = x[-(K - 1) + j, c] (oldest first), zeros when there is no
    state; after the call the state holds the last K - 1 inputs of the sequence
    (older state entries shift in when the sequence is shorter than K - 1);
  * no activation unless asked for (silu(y) = y * sigmoid(y) is an option);
  * the channels are laid out [q heads | k heads | v heads]; q and k heads are
    L2-normalised after the conv as y / sqrt(sum(y^2) + eps).
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        if not x.dtype.is_floating_point:
            return np.ascontiguousarray(x.numpy()).astype(np.float64)
        x = x.double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _offsets(cu_seqlens, T):
    if cu_seqlens is None:
        return np.array([0, T], dtype=np.int64)
    if hasattr(cu_seqlens, "detach"):
        cu_seqlens = cu_seqlens.detach().to("cpu").numpy()
    return np.asarray(cu_seqlens, dtype=np.int64)


def causal_conv1d(x, weight, cu_seqlens=None, state=None, silu=False):
    """Depthwise causal conv of a packed batch x [T, C] with weight [C, K], fp64.

    state: [N, C, K-1] inputs before each sequence (None = zeros).
    Returns (y [T, C], new_state [N, C, K-1]).
    """
    x, w = _f64(x), _f64(weight)
    T, C = x.shape
    if w.ndim != 2 or w.shape[0] != C or w.shape[1] < 1:
        raise ValueError("weight must be [C, K]")
    K = w.shape[1]
    cu = _offsets(cu_seqlens, T)
    n = cu.shape[0] - 1
    s = np.zeros((n, C, K - 1)) if state is None else _f64(state)
    if s.shape != (n, C, K - 1):
        raise ValueError("state must be [N, C, K-1]")
    y = np.zeros((T, C))
    new_state = np.zeros((n, C, K - 1))
    for i in range(n):
        a, b = int(cu[i]), int(cu[i + 1])
        # the sequence's inputs, preceded by its K-1 earlier inputs from the state
        xs = np.concatenate([s[i].T, x[a:b]], axis=0)          # [K-1 + L, C]
        for t in range(b - a):
            acc = np.zeros(C)
            for j in range(K):
                acc += w[:, j] * xs[t + j]                      # x[t - K + 1 + j]
            y[a + t] = acc
        new_state[i] = xs[xs.shape[0] - (K - 1):].T if K > 1 else new_state[i]
    if silu:
        y = y / (1.0 + np.exp(-y))
    return y, new_state


def l2_normalise_heads(y, head_dim, eps):
    """y [T, H * head_dim] -> each head block divided by sqrt(sum of squares + eps)."""
    y = _f64(y)
    T, C = y.shape
    h = y.reshape(T, C // head_dim, head_dim)
    return (h / np.sqrt(np.sum(h * h, axis=-1, keepdims=True) + float(eps))).reshape(T, C)


def conv_qkv(x, weight, hqk, hv, dk, dv, cu_seqlens=None, state=None, silu=False, l2norm=True, eps=1e-6):
    """The conv over the packed projections [q heads | k heads | v heads], then q and k
    L2-normalised per head.  Returns (q [T, HQK, dk], k [T, HQK, dk], v [T, HV, dv],
    new_state [N, C, K-1])."""
    y, new_state = causal_conv1d(x, weight, cu_seqlens, state, silu)
    T = y.shape[0]
    nq = hqk * dk
    if y.shape[1] != 2 * nq + hv * dv:
        raise ValueError("x must have 2 * HQK * dk + HV * dv channels")
    q, k, v = y[:, :nq], y[:, nq:2 * nq], y[:, 2 * nq:]
    if l2norm:
        q, k = l2_normalise_heads(q, dk, eps), l2_normalise_heads(k, dk, eps)
    return q.reshape(T, hqk, dk), k.reshape(T, hqk, dk), v.reshape(T, hv, dv), new_state
