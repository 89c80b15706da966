"""Second, independent statements of the gated delta rule used to pin the oracle.

Nothing here is used by the product.  Each function restates a formula from
the pages in numpy so that the sequential oracle can be checked against it:

* `closed_form_products`: the closed-form update of the Qwen3.5-9B
  architecture page (section Gated DeltaNet), S_t = a_t (I - b_t k_t k_t^T)
  S_{t-1} + b_t k_t v_t^T, unrolled into the explicit sum over j of the
  factor products A_t ... A_{j+1} (b_j k_j v_j^T) plus A_t ... A_1 S_0, every
  dk x dk factor materialised.
* `chunkwise`: the chunkwise-parallel form of the NPU page (section "How it
  works"), in this repository's notation: per chunk, with G the running sum of
  g, gamma = exp(G), lambda = exp(G_last - G), Gamma = exp(G_last), N the
  strictly lower matrix of beta_t exp(G_t - G_j) k_t.k_j and A the lower
  matrix of exp(G_t - G_j) q_t.k_j,
      D = (I + N)^-1 diag(beta) (V - diag(gamma) K S)
      O = diag(gamma) Q S + A D,     S <- Gamma S + K^T diag(lambda) D
  with three ways to form (I + N)^-1: forward substitution (the Candle
  pull-request page, section Chunked GatedDeltaNet Scan), exact block doubling
  (D + C)^-1 = D^-1 - D^-1 C D^-1 and the product series
  (I - N)(I + N^2)(I + N^4)... (both on the NPU page).
  `masked` chooses the log-space masking of the same pull-request page (zero
  the upper-triangle exponent before exp, zero the result after) or the naive
  exp of the whole difference matrix followed by a 0/1 mask.
"""
from __future__ import annotations

import numpy as np


def closed_form_products(q, k, v, g, beta, s0, scale):
    """One sequence, one head.  q, k: [T, dk]; v: [T, dv]; g, beta: [T]; s0: [dk, dv]."""
    T, dk = k.shape
    eye = np.eye(dk)
    A = [np.exp(g[t]) * (eye - beta[t] * np.outer(k[t], k[t])) for t in range(T)]
    outs = []
    S_t = None
    for t in range(T):
        # prod(a..b) = A_b A_{b-1} ... A_a (applied right to left)
        def prod(lo, hi):
            P = eye.copy()
            for m in range(lo, hi + 1):
                P = A[m] @ P
            return P
        S_t = prod(0, t) @ s0
        for j in range(t + 1):
            S_t = S_t + prod(j + 1, t) @ (beta[j] * np.outer(k[j], v[j]))
        outs.append(scale * (S_t.T @ q[t]))
    return np.array(outs), S_t


def inv_forward_substitution(N):
    """(I + N)^-1 for strictly lower-triangular N, one row at a time."""
    C = N.shape[0]
    T = np.zeros_like(N)
    for t in range(C):
        row = np.zeros(C, dtype=N.dtype)
        row[t] = 1.0
        for j in range(t):
            row = row - N[t, j] * T[j]
        T[t] = row
    return T


def inv_block_doubling(N):
    """(I + N)^-1 by exact block doubling: split M = I + N into D (block diagonal) + C
    (the lower off-diagonal block); (D + C)^-1 = D^-1 - D^-1 C D^-1, recursively."""
    M = np.eye(N.shape[0], dtype=N.dtype) + N

    def inv(M):
        n = M.shape[0]
        if n == 1:
            return np.array([[1.0 / M[0, 0]]], dtype=M.dtype)
        h = n // 2
        Dinv = np.zeros_like(M)
        Dinv[:h, :h] = inv(M[:h, :h])
        Dinv[h:, h:] = inv(M[h:, h:])
        Cm = np.zeros_like(M)
        Cm[h:, :h] = M[h:, :h]
        return Dinv - Dinv @ Cm @ Dinv

    return inv(M)


def inv_product_series(N):
    """(I + N)^-1 = (I - N)(I + N^2)(I + N^4)... (exact once 2^m >= size, N nilpotent)."""
    C = N.shape[0]
    eye = np.eye(C, dtype=N.dtype)
    R = eye - N
    P = N @ N
    span = 2
    while span < C:
        R = R @ (eye + P)
        P = P @ P
        span *= 2
    return R


_INVERSES = {"forward": inv_forward_substitution, "doubling": inv_block_doubling,
             "series": inv_product_series}


def chunkwise(q, k, v, g, beta, s0, scale, chunk, inverse="forward", masked=True, dtype=np.float64):
    """One sequence, one head, chunk by chunk.  Returns (o [T, dv], S_T [dk, dv])."""
    q, k, v, g, beta = (np.asarray(x, dtype=dtype) for x in (q, k, v, g, beta))
    S = np.asarray(s0, dtype=dtype).copy()
    T = k.shape[0]
    o = np.zeros((T, v.shape[1]), dtype=dtype)
    inv = _INVERSES[inverse]
    with np.errstate(over="ignore", invalid="ignore"):
        for s in range(0, T, chunk):
            Q, K, V = q[s:s + chunk], k[s:s + chunk], v[s:s + chunk]
            b, C = beta[s:s + chunk], K.shape[0]
            G = np.cumsum(g[s:s + chunk]).astype(dtype)
            diff = G[:, None] - G[None, :]
            lower = np.tril(np.ones((C, C), dtype=bool))
            strict = np.tril(np.ones((C, C), dtype=bool), -1)
            if masked:
                E = np.exp(np.where(lower, diff, 0)).astype(dtype) * lower
            else:
                E = np.exp(diff).astype(dtype) * lower.astype(dtype)
            N = (b[:, None] * E * (K @ K.T)) * strict
            Tinv = inv(N.astype(dtype))
            eG = np.exp(G).astype(dtype)
            D = Tinv @ (b[:, None] * (V - eG[:, None] * (K @ S)))
            O = eG[:, None] * (Q @ S) + (E * (Q @ K.T)) @ D
            o[s:s + C] = scale * O
            lam = np.exp(G[-1] - G).astype(dtype)
            S = np.exp(G[-1]).astype(dtype) * S + K.T @ (lam[:, None] * D)
    return o, S
