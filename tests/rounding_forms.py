"""CPU emulation of where the chunk step rounds its matrix-core operands to bf16, for three
associations of the same chunkwise products (test helper; the product does not use it).

Per chunk of one value head (chunkwise form of the NPU page, section "How it works"), with
gamma = exp(G), lambda = exp(G_last - G), Gamma = exp(G_last), T = (I + N)^-1 and A the
decayed query-key matrix carrying the output scale:
  direct:    X = beta (V - gamma K S),  D = T X,  O = scale gamma Q S + A D,
             S <- Gamma S + K^T (lambda D)         (operands rounded: S, T, X, D, lambda D, A)
  wy:        W' = T (beta gamma K),  U = T (beta V),  D = U - W' S, then as direct
             (operands rounded: S, W', U, D, lambda D, A)
  absorbed:  W = K^T lambda T,  M = A T  (formed without rounding),
             O = scale gamma Q S + M X,  S <- Gamma S + W X   (operands rounded: S, X, W, M)
  tform:     Y = T X with T as a hi/lo bf16 pair,  S <- Gamma S + K^T (lambda Y) with lambda Y
             as a hi/lo pair,  O = scale gamma Q S + A Y with A and Y as hi/lo pairs (the
             lo x lo product dropped)              (operands rounded: S, X; T, lambda Y, A, Y split)
Every product accumulates in fp32; T comes from an fp64 inverse (the solve is not what is
compared here).
"""
import numpy as np
import torch


def _bf(x):
    return x.to(torch.bfloat16).to(torch.float32)


def _split(x):
    hi = _bf(x)
    return hi, _bf(x - hi)


def run(q, k, v, g, beta, form, chunk=64, scale=None):
    """One sequence of one value head: q, k [T, dk], v [T, dv] (any float dtype), g, beta [T].
    Returns (o [T, dv], final S [dk, dv]) as fp64 numpy arrays."""
    q, k, v = q.float(), k.float(), v.float()
    g, beta = g.double(), beta.float()
    T, dk = q.shape
    dv = v.shape[1]
    scale = dk ** -0.5 if scale is None else scale
    S = torch.zeros(dk, dv)
    o = torch.zeros(T, dv)
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        L = c1 - c0
        G = torch.cumsum(g[c0:c1], 0)
        low = torch.tril(torch.ones(L, L, dtype=torch.bool))
        E = torch.where(low, torch.exp(torch.where(low, G[:, None] - G[None, :], torch.zeros(L, L))),
                        torch.zeros(L, L)).float()
        K, Q, V, b = k[c0:c1], q[c0:c1], v[c0:c1], beta[c0:c1]
        N = torch.tril(b[:, None] * E * (K @ K.T), -1)
        Tm = torch.linalg.inv(torch.eye(L, dtype=torch.float64) + N.double()).float()
        A = scale * E * (Q @ K.T)
        gam, lam = torch.exp(G).float(), torch.exp(G[-1] - G).float()
        Gam = float(torch.exp(G[-1]))
        Sb = _bf(S)
        if form == "tform":
            X = _bf(b[:, None] * V - (b * gam)[:, None] * (K @ Sb))
            Th, Tl = _split(Tm)
            Y = Th @ X + Tl @ X
            Dh, Dl = _split(lam[:, None] * Y)
            Ah, Al = _split(A)
            Yh, Yl = _split(Y)
            o[c0:c1] = scale * gam[:, None] * (Q @ Sb) + Ah @ Yh + Ah @ Yl + Al @ Yh
            S = Gam * S + K.T @ Dh + K.T @ Dl
            continue
        if form == "absorbed":
            W = (K.T * lam[None, :]) @ Tm
            M = A @ Tm
            X = _bf(b[:, None] * V - (b * gam)[:, None] * (K @ Sb))
            o[c0:c1] = scale * gam[:, None] * (Q @ Sb) + _bf(M) @ X
            S = Gam * S + _bf(W) @ X
            continue
        if form == "direct":
            X = b[:, None] * V - (b * gam)[:, None] * (K @ Sb)
            D = _bf(Tm) @ _bf(X)
        elif form == "wy":
            Wp = Tm @ ((b * gam)[:, None] * K)
            U = Tm @ (b[:, None] * V)
            D = _bf(U) - _bf(Wp) @ Sb
        else:
            raise KeyError(form)
        o[c0:c1] = scale * gam[:, None] * (Q @ Sb) + _bf(A) @ _bf(D)
        S = Gam * S + K.T @ _bf(lam[:, None] * D)
    return o.double().numpy(), S.double().numpy()


def max_rel(x, ref):
    return float(np.max(np.abs(x - ref)) / np.max(np.abs(ref)))
