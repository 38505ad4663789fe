"""Chunked form of the KDA delta rule, in fp64 numpy (a test aid, not the oracle).

It restates the recurrence over chunks of C tokens so that the algebra the HIP
kernels use can be checked against the token-by-token oracle.  Within a chunk
of c <= C tokens (rows r, i = 0..c-1) with state S0 at its start:

    G_r   = sum_{j<=r} g_j                     per key channel (inclusive cumsum)
    A_ri  = beta_r * sum_c kh_rc kh_ic exp(G_rc - G_ic)      for i < r
    M_ri  =          sum_c qh_rc kh_ic exp(G_rc - G_ic)      for i <= r
    Tb    = (I + A)^-1 Diag(beta)
    X     = V - (kh * exp(G)) S0
    U     = Tb X
    O     = scale * ((qh * exp(G)) S0 + M U)
    S_c   = Diag(exp(G_last)) S0 + (kh * exp(G_last - G))^T U

The ``rnd`` hook rounds chosen operands (e.g. to bf16) to estimate what a
reduced-precision operand costs against the fp64 oracle.
"""
from __future__ import annotations

import numpy as np


def _ident(x):
    return x


def bf16_round(x):
    """Round fp64 values to bf16 (ties to even) through fp32; overflow -> inf."""
    f = np.asarray(x, np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def chunk_document(q, k, v, g, beta, C: int = 64, scale=None, eps: float = 1e-6,
                   rnd=None, rnd_state=None, rnd_out=None, initial_state=None,
                   final_state: bool = False):
    """One document, one head: q, k, g [L, K]; v [L, V]; beta [L]; initial_state
    [K, V] or None (zeros).  Returns o [L, V], or (o, S_last) with final_state."""
    rnd = rnd or _ident
    rnd_state = rnd_state or _ident
    rnd_out = rnd_out or _ident
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    L, K = q.shape
    V = v.shape[1]
    if scale is None:
        scale = K ** -0.5
    qh = q / np.sqrt((q * q).sum(-1, keepdims=True) + eps)
    kh = k / np.sqrt((k * k).sum(-1, keepdims=True) + eps)
    S = np.zeros((K, V)) if initial_state is None else np.array(initial_state, np.float64)
    o = np.zeros((L, V))
    for s in range(0, L, C):
        e = min(L, s + C)
        c = e - s
        G = np.cumsum(g[s:e], axis=0)                       # [c, K]
        diff = G[:, None, :] - G[None, :, :]                # [r, i, K]
        tri_strict = np.tril(np.ones((c, c)), -1)
        tri_incl = np.tril(np.ones((c, c)))
        with np.errstate(over="ignore", invalid="ignore"):
            E = np.where(tri_incl[:, :, None] > 0, np.exp(diff), 0.0)
        A = beta[s:e, None] * np.einsum("rc,ic,ric->ri", kh[s:e], kh[s:e], E) * tri_strict
        M = np.einsum("rc,ic,ric->ri", qh[s:e], kh[s:e], E) * tri_incl
        Tb = np.linalg.solve(np.eye(c) + A, np.diag(beta[s:e]))
        Kt = rnd(kh[s:e] * np.exp(G))
        Qt = rnd(qh[s:e] * np.exp(G))
        Kb = rnd(kh[s:e] * np.exp(G[-1][None, :] - G))
        Sb = rnd_state(S)
        X = v[s:e] - Kt @ Sb
        U = rnd(Tb) @ rnd(X)
        Ub = rnd(U)
        o[s:e] = rnd_out(scale * (Qt @ Sb + rnd(M) @ Ub))
        S = np.exp(G[-1])[:, None] * S + Kb.T @ Ub
    return (o, S) if final_state else o
