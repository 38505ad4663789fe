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


def f16_round(x):
    """Round to fp16 (ties to even, subnormals kept) through fp32."""
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float16).astype(np.float64)


def pow2_f16(x, block=None, two_way=True):
    """fp16 rounding behind an exact power-of-two scale, as the kernels store
    their fp16 operands: per group of ``block`` columns (all columns when None)
    the largest magnitude m picks e = 0 when 2^-4 <= m < 2^14, and otherwise
    e with m 2^-e in [2^13, 2^14); x 2^-e is rounded to fp16 and multiplied
    back by 2^e.  With ``two_way`` False, e is never negative (values are only
    ever scaled down), so small inputs fall into the fp16 subnormal range."""
    x = np.asarray(x, np.float64)
    out = np.empty_like(x)
    cols = x.shape[-1]
    block = block or cols
    for c0 in range(0, cols, block):
        part = x[..., c0:c0 + block]
        m = float(np.abs(part).max()) if part.size else 0.0
        if m == 0.0:
            out[..., c0:c0 + block] = 0.0
            continue
        e = np.frexp(np.float32(m))[1] - 1 - 13
        if 2.0 ** -4 <= m < 2.0 ** 14 or (not two_way and e < 0):
            e = 0
        out[..., c0:c0 + block] = f16_round(part * 2.0 ** -e) * 2.0 ** e
    return out


def kernel_precision_ops(two_way=True):
    """Operand roundings of the forward kernels: Qt, Kt and the MFMA copy of S
    in bf16; KbT and M in fp16 (both bounded by 1); Tb in fp16 with one
    power-of-two scale per chunk; X and U in fp16 with one scale per 32 value
    columns (one wave's columns)."""
    return dict(Qt=bf16_round, Kt=bf16_round, S=bf16_round, Kb=f16_round, M=f16_round,
                Tb=lambda x: pow2_f16(x, None, two_way),
                X=lambda x: pow2_f16(x, 32, two_way),
                U=lambda x: pow2_f16(x, 32, two_way))


def chunk_document(q, k, v, g, beta, C: int = 64, scale=None, eps: float = 1e-6,
                   rnd=None, rnd_state=None, rnd_out=None, initial_state=None,
                   final_state: bool = False, ops=None):
    """One document, one head: q, k, g [L, K]; v [L, V]; beta [L]; initial_state
    [K, V] or None (zeros).  Returns o [L, V], or (o, S_last) with final_state.
    ``ops`` (see kernel_precision_ops) rounds each named operand on its own and
    replaces rnd / rnd_state."""
    rnd = rnd or _ident
    rnd_state = rnd_state or _ident
    rnd_out = rnd_out or _ident
    op = {name: rnd for name in ("Qt", "Kt", "Kb", "M", "Tb", "X", "U")}
    op["S"] = rnd_state
    if ops is not None:
        op.update(ops)
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
        Kt = op["Kt"](kh[s:e] * np.exp(G))
        Qt = op["Qt"](qh[s:e] * np.exp(G))
        Kb = op["Kb"](kh[s:e] * np.exp(G[-1][None, :] - G))
        Sb = op["S"](S)
        X = v[s:e] - Kt @ Sb
        U = op["Tb"](Tb) @ op["X"](X)
        Ub = op["U"](U)
        o[s:e] = rnd_out(scale * (Qt @ Sb + op["M"](M) @ Ub))
        S = np.exp(G[-1])[:, None] * S + Kb.T @ Ub
    return (o, S) if final_state else o


def chunk_document_backward(q, k, v, g, beta, do, C: int = 64, scale=None, eps: float = 1e-6,
                            initial_state=None, d_final_state=None):
    """Gradients of one document, one head, by the chunked backward the GPU
    implements (fp64).  q, k, g [L, K]; v, do [L, V]; beta [L].  Returns
    dq, dk, dv, dg, dbeta, dh0.

    Per chunk (rows r, i; state S0 at its start, dSc = dL/dS at its end):
        dU   = scale M^T dO + Kbar dSc           dX = Tb^T dU  (= dV)
        dS0  = D dSc + scale Qt^T dO - Kt^T dX   (handed to the previous chunk)
        dQt  = scale dO S0^T,  dKt = -dX S0^T,   dKbar = U dSc^T,  dD = rowsum(dSc * S0)
        dM   = scale tril(dO U^T),  dTb = tril(dU X^T)
        dbeta_i += sum_r dTb_ri T_ri,  dT = dTb diag(beta),  dA = -T^T dT T^T (strict lower)
        dbeta_r += sum_i dA_ri Kk_ri,  dKk = diag(beta) dA
    then the bilinear forms M = tril(sum_c qh_rc kh_ic E_ric), Kk (strict) with
    E_ric = exp(G_rc - G_ic), the decayed tiles Qt, Kt, Kbar, D, the in-chunk
    cumsum G of g, and the l2 norms."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    do = np.asarray(do, np.float64)
    L, K = q.shape
    V = v.shape[1]
    if scale is None:
        scale = K ** -0.5
    nq = np.sqrt((q * q).sum(-1, keepdims=True) + eps)
    nk = np.sqrt((k * k).sum(-1, keepdims=True) + eps)
    qh, kh = q / nq, k / nk
    # forward: states at chunk starts
    starts = list(range(0, L, C))
    S = np.zeros((K, V)) if initial_state is None else np.array(initial_state, np.float64)
    S_at = []
    per = []
    for s in starts:
        e = min(L, s + C)
        c = e - s
        G = np.cumsum(g[s:e], axis=0)
        E = np.exp(np.where(np.tril(np.ones((c, c)))[:, :, None] > 0,
                            G[:, None, :] - G[None, :, :], -np.inf))
        Kq = np.einsum("rc,ic,ric->ri", qh[s:e], kh[s:e], E)
        Kk = np.einsum("rc,ic,ric->ri", kh[s:e], kh[s:e], E) * np.tril(np.ones((c, c)), -1)
        M = Kq * np.tril(np.ones((c, c)))
        T = np.linalg.inv(np.eye(c) + beta[s:e, None] * Kk)
        Tb = T * beta[s:e][None, :]
        eG = np.exp(G)
        Qt, Kt = qh[s:e] * eG, kh[s:e] * eG
        Kb = kh[s:e] * np.exp(G[-1][None, :] - G)
        D = np.exp(G[-1])
        X = v[s:e] - Kt @ S
        U = Tb @ X
        S_at.append(S)
        per.append(dict(s=s, e=e, c=c, G=G, E=E, Kk=Kk, M=M, T=T, Tb=Tb, eG=eG, Qt=Qt, Kt=Kt,
                        Kb=Kb, D=D, X=X, U=U))
        S = D[:, None] * S + Kb.T @ U
    dq_h = np.zeros_like(q)
    dk_h = np.zeros_like(k)
    dv = np.zeros_like(v)
    dg = np.zeros_like(g)
    dbeta = np.zeros_like(beta)
    dS = np.zeros((K, V)) if d_final_state is None else np.array(d_final_state, np.float64)
    for S0, P in reversed(list(zip(S_at, per))):
        s, e, c = P["s"], P["e"], P["c"]
        dO = do[s:e]
        dU = scale * P["M"].T @ dO + P["Kb"] @ dS
        dX = P["Tb"].T @ dU
        dv[s:e] = dX
        dQt = scale * dO @ S0.T
        dKt = -dX @ S0.T
        dKb = P["U"] @ dS.T
        dD = (dS * S0).sum(1)
        dM = scale * np.tril(dO @ P["U"].T)
        dTb = np.tril(dU @ P["X"].T)
        db = (dTb * P["T"]).sum(0)
        dT = dTb * beta[s:e][None, :]
        dA = np.tril(-P["T"].T @ dT @ P["T"].T, -1)
        db += (dA * P["Kk"]).sum(1)
        dKk = beta[s:e][:, None] * dA
        dbeta[s:e] = db
        E = P["E"]
        qs, ks = qh[s:e], kh[s:e]
        dqh = np.einsum("ri,ic,ric->rc", dM, ks, E)
        dkh = (np.einsum("ri,rc,ric->ic", dM, qs, E) + np.einsum("ri,rc,ric->ic", dKk, ks, E)
               + np.einsum("ri,ic,ric->rc", dKk, ks, E))
        W = (dM[:, :, None] * qs[:, None, :] + dKk[:, :, None] * ks[:, None, :]) * ks[None, :, :] * E
        dG = W.sum(1) - W.sum(0)
        dqh += dQt * P["eG"]
        dG += dQt * P["Qt"]
        dkh += dKt * P["eG"]
        dG += dKt * P["Kt"]
        eb = np.exp(P["G"][-1][None, :] - P["G"])
        dkh += dKb * eb
        dG -= dKb * P["Kb"]
        dG[-1] += (dKb * P["Kb"]).sum(0) + dD * P["D"]
        dg[s:e] = np.cumsum(dG[::-1], axis=0)[::-1]
        dq_h[s:e] = dqh
        dk_h[s:e] = dkh
        dS = P["D"][:, None] * dS + scale * P["Qt"].T @ dO - P["Kt"].T @ dX
    dq = (dq_h - qh * (qh * dq_h).sum(-1, keepdims=True)) / nq
    dk = (dk_h - kh * (kh * dk_h).sum(-1, keepdims=True)) / nk
    return dq, dk, dv, dg, dbeta, dS
