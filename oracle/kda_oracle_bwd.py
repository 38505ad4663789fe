"""fp64 CPU oracle for the gradients of the KDA forward.

TEST INFRASTRUCTURE ONLY, like ``kda_oracle``: only ``tests/`` use it.  It
shares no code with the HIP path.

What it computes: the gradients of ``L = sum_t <o_t, do_t> + <S_L, dS_L>``
with respect to q, k, v, g, beta and the initial state S_0, where o and S_L are
the outputs of the oracle's token recurrence (``kda_oracle.kda_document``).
The backward of the pages' fused forward (page "nemo_automodel.components.
models.kimi_k3.kda_fused", package docstring: a backward kernel that
recomputes every intermediate from q, k, v, g, beta and cu_seqlens) computes
these same gradients.

How: the token recurrence is written once more with torch fp64 CPU tensors
and differentiated by torch.autograd (a library primitive; no hand-derived
gradient formula appears here).  The recurrence is identical to the numpy
oracle's, which a test checks value for value.  Long documents are processed
in segments (checkpointing): the forward states at the segment starts come
from the numpy oracle, and each segment is differentiated on its own with the
state gradient handed from the segment after it.  That is the chain rule
applied at the segment boundary, so the result is the same up to fp64
rounding.
"""
from __future__ import annotations

import numpy as np

from .kda_oracle import DEFAULT_EPS, kda_document

SEGMENT = 256


def _torch():
    import torch
    return torch


def forward_torch(q, k, v, g, beta, s0, scale: float, eps: float):
    """The token recurrence on torch fp64 tensors (differentiable).

    q, k, g: [L, H, K]; v: [L, H, V]; beta: [L, H]; s0: [H, K, V].
    Returns (o [L, H, V], S_L [H, K, V])."""
    torch = _torch()
    qn = q / torch.sqrt((q * q).sum(-1, keepdim=True) + eps)
    kn = k / torch.sqrt((k * k).sum(-1, keepdim=True) + eps)
    S = s0
    outs = []
    for t in range(q.shape[0]):
        S = S * torch.exp(g[t])[:, :, None]                      # Diag(exp g_t) S
        pred = torch.einsum("hk,hkv->hv", kn[t], S)              # (D S)^T k
        S = S + beta[t][:, None, None] * kn[t][:, :, None] * (v[t] - pred)[:, None, :]
        outs.append(scale * torch.einsum("hk,hkv->hv", qn[t], S))
    o = torch.stack(outs) if outs else q.new_zeros((0,) + tuple(v.shape[1:]))
    return o, S


def kda_document_backward(q, k, v, g, beta, do, initial_state=None, d_final_state=None,
                          scale: float | None = None, eps: float = DEFAULT_EPS,
                          segment: int = SEGMENT):
    """Gradients of one document, all given heads at once.

    q, k, g: [L, H, K]; v, do: [L, H, V]; beta: [L, H]; initial_state,
    d_final_state: [H, K, V] or None (zero).  Returns a dict of fp64 arrays
    dq, dk, dv, dg (shapes of the inputs), dbeta [L, H] and dh0 [H, K, V]."""
    torch = _torch()
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    do = np.asarray(do, np.float64)
    L, H, K = q.shape
    V = v.shape[-1]
    if scale is None:
        scale = K ** -0.5
    s0 = np.zeros((H, K, V)) if initial_state is None else np.asarray(initial_state, np.float64)
    # forward states at the segment starts (numpy oracle)
    starts = list(range(0, L, segment)) or [0]
    states = [s0]
    for a in starts[:-1]:
        b = a + segment
        _, s = kda_document(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], scale, eps,
                            initial_state=states[-1], final_state=True)
        states.append(s)
    grads = {name: np.zeros_like(x) for name, x in
             (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("dbeta", beta))}
    dS = np.zeros((H, K, V)) if d_final_state is None else np.asarray(d_final_state, np.float64)
    for a, s_a in reversed(list(zip(starts, states))):
        b = min(L, a + segment)
        ts = [torch.tensor(x[a:b], dtype=torch.float64, requires_grad=True)
              for x in (q, k, v, g, beta)]
        st = torch.tensor(s_a, dtype=torch.float64, requires_grad=True)
        o, s_end = forward_torch(*ts, st, scale, eps)
        loss = (o * torch.tensor(do[a:b])).sum() + (s_end * torch.tensor(dS)).sum()
        gs = torch.autograd.grad(loss, ts + [st], allow_unused=True)
        for name, gr, x in zip(("dq", "dk", "dv", "dg", "dbeta"), gs[:5], ts):
            if gr is not None:
                grads[name][a:b] = gr.numpy()
        dS = gs[5].numpy() if gs[5] is not None else np.zeros((H, K, V))
    grads["dh0"] = dS
    return grads


def kda_backward(q, k, v, g, beta, do, cu_seqlens, initial_state=None, d_final_state=None,
                 scale: float | None = None, eps: float = DEFAULT_EPS):
    """Packed gradients: every document of ``cu_seqlens`` (read exactly, N + 1
    entries) from ``initial_state[d]`` (or zero) with ``d_final_state[d]``
    (or zero).  Returns dq, dk, dv, dg [T, ...], dbeta [T, H], dh0 [N, H, K, V]."""
    from .kda_oracle import document_bounds
    T, H, K = q.shape
    V = v.shape[-1]
    bounds = document_bounds(cu_seqlens, T, exact=True)
    out = {name: np.zeros(np.shape(x), np.float64) for name, x in
           (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("dbeta", beta))}
    out["dh0"] = np.zeros((len(bounds), H, K, V))
    for d, (a, b) in enumerate(bounds):
        r = kda_document_backward(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], do[a:b],
                                  None if initial_state is None else initial_state[d],
                                  None if d_final_state is None else d_final_state[d],
                                  scale, eps)
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            out[name][a:b] = r[name]
        out["dh0"][d] = r["dh0"]
    return out


# ---------------------------------------------------------------------------
# task-parallel driver: independent (document, head-range) tasks on a fork
# pool, like kda_oracle.kda_tasks
# ---------------------------------------------------------------------------

_SHARED: dict = {}


def _worker_init(shared=None):
    import torch
    torch.set_num_threads(1)
    if shared is not None:
        _SHARED.update(shared)


def _run_task(task):
    a, b, h0, h1, d = task
    s = _SHARED
    init = s["initial_state"]
    dfin = s["d_final_state"]
    r = kda_document_backward(s["q"][a:b, h0:h1], s["k"][a:b, h0:h1], s["v"][a:b, h0:h1],
                              s["g"][a:b, h0:h1], s["beta"][a:b, h0:h1], s["do"][a:b, h0:h1],
                              None if init is None else init[d, h0:h1],
                              None if dfin is None else dfin[d, h0:h1])
    return task, r


def kda_backward_tasks(q, k, v, g, beta, do, tasks, initial_state=None, d_final_state=None,
                       workers: int | None = None):
    """Yield ``(task, grads)`` for tasks ``(a, b, h0, h1, d)``: tokens [a, b) of
    document d, heads [h0, h1).  Longest first, on ``workers`` processes.

    The workers are spawned (not forked): autograd cannot run in a process
    forked from one that has used it, and the caller may have."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    from .kda_oracle import default_workers
    tasks = sorted(tasks, key=lambda t: -(t[1] - t[0]) * (t[3] - t[2]))
    workers = min(workers or default_workers(), len(tasks))
    shared = dict(q=q, k=k, v=v, g=g, beta=beta, do=do, initial_state=initial_state,
                  d_final_state=d_final_state)
    if workers <= 1:
        _SHARED.update(shared)
        try:
            for t in tasks:
                yield _run_task(t)
        finally:
            _SHARED.clear()
        return
    with ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn"),
                             initializer=_worker_init, initargs=(shared,)) as ex:
        for r in ex.map(_run_task, tasks, chunksize=1):
            yield r
