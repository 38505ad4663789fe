"""fp64 CPU oracle for the Kimi Delta Attention (KDA) forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path; the only thing both sides share is the seeded input generator
(``kda_workloads``), which holds none of the method's arithmetic.

What it computes (page "nemo_automodel.components.models.kimi_k3.kda_fused",
package docstring and the ``fused_chunk_kda`` / ``fused_kda_unsupported_reason``
entries): the KDA delta rule, specialised to

* one recurrent state ``S`` of shape K x V per (document, head): it starts at
  zero in each document and is not returned (the package docstring, and the
  ``fused_chunk_kda`` entry, which resets the state at each packed-document
  boundary).
  The state-carrying variant starts each document from a given ``S_0`` and
  also returns its last state, the convention of FLA's ``chunk_kda``
  (``initial_state``, ``output_final_state``), of which ``fused_chunk_kda`` is
  the drop-in with the final state switched off (same page, ``fused_chunk_kda``
  entry).  ``S_0 = 0`` gives back the plain forward;
* q and k l2-normalised inside the operator (``use_qk_l2norm_in_kernel``);
* a log decay ``g`` per token, head and key channel, bounded below (the
  package docstring; the K3 model page's ``KimiKDAFp32Params`` returns an fp32
  ``[b, s, h, d]`` decay);
* packed documents delimited by int32 ``cu_seqlens``.

The pages print no formula for the recurrence.  The oracle takes the KDA
delta rule in its plain token-by-token form:

    S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
    o_t = K**-0.5 * S_t^T q_t

with k_t, q_t the l2-normalised vectors ``x / sqrt(sum(x*x) + eps)`` and
``eps = 1e-6``.  The output uses the state *after* token t's write.  The
second update line below is the same expression multiplied out:
``(I - b k k^T) D S + b k v^T = D S + b k (v - (D S)^T k)^T``.

Everything runs in fp64.  The caller passes the exact values the GPU path
receives (bf16 q, k, v widened exactly; fp32 g, beta widened exactly).
"""
from __future__ import annotations

import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

DEFAULT_EPS = 1e-6


def l2_normalise(x: np.ndarray, eps: float = DEFAULT_EPS) -> np.ndarray:
    """``x / sqrt(sum(x**2) + eps)`` over the last axis (in-kernel q/k l2 norm)."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def kda_document(q, k, v, g, beta, scale: float | None = None,
                 eps: float = DEFAULT_EPS, initial_state=None, final_state: bool = False):
    """Run one document, all given heads at once.

    q, k: [L, H, K]; v: [L, H, V]; g: [L, H, K]; beta: [L, H];
    initial_state: [H, K, V] (S_0 of every head, key channel first) or None
    for zeros.  Returns o: [L, H, V] in fp64, or ``(o, S_L)`` when
    ``final_state`` is set (S_L = S_0 for an empty document).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    L, H, K = q.shape
    V = v.shape[-1]
    if scale is None:
        scale = K ** -0.5
    qn = l2_normalise(q, eps)
    kn = l2_normalise(k, eps)
    if initial_state is None:
        S = np.zeros((H, K, V))
    else:
        S = np.array(initial_state, np.float64, copy=True).reshape(H, K, V)
    o = np.empty((L, H, V))
    for t in range(L):
        # Diag(exp(g_t)) S_{t-1}: the decay scales the rows of S (key channels)
        S *= np.exp(g[t])[:, :, None]
        kt = kn[t]                                           # [H, K]
        pred = np.matmul(kt[:, None, :], S)[:, 0, :]         # (D S)^T k  -> [H, V]
        S += beta[t][:, None, None] * kt[:, :, None] * (v[t] - pred)[:, None, :]
        o[t] = scale * np.matmul(qn[t][:, None, :], S)[:, 0, :]   # S_t^T q_t
    return (o, S) if final_state else o


def document_bounds(cu_seqlens, T: int, exact: bool = False) -> list[tuple[int, int]]:
    """Documents ``[cu[i], cu[i+1])`` of a packed stream (``None`` = one document).

    By default the list is read up to the first entry equal to T.  With
    ``exact`` every entry counts (N + 1 entries are N documents, the last
    entry must be T): the reading used when states are passed per document.
    Zero-length documents are kept (they produce no output)."""
    if cu_seqlens is None:
        return [(0, T)]
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    if not cu or cu[0] != 0:
        raise ValueError("cu_seqlens must start at 0")
    out = []
    for a, b in zip(cu[:-1], cu[1:]):
        if b < a or b > T:
            raise ValueError("cu_seqlens must be non-decreasing and end at T")
        out.append((a, b))
        if b == T and not exact:
            break
    if (out[-1][1] if out else 0) != T:
        raise ValueError("cu_seqlens must reach T")
    return out


def kda_forward(q, k, v, g, beta, cu_seqlens=None, scale: float | None = None,
                eps: float = DEFAULT_EPS, initial_state=None, output_final_state: bool = False):
    """Packed forward: q, k, g [T, H, K], v [T, H, V], beta [T, H] -> o [T, H, V] (fp64).

    With ``initial_state`` ([N, H, K, V], document d starts from
    ``initial_state[d]``) or ``output_final_state``, the N + 1 entries of
    ``cu_seqlens`` are read exactly and ``(o, final [N, H, K, V])`` is returned."""
    T = q.shape[0]
    o = np.zeros((T,) + tuple(v.shape[1:]))
    stateful = initial_state is not None or output_final_state
    bounds = document_bounds(cu_seqlens, T, exact=stateful)
    if not stateful:
        for a, b in bounds:
            if b > a:
                o[a:b] = kda_document(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], scale, eps)
        return o
    H, K, V = q.shape[1], q.shape[2], v.shape[2]
    final = np.zeros((len(bounds), H, K, V))
    for d, (a, b) in enumerate(bounds):
        s0 = None if initial_state is None else initial_state[d]
        o[a:b], final[d] = kda_document(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], scale, eps,
                                        initial_state=s0, final_state=True)
    return o, final


# ---------------------------------------------------------------------------
# task-parallel driver: independent (document, head-range) tasks on a process
# pool.  Inputs are inherited by the forked workers, not pickled.
# ---------------------------------------------------------------------------

_SHARED: dict = {}


def _worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:  # pragma: no cover
        pass


def _run_task(task):
    a, b, h0, h1 = task[:4]
    s = _SHARED
    init = s["initial_state"]
    s0 = None if init is None else init[task[4], h0:h1]
    res = kda_document(s["q"][a:b, h0:h1], s["k"][a:b, h0:h1], s["v"][a:b, h0:h1],
                       s["g"][a:b, h0:h1], s["beta"][a:b, h0:h1], s["scale"], s["eps"],
                       initial_state=s0, final_state=s["final_state"])
    return (task,) + (res if s["final_state"] else (res,))


def default_workers() -> int:
    """Worker processes for the task pools: the CPUs this process may use, at
    most 12.  Forked workers inherit the parent's open device handles, so when
    the caller has used a GPU every worker also counts as a process holding
    that device; the cap keeps that count small."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(12, n))


def kda_tasks(q, k, v, g, beta, tasks, workers: int | None = None,
              scale: float | None = None, eps: float = DEFAULT_EPS,
              initial_state=None, final_state: bool = False):
    """Yield ``((a, b, h0, h1), o)`` for each task: tokens [a, b) of one document,
    heads [h0, h1).  Tasks are run longest first on ``workers`` processes.

    With states, a task is ``(a, b, h0, h1, d)`` (d = document index into
    ``initial_state`` [N, H, K, V], or None for zeros) and, when
    ``final_state`` is set, ``(task, o, S_last)`` is yielded."""
    import multiprocessing as mp
    tasks = sorted(tasks, key=lambda t: -(t[1] - t[0]) * (t[3] - t[2]))
    workers = workers or default_workers()
    _SHARED.update(q=q, k=k, v=v, g=g, beta=beta, scale=scale, eps=eps,
                   initial_state=initial_state, final_state=final_state)
    try:
        if workers <= 1 or len(tasks) <= 1:
            for t in tasks:
                yield _run_task(t)
            return
        env_keep = {x: os.environ.get(x) for x in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")}
        os.environ["OMP_NUM_THREADS"] = "1"
        os.environ["OPENBLAS_NUM_THREADS"] = "1"
        try:
            ctx = mp.get_context("fork")
            with ProcessPoolExecutor(workers, mp_context=ctx, initializer=_worker_init) as ex:
                for r in ex.map(_run_task, tasks, chunksize=1):
                    yield r
        finally:
            for key, val in env_keep.items():
                if val is None:
                    os.environ.pop(key, None)
                else:
                    os.environ[key] = val
    finally:
        _SHARED.clear()
