"""Pins of the oracle's task-parallel drivers (``oracle.kda_tasks`` and
``oracle.kda_backward_tasks``), through which every GPU parity test gets its
reference values.

A driver runs (document, head-range) tasks longest first on worker processes
and hands back each task's slice of the result.  The pins below run them with
several workers on shuffled tasks of mixed head ranges, per-document initial
states and final states, and require each task's values to equal, bit for
bit, the same slice of the packed oracle (``kda_forward`` / ``kda_backward``)
run in this process.  That fixes the head-range slicing, the indexing of
``initial_state[d]``, the final state and the order of the results after the
longest-first sort.  The packing contract they rely on (each document starts
from its own state; page "nemo_automodel.components.models.kimi_k3.kda_fused",
``fused_chunk_kda`` entry) is pinned separately by the packing tests of the
oracle itself."""
import random

import numpy as np

import oracle
from oracle.kda_oracle_bwd import kda_backward, kda_backward_tasks


def _inputs(T, H, K, V, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, K))
    k = rng.standard_normal((T, H, K))
    v = rng.standard_normal((T, H, V))
    g = -0.3 / (1.0 + np.exp(-rng.standard_normal((T, H, K))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, beta


# documents of different lengths, one empty, so that the longest-first order
# differs from the cu_seqlens order
CU = np.array([0, 7, 7, 30, 41, 60], np.int64)
HEAD_RANGES = [(0, 1), (1, 4), (4, 5), (0, 5)]


def _tasks(cu, with_doc):
    out = []
    for d, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        for h0, h1 in HEAD_RANGES:
            out.append((int(a), int(b), h0, h1, d) if with_doc else (int(a), int(b), h0, h1))
    random.Random(5).shuffle(out)
    return out


def test_forward_tasks_equal_the_packed_oracle_task_for_task():
    T, H, K, V = int(CU[-1]), 5, 8, 6
    q, k, v, g, beta = _inputs(T, H, K, V, seed=1)
    ref = oracle.kda_forward(q, k, v, g, beta, CU)
    tasks = _tasks(CU, with_doc=False)
    seen = []
    for task, o in oracle.kda_tasks(q, k, v, g, beta, tasks, workers=3):
        a, b, h0, h1 = task
        assert o.shape == (b - a, h1 - h0, V)
        assert np.array_equal(o, ref[a:b, h0:h1]), task
        seen.append(task)
    assert sorted(seen) == sorted(tasks)
    # results arrive longest (tokens x heads) first
    work = [(b - a) * (h1 - h0) for a, b, h0, h1 in seen]
    assert work == sorted(work, reverse=True)


def test_forward_tasks_with_states_equal_the_packed_oracle_task_for_task():
    T, H, K, V = int(CU[-1]), 5, 8, 6
    q, k, v, g, beta = _inputs(T, H, K, V, seed=2)
    n_docs = len(CU) - 1
    s0 = 0.3 * np.random.default_rng(3).standard_normal((n_docs, H, K, V))
    ref_o, ref_s = oracle.kda_forward(q, k, v, g, beta, CU, initial_state=s0,
                                      output_final_state=True)
    tasks = _tasks(CU, with_doc=True)
    seen = []
    for task, o, s_last in oracle.kda_tasks(q, k, v, g, beta, tasks, workers=3,
                                            initial_state=s0, final_state=True):
        a, b, h0, h1, d = task
        assert np.array_equal(o, ref_o[a:b, h0:h1]), task
        assert np.array_equal(s_last, ref_s[d, h0:h1]), task
        seen.append(task)
    assert sorted(seen) == sorted(tasks)
    # the empty document hands its initial state back unchanged
    for task, _, s_last in oracle.kda_tasks(q, k, v, g, beta, [(7, 7, 0, 5, 1)], workers=1,
                                            initial_state=s0, final_state=True):
        assert np.array_equal(s_last, s0[1])


def test_backward_tasks_equal_the_packed_oracle_task_for_task():
    cu = np.array([0, 5, 5, 14, 20], np.int64)
    T, H, K, V = int(cu[-1]), 3, 4, 3
    q, k, v, g, beta = _inputs(T, H, K, V, seed=4)
    rng = np.random.default_rng(6)
    do = rng.standard_normal((T, H, V))
    n_docs = len(cu) - 1
    s0 = 0.3 * rng.standard_normal((n_docs, H, K, V))
    dsl = rng.standard_normal((n_docs, H, K, V))
    ref = kda_backward(q, k, v, g, beta, do, cu, initial_state=s0, d_final_state=dsl)
    tasks = []
    for d, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        for h0, h1 in ((0, 1), (1, 3)):
            tasks.append((int(a), int(b), h0, h1, d))
    random.Random(7).shuffle(tasks)
    seen = []
    for task, r in kda_backward_tasks(q, k, v, g, beta, do, tasks, initial_state=s0,
                                      d_final_state=dsl, workers=2):
        a, b, h0, h1, d = task
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            assert np.array_equal(r[name], ref[name][a:b, h0:h1]), (task, name)
        assert np.array_equal(r["dh0"], ref["dh0"][d, h0:h1]), task
        seen.append(task)
    assert sorted(seen) == sorted(tasks)
