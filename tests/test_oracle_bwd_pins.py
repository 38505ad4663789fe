"""Pins of the backward oracle (oracle/kda_oracle_bwd.py) against facts that do
not come from it: central finite differences of the numpy forward oracle,
closed forms, and the chunked backward derived by hand (tests/chunk_model.py),
which the GPU kernels implement."""
import numpy as np
import pytest

import oracle
from chunk_model import chunk_document_backward
from oracle.kda_oracle_bwd import forward_torch, kda_backward, kda_document_backward


def _rand(T, H, K, V, seed, gate_scale=-0.5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, K))
    k = rng.standard_normal((T, H, K))
    v = rng.standard_normal((T, H, V))
    g = gate_scale / (1.0 + np.exp(-rng.standard_normal((T, H, K))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    do = rng.standard_normal((T, H, V))
    s0 = 0.4 * rng.standard_normal((H, K, V))
    dsl = rng.standard_normal((H, K, V))
    return q, k, v, g, beta, do, s0, dsl


def _loss(q, k, v, g, beta, do, s0, dsl):
    o, s = oracle.kda_document(q, k, v, g, beta, initial_state=s0, final_state=True)
    return float((o * do).sum() + (s * dsl).sum())


def test_torch_recurrence_equals_the_numpy_oracle():
    import torch
    q, k, v, g, beta, do, s0, dsl = _rand(9, 2, 6, 5, seed=1)
    o_ref, s_ref = oracle.kda_document(q, k, v, g, beta, initial_state=s0, final_state=True)
    o, s = forward_torch(*(torch.tensor(x) for x in (q, k, v, g, beta, s0)), 6 ** -0.5, 1e-6)
    np.testing.assert_allclose(o.numpy(), o_ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(s.numpy(), s_ref, rtol=1e-13, atol=1e-14)


def test_gradients_equal_central_differences():
    """Every element of every input, against (L(x+h) - L(x-h)) / 2h of the
    numpy forward oracle: catches any mistake in the differentiated program."""
    q, k, v, g, beta, do, s0, dsl = _rand(5, 1, 4, 3, seed=2)
    r = kda_document_backward(q, k, v, g, beta, do, s0, dsl)
    args = [q, k, v, g, beta, do, s0, dsl]
    h = 1e-6
    for idx, name in ((0, "dq"), (1, "dk"), (2, "dv"), (3, "dg"), (4, "dbeta"), (6, "dh0")):
        x = args[idx]
        fd = np.zeros_like(x)
        for j in np.ndindex(x.shape):
            xp = x.copy()
            xp[j] += h
            xm = x.copy()
            xm[j] -= h
            ap = list(args)
            ap[idx] = xp
            am = list(args)
            am[idx] = xm
            fd[j] = (_loss(*ap) - _loss(*am)) / (2 * h)
        np.testing.assert_allclose(r[name], fd, rtol=1e-6, atol=1e-8, err_msg=name)


def test_segmented_backward_equals_one_segment():
    q, k, v, g, beta, do, s0, dsl = _rand(23, 2, 5, 4, seed=3)
    a = kda_document_backward(q, k, v, g, beta, do, s0, dsl, segment=1000)
    b = kda_document_backward(q, k, v, g, beta, do, s0, dsl, segment=3)
    for name in a:
        np.testing.assert_allclose(b[name], a[name], rtol=1e-12, atol=1e-13, err_msg=name)


def test_single_token_closed_form():
    """T = 1, S_0 = 0: o = scale beta (qh . kh) v, so dv = scale beta (qh . kh) do,
    dbeta = scale (qh . kh) (v . do), and the gate has no effect (dg = 0)."""
    q, k, v, g, beta, do, _, _ = _rand(1, 3, 7, 5, seed=4)
    r = kda_document_backward(q, k, v, g, beta, do)
    qn = q / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6)
    kn = k / np.sqrt((k * k).sum(-1, keepdims=True) + 1e-6)
    c = (qn * kn).sum(-1)                                   # [1, H]
    scale = 7 ** -0.5
    np.testing.assert_allclose(r["dv"], scale * (beta * c)[..., None] * do, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["dbeta"], scale * c * (v * do).sum(-1), rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(r["dg"], np.zeros_like(g))
    # the state gradient of a zero-length document passes straight through
    _, _, _, _, _, _, _, dsl = _rand(1, 3, 7, 5, seed=5)
    e = kda_document_backward(q[:0], k[:0], v[:0], g[:0], beta[:0], do[:0], None, dsl)
    np.testing.assert_array_equal(e["dh0"], dsl)


@pytest.mark.parametrize("C", [16, 64])
@pytest.mark.parametrize("gate_scale", [-5.5, -0.05, 0.0])
def test_chunked_backward_matches_the_oracle(C, gate_scale):
    """The hand-derived chunked backward (what the GPU computes) equals the
    autograd oracle over full chunks and a ragged tail, with S_0 and dS_L."""
    L, K, V = 150, 8, 6
    q, k, v, g, beta, do, s0, dsl = _rand(L, 1, K, V, seed=6)
    if gate_scale == -5.5:
        g = np.full_like(g, -5.5)
    else:
        g = g * (gate_scale / -0.5)
    r = kda_document_backward(q, k, v, g, beta, do, s0, dsl)
    c = chunk_document_backward(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], do[:, 0], C=C,
                                initial_state=s0[0], d_final_state=dsl[0])
    for name, got in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), c):
        ref = r[name][:, 0] if name != "dh0" else r[name][0]
        np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-10, err_msg=name)


def test_packed_backward_is_per_document():
    lengths = [7, 0, 12, 3]
    T = sum(lengths)
    q, k, v, g, beta, do, _, _ = _rand(T, 2, 5, 4, seed=7)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    s0 = 0.3 * np.random.default_rng(8).standard_normal((len(lengths), 2, 5, 4))
    dsl = np.random.default_rng(9).standard_normal((len(lengths), 2, 5, 4))
    r = kda_backward(q, k, v, g, beta, do, cu, s0, dsl)
    a = 0
    for d, L in enumerate(lengths):
        rd = kda_document_backward(q[a:a + L], k[a:a + L], v[a:a + L], g[a:a + L],
                                   beta[a:a + L], do[a:a + L], s0[d], dsl[d])
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            np.testing.assert_array_equal(r[name][a:a + L], rd[name])
        np.testing.assert_array_equal(r["dh0"][d], rd["dh0"])
        a += L
    np.testing.assert_array_equal(r["dh0"][1], dsl[1])
