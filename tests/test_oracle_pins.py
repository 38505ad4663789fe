"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names the plausible mistake it would catch.  The recurrence is the
KDA delta rule the kda_fused page specialises (package docstring: K = V = 128,
q/k l2-normalised inside the kernel, bounded log gate, no initial or final
state, state reset at every packed-document boundary).
"""
import json
import os

import numpy as np
import pytest

import oracle
from chunk_model import chunk_document
from kda_workloads import make_inputs, one_hot_keys

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(T, H, K, V, seed, gate_scale=-5.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, K))
    k = rng.standard_normal((T, H, K))
    v = rng.standard_normal((T, H, V))
    g = gate_scale / (1.0 + np.exp(-rng.standard_normal((T, H, K))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, beta


# --------------------------------------------------------------------------
# hand-worked example (tests/golden): decay on key rows, decay before write,
# inclusive output, delta term sign and beta placement, all at once
# --------------------------------------------------------------------------

def test_hand_example_golden():
    with open(os.path.join(GOLDEN, "hand_example_k2_t3.json")) as f:
        ex = json.load(f)
    q = np.array(ex["q"], float)[:, None, :]
    k = np.array(ex["k"], float)[:, None, :]
    v = np.array(ex["v"], float)[:, None, :]
    g = np.log(np.array(ex["decay"], float))[:, None, :]
    beta = np.array(ex["beta"], float)[:, None]
    o = oracle.kda_document(q, k, v, g, beta, eps=ex["eps"])[:, 0, :]
    np.testing.assert_allclose(o, np.array(ex["expected_o"]), rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# T = 1 closed form: o = scale * beta * (qh . kh) v  (scale, l2 norm, eps,
# output taken after the write)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("K,V", [(128, 128), (5, 3)])
def test_single_token_closed_form(K, V):
    q, k, v, g, beta = _rand(1, 4, K, V, seed=1)
    o = oracle.kda_document(q, k, v, g, beta)
    eps = 1e-6
    qn = q / np.sqrt((q * q).sum(-1, keepdims=True) + eps)
    kn = k / np.sqrt((k * k).sum(-1, keepdims=True) + eps)
    expect = K ** -0.5 * beta[..., None] * (qn * kn).sum(-1, keepdims=True) * v
    np.testing.assert_allclose(o, expect, rtol=1e-13, atol=1e-15)


def test_l2norm_epsilon_reading():
    """q = c e_0 with c^2 comparable to eps: qh_0 = c / sqrt(c^2 + 1e-6)."""
    K = V = 4
    c = 1e-3
    q = np.zeros((1, 1, K)); q[0, 0, 0] = c
    k = np.zeros((1, 1, K)); k[0, 0, 0] = 1.0
    v = np.ones((1, 1, V))
    g = np.zeros((1, 1, K))
    beta = np.ones((1, 1))
    o = oracle.kda_document(q, k, v, g, beta)
    qh0 = c / np.sqrt(c * c + 1e-6)          # = 1/sqrt(2)
    kh0 = 1.0 / np.sqrt(1.0 + 1e-6)
    np.testing.assert_allclose(o[0, 0], K ** -0.5 * qh0 * kh0 * np.ones(V), rtol=1e-14)
    assert abs(qh0 - 2 ** -0.5) < 1e-15


def test_l2norm_epsilon_is_immaterial_at_workload_norms():
    """The pages give no epsilon for the in-kernel l2 norm.  At the workloads'
    norms (|x|^2 ~ 128 for N(0,1) rows) the reading eps = 1e-6 and eps = 0 give
    the same output to 1e-7 relative: the choice cannot move a parity result."""
    q, k, v, g, beta = _rand(40, 2, 128, 128, seed=12)
    o_eps = oracle.kda_document(q, k, v, g, beta, eps=1e-6)
    o_0 = oracle.kda_document(q, k, v, g, beta, eps=0.0)
    rel = np.linalg.norm(o_eps - o_0) / np.linalg.norm(o_0)
    assert 0.0 < rel < 1e-7, rel


# --------------------------------------------------------------------------
# beta = 0: nothing is ever written, the state stays zero (no initial state)
# --------------------------------------------------------------------------

def test_beta_zero_gives_zero():
    q, k, v, g, beta = _rand(37, 3, 8, 8, seed=2)
    o = oracle.kda_document(q, k, v, g, np.zeros_like(beta))
    assert np.all(o == 0.0)


# --------------------------------------------------------------------------
# g = 0, beta = 1, orthonormal keys: the delta rule reduces to causal linear
# attention o_t = scale * sum_{i<=t} (kh_i . qh_t) v_i
# --------------------------------------------------------------------------

def test_orthonormal_keys_reduce_to_linear_attention():
    K, V, T = 16, 7, 12
    rng = np.random.default_rng(3)
    Qm, _ = np.linalg.qr(rng.standard_normal((K, K)))
    k = (Qm[:, :T].T * rng.uniform(0.5, 3.0, size=(T, 1)))[:, None, :]
    q = rng.standard_normal((T, 1, K))
    v = rng.standard_normal((T, 1, V))
    g = np.zeros((T, 1, K))
    beta = np.ones((T, 1))
    o = oracle.kda_document(q, k, v, g, beta, eps=0.0)[:, 0]
    kn = k[:, 0] / np.linalg.norm(k[:, 0], axis=-1, keepdims=True)
    qn = q[:, 0] / np.linalg.norm(q[:, 0], axis=-1, keepdims=True)
    scores = np.tril(qn @ kn.T)
    np.testing.assert_allclose(o, K ** -0.5 * scores @ v[:, 0], rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# one-hot keys on distinct channels c_i, beta = 1: the write of token i sits in
# row c_i and decays by g_{j, c_i} for j = i+1..t only (decay acts on key
# channels, and is applied before the token's own write)
# --------------------------------------------------------------------------

def test_one_hot_distinct_channels_closed_form():
    K, V, T = 12, 5, 9
    rng = np.random.default_rng(4)
    ch = rng.permutation(K)[:T]
    k = np.zeros((T, 1, K)); k[np.arange(T), 0, ch] = rng.uniform(0.5, 2.0, T)
    q = rng.standard_normal((T, 1, K))
    v = rng.standard_normal((T, 1, V))
    g = -3.0 * rng.uniform(0, 1, (T, 1, K))
    beta = np.ones((T, 1))
    o = oracle.kda_document(q, k, v, g, beta, eps=0.0)[:, 0]
    qn = q[:, 0] / np.linalg.norm(q[:, 0], axis=-1, keepdims=True)
    expect = np.zeros((T, V))
    for t in range(T):
        for i in range(t + 1):
            c = ch[i]
            decay = np.exp(g[i + 1:t + 1, 0, c].sum())
            expect[t] += qn[t, c] * decay * v[i, 0]
    np.testing.assert_allclose(o, K ** -0.5 * expect, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# the same one-hot key repeated with beta in (0,1): row c follows the scalar
# recurrence s_t = (1 - beta_t) a_t s_{t-1} + beta_t v_t, other rows stay 0
# (sign of the delta term, where beta enters)
# --------------------------------------------------------------------------

def test_repeated_key_scalar_recurrence():
    K, V, T, c = 6, 4, 15, 2
    rng = np.random.default_rng(5)
    k = np.zeros((T, 1, K)); k[:, 0, c] = rng.uniform(0.3, 2.0, T)
    q = rng.standard_normal((T, 1, K))
    v = rng.standard_normal((T, 1, V))
    g = -rng.uniform(0, 2, (T, 1, K))
    beta = rng.uniform(0.05, 0.95, (T, 1))
    o = oracle.kda_document(q, k, v, g, beta, eps=0.0)[:, 0]
    qn = q[:, 0] / np.linalg.norm(q[:, 0], axis=-1, keepdims=True)
    s = np.zeros(V)
    for t in range(T):
        s = (1 - beta[t, 0]) * np.exp(g[t, 0, c]) * s + beta[t, 0] * v[t, 0]
        np.testing.assert_allclose(o[t], K ** -0.5 * qn[t, c] * s, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------
# brute force: S_t = sum_{i<=t} (P_t ... P_{i+1}) beta_i kh_i v_i^T with
# P_j = (I - beta_j kh_j kh_j^T) Diag(exp(g_j)) as explicit K x K matrices
# --------------------------------------------------------------------------

@pytest.mark.parametrize("K,V,T", [(4, 4, 6), (4, 3, 6), (3, 5, 5), (128, 128, 3)])
def test_brute_force_transition_products(K, V, T):
    q, k, v, g, beta = _rand(T, 1, K, V, seed=6 + K + V)
    eps = 1e-6
    o = oracle.kda_document(q, k, v, g, beta)[:, 0]
    kn = k[:, 0] / np.sqrt((k[:, 0] ** 2).sum(-1, keepdims=True) + eps)
    qn = q[:, 0] / np.sqrt((q[:, 0] ** 2).sum(-1, keepdims=True) + eps)
    P = [(np.eye(K) - beta[j, 0] * np.outer(kn[j], kn[j])) @ np.diag(np.exp(g[j, 0]))
         for j in range(T)]
    for t in range(T):
        St = np.zeros((K, V))
        for i in range(t + 1):
            prod = np.eye(K)
            for j in range(t, i, -1):
                prod = prod @ P[j]
            St += prod @ (beta[i, 0] * np.outer(kn[i], v[i, 0]))
        np.testing.assert_allclose(o[t], K ** -0.5 * St.T @ qn[t], rtol=1e-11, atol=1e-13)


# --------------------------------------------------------------------------
# packing: a packed stream equals its documents run separately (state reset
# at every boundary, offsets); zero-length documents are allowed
# --------------------------------------------------------------------------

def test_packed_equals_separate_documents():
    lengths = [5, 0, 1, 17, 0, 9]
    T = sum(lengths)
    q, k, v, g, beta = _rand(T, 2, 8, 6, seed=7)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    o = oracle.kda_forward(q, k, v, g, beta, cu)
    a = 0
    for L in lengths:
        if L:
            np.testing.assert_array_equal(
                o[a:a + L], oracle.kda_document(q[a:a + L], k[a:a + L], v[a:a + L],
                                                g[a:a + L], beta[a:a + L]))
        a += L
    # and it is NOT the single-document answer (the reset matters)
    o_single = oracle.kda_forward(q, k, v, g, beta, None)
    assert np.abs(o[5:] - o_single[5:]).max() > 1e-6


def test_cu_seqlens_reading():
    assert oracle.document_bounds(None, 7) == [(0, 7)]
    assert oracle.document_bounds([0, 3, 3, 7], 7) == [(0, 3), (3, 3), (3, 7)]
    # the list ends at the first entry equal to T
    assert oracle.document_bounds([0, 7, 7, 7], 7) == [(0, 7)]
    for bad in ([1, 7], [0, 4, 2, 7], [0, 3], [0, 8]):
        with pytest.raises(ValueError):
            oracle.document_bounds(bad, 7)


# --------------------------------------------------------------------------
# invariants: linear in v; q, k scale-free (eps = 0); head permutation
# equivariance; a document does not depend on its neighbours or its offset
# --------------------------------------------------------------------------

def test_invariants():
    q, k, v, g, beta = _rand(21, 3, 8, 8, seed=8)
    v2 = np.random.default_rng(9).standard_normal(v.shape)
    o1 = oracle.kda_document(q, k, v, g, beta)
    o2 = oracle.kda_document(q, k, v2, g, beta)
    o12 = oracle.kda_document(q, k, 2.0 * v - 3.0 * v2, g, beta)
    np.testing.assert_allclose(o12, 2 * o1 - 3 * o2, rtol=1e-11, atol=1e-12)
    a = oracle.kda_document(q, k, v, g, beta, eps=0.0)
    b = oracle.kda_document(7.0 * q, 0.25 * k, v, g, beta, eps=0.0)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)
    perm = [2, 0, 1]
    c = oracle.kda_document(q[:, perm], k[:, perm], v[:, perm], g[:, perm], beta[:, perm])
    np.testing.assert_array_equal(c, o1[:, perm])


def test_state_norm_bound():
    """||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t|| (||kh|| <= 1, beta in [0,1], decay <= 1),
    checked through the output bound |o_t| <= scale * ||S_t||_2 <= scale * sum beta_i ||v_i||."""
    q, k, v, g, beta = _rand(50, 2, 8, 8, seed=10, gate_scale=-0.01)
    o = oracle.kda_document(q, k, v, g, beta)
    bound = np.cumsum(beta[..., None] * np.linalg.norm(v, axis=-1, keepdims=True), axis=0)
    assert np.all(np.linalg.norm(o, axis=-1, keepdims=True) <= 8 ** -0.5 * bound + 1e-12)


# --------------------------------------------------------------------------
# the chunked form (the algebra the HIP kernels implement) equals the oracle
# --------------------------------------------------------------------------

@pytest.mark.parametrize("C", [1, 16, 64])
@pytest.mark.parametrize("gate_scale", [-5.5, -0.05, 0.0])
def test_chunk_form_matches_oracle(C, gate_scale):
    T, K, V = 150, 16, 12          # two full 64-chunks and a ragged tail
    q, k, v, g, beta = _rand(T, 1, K, V, seed=11)
    if gate_scale == -5.5:
        g = np.full_like(g, -5.5)  # every token at the bound
    else:
        g = g * (gate_scale / -5.0)
    o = oracle.kda_document(q, k, v, g, beta)[:, 0]
    oc = chunk_document(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], C=C)
    np.testing.assert_allclose(oc, o, rtol=1e-9, atol=1e-10)


def test_chunk_form_full_head_dim():
    inp = make_inputs(200, 1, 12, [0, 200])
    inp.k[:] = one_hot_keys(200, 1, 12)
    o = oracle.kda_document(inp.q, inp.k, inp.v, inp.g, inp.beta)[:, 0]
    oc = chunk_document(inp.q[:, 0], inp.k[:, 0], inp.v[:, 0], inp.g[:, 0], inp.beta[:, 0])
    np.testing.assert_allclose(oc, o, rtol=1e-9, atol=1e-10)


# --------------------------------------------------------------------------
# initial / final state (the state-carrying variant: document d starts from
# S_0 = initial_state[d] and returns its last state)
# --------------------------------------------------------------------------

def _state(H, K, V, seed, std=0.5):
    return std * np.random.default_rng(seed).standard_normal((H, K, V))


def test_state_beta_zero_closed_form():
    """beta = 0: nothing is written, so S_t = Diag(exp(G_t)) S_0 with G_t the
    inclusive cumsum of g, and o_t = scale * S_0^T (qh_t * exp(G_t)).  Catches a
    decay applied to the wrong axis of S_0, one token late or not at all, and
    S_0 entering transposed."""
    T, H, K, V = 9, 2, 6, 4
    q, k, v, g, beta = _rand(T, H, K, V, seed=31, gate_scale=-0.7)
    beta[:] = 0.0
    s0 = _state(H, K, V, 32)
    o, sT = oracle.kda_document(q, k, v, g, beta, initial_state=s0, final_state=True)
    G = np.cumsum(g, axis=0)                                    # [T, H, K]
    qn = q / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6)
    for t in range(T):
        for h in range(H):
            np.testing.assert_allclose(o[t, h], K ** -0.5 * s0[h].T @ (qn[t, h] * np.exp(G[t, h])),
                                       rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sT, np.exp(G[-1])[:, :, None] * s0, rtol=1e-12, atol=1e-14)


def test_state_unit_beta_writes_value():
    """beta_t = 1 and ||kh_t|| = 1: the write replaces the state's value along
    kh_t, so S_t^T kh_t = v_t whatever S_0 and the history were; with q_t = k_t
    the output is scale * v_t (eps = 0 keeps ||kh|| exactly 1)."""
    T, H, K, V = 7, 3, 8, 5
    q, k, v, g, beta = _rand(T, H, K, V, seed=33, gate_scale=-0.3)
    beta[-1] = 1.0
    q[-1] = 3.0 * k[-1]
    s0 = _state(H, K, V, 34, std=2.0)
    o, sT = oracle.kda_document(q, k, v, g, beta, eps=0.0, initial_state=s0, final_state=True)
    kn = k[-1] / np.linalg.norm(k[-1], axis=-1, keepdims=True)
    np.testing.assert_allclose(np.einsum("hkv,hk->hv", sT, kn), v[-1], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(o[-1], K ** -0.5 * v[-1], rtol=1e-11, atol=1e-12)


def test_state_segment_composition():
    """Running [0, L) equals running [0, a) and then [a, L) from the state the
    first part returned, for every cut a (the recurrence is a semigroup); a
    zero-length document returns its initial state."""
    T, H, K, V = 23, 2, 8, 6
    q, k, v, g, beta = _rand(T, H, K, V, seed=35, gate_scale=-0.4)
    s0 = _state(H, K, V, 36)
    o, sT = oracle.kda_document(q, k, v, g, beta, initial_state=s0, final_state=True)
    for a in (0, 1, 11, 22, 23):
        o1, s1 = oracle.kda_document(q[:a], k[:a], v[:a], g[:a], beta[:a], initial_state=s0,
                                     final_state=True)
        o2, s2 = oracle.kda_document(q[a:], k[a:], v[a:], g[a:], beta[a:], initial_state=s1,
                                     final_state=True)
        np.testing.assert_allclose(np.concatenate([o1, o2]), o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(s2, sT, rtol=1e-12, atol=1e-13)
    _, s_empty = oracle.kda_document(q[:0], k[:0], v[:0], g[:0], beta[:0], initial_state=s0,
                                     final_state=True)
    np.testing.assert_array_equal(s_empty, s0)


def test_state_linearity():
    """o and the last state are jointly linear in (S_0, v): a state that is
    added after the decay, or scaled by beta, breaks one of the two checks
    together with the closed form above."""
    T, H, K, V = 15, 2, 6, 6
    q, k, v, g, beta = _rand(T, H, K, V, seed=37, gate_scale=-0.2)
    s0 = _state(H, K, V, 38)
    o, sT = oracle.kda_document(q, k, v, g, beta, initial_state=s0, final_state=True)
    o_v, s_v = oracle.kda_document(q, k, v, g, beta, final_state=True)
    o_s, s_s = oracle.kda_document(q, k, 0 * v, g, beta, initial_state=s0, final_state=True)
    np.testing.assert_allclose(o, o_v + o_s, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(sT, s_v + s_s, rtol=1e-11, atol=1e-12)
    assert np.abs(o_s).max() > 1e-3          # the state reaches the output


def test_state_packed_exact_reading():
    """With states, every cu_seqlens entry delimits a document (trailing empty
    documents included) and document d starts from initial_state[d]."""
    lengths = [6, 0, 10, 3, 0]
    T = sum(lengths)
    H, K, V = 2, 6, 5
    q, k, v, g, beta = _rand(T, H, K, V, seed=39, gate_scale=-0.5)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    s0 = np.stack([_state(H, K, V, 40 + d) for d in range(len(lengths))])
    o, fin = oracle.kda_forward(q, k, v, g, beta, cu, initial_state=s0, output_final_state=True)
    assert fin.shape == (len(lengths), H, K, V)
    a = 0
    for d, L in enumerate(lengths):
        od, sd = oracle.kda_document(q[a:a + L], k[a:a + L], v[a:a + L], g[a:a + L],
                                     beta[a:a + L], initial_state=s0[d], final_state=True)
        np.testing.assert_array_equal(o[a:a + L], od)
        np.testing.assert_array_equal(fin[d], sd)
        a += L
    np.testing.assert_array_equal(fin[1], s0[1])
    np.testing.assert_array_equal(fin[4], s0[4])
    # zero initial state is the plain forward
    o0, _ = oracle.kda_forward(q, k, v, g, beta, cu, output_final_state=True)
    np.testing.assert_array_equal(o0, oracle.kda_forward(q, k, v, g, beta, cu))
    assert oracle.document_bounds([0, 3, 7, 7], 7, exact=True) == [(0, 3), (3, 7), (7, 7)]


@pytest.mark.parametrize("C", [16, 64])
def test_chunk_form_with_state_matches_oracle(C):
    """The chunked form with S_0 != 0 (the term e^G S_0 in X, O and the state
    carry) equals the token recurrence, over full chunks and a ragged tail."""
    T, K, V = 150, 16, 12
    q, k, v, g, beta = _rand(T, 1, K, V, seed=41, gate_scale=-0.05)
    s0 = _state(1, K, V, 42)
    o, sT = oracle.kda_document(q, k, v, g, beta, initial_state=s0, final_state=True)
    oc, sc = chunk_document(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], C=C,
                            initial_state=s0[0], final_state=True)
    np.testing.assert_allclose(oc, o[:, 0], rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(sc, sT[0], rtol=1e-9, atol=1e-10)
