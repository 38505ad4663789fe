"""The forward kernels' operand precisions, modelled on the CPU in fp64 with
explicit rounding (tests/chunk_model.py, kernel_precision_ops), against the
fp64 oracle.

The kernels keep X = V - Kt S, U = Tb X and Tb itself in fp16 behind an exact
power-of-two scale.  These tests fix why the scale has to work in both
directions: v and beta may be arbitrarily small (v is any bf16, beta any
finite value), and without scaling up, X, U and Tb fall into the fp16
subnormal range and lose their precision."""
import numpy as np
import pytest

import oracle
from chunk_model import chunk_document, kernel_precision_ops
from kda_workloads import make_inputs

REL_L2_TOL = 5e-3


def _case(v_scale, beta_scale, gate_scale=1.0, T=512, seed=3):
    inp = make_inputs(T, 1, seed=seed, cu_seqlens=np.array([0, T], np.int32))
    q, k = inp.q[:, 0], inp.k[:, 0]
    g = inp.g[:, 0] * gate_scale
    v = inp.v[:, 0] * v_scale
    beta = inp.beta[:, 0] * beta_scale
    ref = oracle.kda_document(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None])[:, 0]
    return (q, k, v, g, beta), ref


def _rel(args, ref, two_way):
    o = chunk_document(*args, ops=kernel_precision_ops(two_way))
    return np.linalg.norm(o - ref) / np.linalg.norm(ref)


@pytest.mark.parametrize("v_scale,beta_scale", [(1.0, 1.0), (1e-6, 1.0), (1.0, 1e-5),
                                                (1e-6, 1e-5), (2.0 ** 40, 1.0)])
def test_two_way_scaling_meets_the_bar_at_any_magnitude(v_scale, beta_scale):
    args, ref = _case(v_scale, beta_scale)
    rel = _rel(args, ref, two_way=True)
    assert rel < 1e-3, rel


def test_two_way_scaling_with_a_slowly_decaying_state():
    args, ref = _case(1e-6, 1e-5, gate_scale=0.01)
    assert _rel(args, ref, two_way=True) < 2e-3


@pytest.mark.parametrize("v_scale,beta_scale", [(1e-6, 1.0), (1e-6, 1e-5)])
def test_scaling_only_down_fails_on_small_inputs(v_scale, beta_scale):
    """What the scale guards against: with X and U only ever scaled down, the
    same inputs miss the parity bar."""
    args, ref = _case(v_scale, beta_scale)
    assert _rel(args, ref, two_way=False) > REL_L2_TOL
