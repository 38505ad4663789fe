"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point that include/kda.h declares, and rejects bad arguments with
the documented status codes before touching the GPU."""
import ctypes
import os
import re

import pytest

import linear_attention_sequence_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "kda.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert _declared_functions() == ["kda_chunk_bwd", "kda_chunk_fwd", "kda_chunk_fwd_noalloc",
                                     "kda_chunk_fwd_state", "kda_debug_set_bwd_workspace_limit",
                                     "kda_debug_set_split_policy", "kda_device_status",
                                     "kda_last_error", "kda_recurrent_fwd"]


def test_library_exports_every_declared_symbol():
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so not built")
    lib = ctypes.CDLL(kda.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


# a plausible, 16-byte aligned fake address: never dereferenced because every
# call below fails validation first
P = 1 << 20


def _call(**kw):
    args = dict(q=P, k=P, v=P, g=P, beta=P, cu=None, T=128, H=2, chunk=64, gate_bound=-5.0,
                out=P, stream=None)
    args.update(kw)
    rc = kda.kda_chunk_fwd(args["q"], args["k"], args["v"], args["g"], args["beta"], args["cu"],
                           args["T"], args["H"], args["chunk"], args["gate_bound"], args["out"],
                           args["stream"])
    return rc, kda.kda_last_error()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(T=-1), kda.KDA_ERR_BAD_SHAPE, "T must be >= 0"),
    (dict(T=2**31), kda.KDA_ERR_BAD_SHAPE, "INT32_MAX"),
    (dict(H=0), kda.KDA_ERR_BAD_SHAPE, "H must be >= 1"),
    (dict(H=5000), kda.KDA_ERR_BAD_SHAPE, "KDA_MAX_HEADS"),
    (dict(q=None), kda.KDA_ERR_NULL_PTR, "q is NULL"),
    (dict(k=None), kda.KDA_ERR_NULL_PTR, "k is NULL"),
    (dict(v=None), kda.KDA_ERR_NULL_PTR, "v is NULL"),
    (dict(g=None), kda.KDA_ERR_NULL_PTR, "g is NULL"),
    (dict(beta=None), kda.KDA_ERR_NULL_PTR, "beta is NULL"),
    (dict(out=None), kda.KDA_ERR_NULL_PTR, "out is NULL"),
    (dict(chunk=32), kda.KDA_ERR_UNSUPPORTED, "chunk must be 64"),
    (dict(gate_bound=0.0), kda.KDA_ERR_UNSUPPORTED, "gate_bound"),
    (dict(gate_bound=-6.0), kda.KDA_ERR_UNSUPPORTED, "gate_bound"),
    (dict(gate_bound=float("nan")), kda.KDA_ERR_UNSUPPORTED, "gate_bound"),
    (dict(q=P + 8), kda.KDA_ERR_ALIGN, "q is not 16-byte aligned"),
    (dict(g=P + 4), kda.KDA_ERR_ALIGN, "g is not 16-byte aligned"),
    (dict(out=P + 2), kda.KDA_ERR_ALIGN, "out is not 16-byte aligned"),
    (dict(beta=P + 2), kda.KDA_ERR_ALIGN, "beta is not 4-byte aligned"),
    (dict(cu=P + 2), kda.KDA_ERR_ALIGN, "cu_seqlens is not 4-byte aligned"),
])
def test_argument_validation(kw, code, msg):
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so not built")
    rc, err = _call(**kw)
    assert rc == code
    assert msg in err


def test_first_violated_condition_is_reported():
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so not built")
    rc, err = _call(q=None, chunk=32, H=0)
    assert rc == kda.KDA_ERR_BAD_SHAPE and "H must be" in err
    rc, err = _call(q=None, chunk=32)
    assert rc == kda.KDA_ERR_NULL_PTR and "q is NULL" in err


def test_empty_stream_is_a_noop():
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so not built")
    rc, err = _call(T=0, q=None, k=None, v=None, g=None, beta=None, out=None)
    assert rc == kda.KDA_OK and err == ""


def _call_state(**kw):
    args = dict(q=P, k=P, v=P, g=P, beta=P, cu=None, n_docs=1, T=128, H=2, chunk=64,
                gate_bound=-5.0, h0=None, ht=P, out=P, stream=None)
    args.update(kw)
    rc = kda.kda_chunk_fwd_state(args["q"], args["k"], args["v"], args["g"], args["beta"],
                                 args["cu"], args["n_docs"], args["T"], args["H"], args["chunk"],
                                 args["gate_bound"], args["h0"], args["ht"], args["out"],
                                 args["stream"])
    return rc, kda.kda_last_error()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(T=-1), kda.KDA_ERR_BAD_SHAPE, "T must be >= 0"),
    (dict(H=0), kda.KDA_ERR_BAD_SHAPE, "H must be >= 1"),
    (dict(n_docs=0), kda.KDA_ERR_BAD_SHAPE, "n_docs must be >= 1"),
    (dict(n_docs=2), kda.KDA_ERR_BAD_SHAPE, "n_docs must be 1 when cu_seqlens is NULL"),
    (dict(n_docs=2**30, cu=P), kda.KDA_ERR_BAD_SHAPE, "n_docs * H"),
    (dict(q=None), kda.KDA_ERR_NULL_PTR, "q is NULL"),
    (dict(out=None), kda.KDA_ERR_NULL_PTR, "out is NULL"),
    (dict(chunk=32), kda.KDA_ERR_UNSUPPORTED, "chunk must be 64"),
    (dict(gate_bound=1.0), kda.KDA_ERR_UNSUPPORTED, "gate_bound"),
    (dict(T=0, q=None, chunk=32), kda.KDA_ERR_UNSUPPORTED, "chunk must be 64"),
    (dict(v=P + 4), kda.KDA_ERR_ALIGN, "v is not 16-byte aligned"),
    (dict(cu=P + 2), kda.KDA_ERR_ALIGN, "cu_seqlens is not 4-byte aligned"),
    (dict(h0=P + 8), kda.KDA_ERR_ALIGN, "initial_state is not 16-byte aligned"),
    (dict(ht=P + 4), kda.KDA_ERR_ALIGN, "final_state is not 16-byte aligned"),
])
def test_state_argument_validation(kw, code, msg):
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so not built")
    rc, err = _call_state(**kw)
    assert rc == code
    assert msg in err


def test_state_empty_stream_without_final_state_is_a_noop():
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so not built")
    rc, err = _call_state(T=0, q=None, k=None, v=None, g=None, beta=None, out=None, ht=None,
                          h0=P)
    assert rc == kda.KDA_OK and err == ""


def _call_rec(**kw):
    args = dict(q=P, k=P, v=P, g=P, beta=P, cu=None, n_docs=1, T=4, H=2, h0=P, ht=P, out=P,
                stream=None)
    args.update(kw)
    rc = kda.kda_recurrent_fwd(args["q"], args["k"], args["v"], args["g"], args["beta"],
                               args["cu"], args["n_docs"], args["T"], args["H"], args["h0"],
                               args["ht"], args["out"], args["stream"])
    return rc, kda.kda_last_error()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(T=-1), kda.KDA_ERR_BAD_SHAPE, "T must be >= 0"),
    (dict(H=0), kda.KDA_ERR_BAD_SHAPE, "H must be >= 1"),
    (dict(n_docs=0), kda.KDA_ERR_BAD_SHAPE, "n_docs must be >= 1"),
    (dict(n_docs=2), kda.KDA_ERR_BAD_SHAPE, "n_docs must be 1 when cu_seqlens is NULL"),
    (dict(n_docs=2**29 + 1, cu=P), kda.KDA_ERR_BAD_SHAPE, "n_docs * H"),
    # 2 x 64 work-items per (document, head): the launch stays below 2^32
    (dict(n_docs=2**24 + 1, cu=P), kda.KDA_ERR_BAD_SHAPE, "n_docs * H must be <= 2^25"),
    (dict(g=None), kda.KDA_ERR_NULL_PTR, "g is NULL"),
    (dict(k=P + 2), kda.KDA_ERR_ALIGN, "k is not 16-byte aligned"),
    (dict(h0=P + 4), kda.KDA_ERR_ALIGN, "initial_state is not 16-byte aligned"),
    (dict(ht=P + 8), kda.KDA_ERR_ALIGN, "final_state is not 16-byte aligned"),
])
def test_recurrent_argument_validation(kw, code, msg):
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so not built")
    rc, err = _call_rec(**kw)
    assert rc == code
    assert msg in err


def _call_bwd(**kw):
    args = dict(q=P, k=P, v=P, g=P, beta=P, cu=None, n_docs=1, T=64, H=2, chunk=64,
                gate_bound=-5.0, h0=None, do=P, dht=None, dq=P, dk=P, dv=P, dg=P, db=P,
                dh0=None, stream=None)
    args.update(kw)
    rc = kda.kda_chunk_bwd(*(args[x] for x in ("q", "k", "v", "g", "beta", "cu", "n_docs", "T",
                                               "H", "chunk", "gate_bound", "h0", "do", "dht",
                                               "dq", "dk", "dv", "dg", "db", "dh0", "stream")))
    return rc, kda.kda_last_error()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(T=-1), kda.KDA_ERR_BAD_SHAPE, "T must be >= 0"),
    (dict(n_docs=0), kda.KDA_ERR_BAD_SHAPE, "n_docs must be >= 1"),
    (dict(n_docs=3), kda.KDA_ERR_BAD_SHAPE, "n_docs must be 1 when cu_seqlens is NULL"),
    (dict(n_docs=2**28, cu=P), kda.KDA_ERR_BAD_SHAPE, "n_docs * H"),
    # 4 x 512 work-items per (document, head) in the state-gradient chain
    (dict(n_docs=2**20 + 1, cu=P), kda.KDA_ERR_BAD_SHAPE, "n_docs * H must be <= 2^21"),
    (dict(do=None), kda.KDA_ERR_NULL_PTR, "d_out is NULL"),
    (dict(dg=None), kda.KDA_ERR_NULL_PTR, "a gradient output is NULL"),
    (dict(chunk=16), kda.KDA_ERR_UNSUPPORTED, "chunk must be 64"),
    (dict(gate_bound=-9.0), kda.KDA_ERR_UNSUPPORTED, "gate_bound"),
    (dict(do=P + 2), kda.KDA_ERR_ALIGN, "d_out is not 16-byte aligned"),
    (dict(dk=P + 4), kda.KDA_ERR_ALIGN, "a gradient output is not aligned"),
    (dict(dht=P + 8), kda.KDA_ERR_ALIGN, "d_final_state is not 16-byte aligned"),
    (dict(dh0=P + 8), kda.KDA_ERR_ALIGN, "d_initial_state is not 16-byte aligned"),
])
def test_backward_argument_validation(kw, code, msg):
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so not built")
    rc, err = _call_bwd(**kw)
    assert rc == code
    assert msg in err


def test_backward_empty_stream_without_state_gradient_is_a_noop():
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so not built")
    rc, err = _call_bwd(T=0, q=None, k=None, v=None, g=None, beta=None, do=None, dq=None,
                        dk=None, dv=None, dg=None, db=None)
    assert rc == kda.KDA_OK and err == ""


def test_unsupported_reason_on_cpu_tensors():
    import torch
    q = torch.zeros(1, 8, 2, 128, dtype=torch.bfloat16)
    r = kda.unsupported_reason(q, q, q, q.float(), torch.zeros(1, 8, 2), None)
    assert "must be on a GPU" in r
    assert "kda_mode" in kda.unsupported_reason(q, q, q, q.float(), None, mode="recurrent")
    s0 = torch.zeros(1, 2, 128, 128)
    assert "must be on a GPU" in kda.unsupported_reason(q, q, q, q.float(),
                                                        torch.zeros(1, 8, 2), None,
                                                        initial_state=s0)
    assert "chunk must be 64" in kda.unsupported_reason(q, q, q, q.float(), None, chunk=16)


def test_split_policy_hook_validates_and_returns_the_previous_policy():
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so not built")
    assert kda.kda_debug_set_split_policy(3) == kda.KDA_ERR_UNSUPPORTED
    assert kda.kda_debug_set_split_policy(-1) == kda.KDA_ERR_UNSUPPORTED
    assert kda.set_split_policy("never") == "auto"
    assert kda.set_split_policy("always") == "never"
    assert kda.set_split_policy("auto") == "always"


def test_bwd_workspace_limit_hook_returns_the_previous_ceiling():
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so not built")
    default = 16 << 30
    assert kda.kda_debug_set_bwd_workspace_limit(1 << 20) == default
    assert kda.kda_debug_set_bwd_workspace_limit(0) == 1 << 20
    assert kda.kda_debug_set_bwd_workspace_limit(0) == default


def test_no_alloc_entry_point_validates_like_kda_chunk_fwd():
    if not os.path.exists(kda.LIB_PATH):
        pytest.skip("libkda.so not built")
    for kw, code, msg in [(dict(T=-1), kda.KDA_ERR_BAD_SHAPE, "T must be >= 0"),
                          (dict(q=None), kda.KDA_ERR_NULL_PTR, "q is NULL"),
                          (dict(chunk=32), kda.KDA_ERR_UNSUPPORTED, "chunk must be 64"),
                          (dict(out=P + 2), kda.KDA_ERR_ALIGN, "out is not 16-byte aligned")]:
        args = dict(q=P, k=P, v=P, g=P, beta=P, cu=None, T=128, H=2, chunk=64, gate_bound=-5.0,
                    out=P, stream=None)
        args.update(kw)
        rc = kda.kda_chunk_fwd_noalloc(*(args[x] for x in ("q", "k", "v", "g", "beta", "cu", "T",
                                                           "H", "chunk", "gate_bound", "out",
                                                           "stream")))
        assert rc == code and msg in kda.kda_last_error()
    assert kda.kda_chunk_fwd_noalloc(None, None, None, None, None, None, 0, 1, 64, -5.0, None,
                                     None) == kda.KDA_OK
