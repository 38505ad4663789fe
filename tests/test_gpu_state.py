"""GPU parity of the state-carrying entry point (kda_chunk_fwd_state) against
the fp64 oracle: document d starts from initial_state[d] and its last state is
returned in final_state[d] (FLA's chunk_kda convention, of which the fused K3
forward is the drop-in with the state switched off).

Bar: output and final state each within relative L2 5e-3 and max absolute
error 3e-2 of the oracle (the state is accumulated in fp32 from bf16 products,
like the output); cases that must agree exactly (zero-length documents, a
document cut at a chunk boundary, zero initial state) are compared bit for bit."""
import numpy as np
import pytest

import oracle
from kda_gpu_util import MAX_ABS_TOL, REL_L2_TOL, log, to_device, set_split
from kda_workloads import (cu_from_lengths, initial_states, make_inputs, with_gate_scale,
                           workload_inputs)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_sequence_amd as kda
    kda.load_library()


def _run(inp, h0=None, final=True, cu=True, dense_batch=None):
    import torch
    import linear_attention_sequence_amd as kda
    d = to_device(inp)
    s0 = None if h0 is None else torch.from_numpy(np.ascontiguousarray(h0)).cuda()
    q, k, v, g, beta = d["q"], d["k"], d["v"], d["g"], d["beta"]
    if dense_batch:
        B = dense_batch
        T = inp.T // B
        q, k, v, g = (x.view(B, T, inp.H, 128) for x in (q, k, v, g))
        beta = beta.view(B, T, inp.H)
    o, ht = kda.chunk_fwd(q, k, v, g, beta, d["cu"] if cu else None, initial_state=s0,
                          output_final_state=final)
    torch.cuda.synchronize()
    if dense_batch:
        o = o.view(inp.T, inp.H, 128)
    return o, ht


def _rel(got, ref):
    d = got - ref
    den = np.sqrt((ref * ref).sum())
    return (np.sqrt((d * d).sum()) / den if den > 0 else np.sqrt((d * d).sum())), \
        (float(np.abs(d).max()) if d.size else 0.0)


def _check(inp, o, ht, h0, label, heads=None):
    """Oracle per (document, head): o over the document, and its last state."""
    cu = [int(x) for x in inp.cu_seqlens]
    heads = range(inp.H) if heads is None else heads
    tasks = [(a, b, h, h + 1, d) for d, (a, b) in enumerate(zip(cu[:-1], cu[1:])) for h in heads]
    o_np = o.float().cpu().numpy().astype(np.float64)
    ht_np = None if ht is None else ht.cpu().numpy().astype(np.float64)
    num_o = den_o = num_s = den_s = 0.0
    mx_o = mx_s = 0.0
    for (a, b, h0_, h1_, d), ref_o, ref_s in oracle.kda_tasks(
            inp.q, inp.k, inp.v, inp.g, inp.beta, tasks, initial_state=h0, final_state=True):
        if b > a:
            diff = o_np[a:b, h0_:h1_] - ref_o
            num_o += float((diff * diff).sum())
            den_o += float((ref_o * ref_o).sum())
            mx_o = max(mx_o, float(np.abs(diff).max()))
        if ht_np is not None:
            diff = ht_np[d, h0_:h1_] - ref_s
            num_s += float((diff * diff).sum())
            den_s += float((ref_s * ref_s).sum())
            mx_s = max(mx_s, float(np.abs(diff).max()))
    rel_o = np.sqrt(num_o / den_o)
    log(f"[parity] {label}: o relL2={rel_o:.3e} maxabs={mx_o:.3e} tasks={len(tasks)}")
    assert rel_o <= REL_L2_TOL and mx_o <= MAX_ABS_TOL, (label, rel_o, mx_o)
    if ht_np is not None:
        rel_s = np.sqrt(num_s / den_s)
        log(f"[parity] {label}: state relL2={rel_s:.3e} maxabs={mx_s:.3e}")
        assert rel_s <= REL_L2_TOL and mx_s <= MAX_ABS_TOL, (label, rel_s, mx_s)


# lengths: ragged tails, an empty document inside and one at the end, a long
# document (> 8 chunks, a split candidate) and a one-token document
LENGTHS = [700, 0, 1, 130, 1500, 64, 0]


@pytest.mark.parametrize("policy", ["never", "always", "auto"])
def test_packed_with_initial_and_final_state(policy):
    if policy != "auto":
        set_split(policy)
    T, H = sum(LENGTHS), 4
    inp = with_gate_scale(make_inputs(T, H, 51, cu_from_lengths(LENGTHS)), 51, -0.05)
    h0 = initial_states(len(LENGTHS), H, 51)
    log(f"[case] state packed policy={policy} lengths={LENGTHS}")
    o, ht = _run(inp, h0)
    _check(inp, o, ht, h0, f"state packed ({policy})")
    # empty documents pass their state through unchanged
    ht_np = ht.cpu().numpy()
    np.testing.assert_array_equal(ht_np[1], h0[1])
    np.testing.assert_array_equal(ht_np[6], h0[6])


def test_split_and_fused_states_are_bit_identical():
    T, H = sum(LENGTHS), 2
    inp = with_gate_scale(make_inputs(T, H, 52, cu_from_lengths(LENGTHS)), 52, -0.3)
    h0 = initial_states(len(LENGTHS), H, 52)
    set_split("never")
    o1, s1 = _run(inp, h0)
    set_split("always")
    o2, s2 = _run(inp, h0)
    assert bool((o1 == o2).all())
    assert bool((s1 == s2).all())


def test_no_decay_with_states():
    """g = 0 (the initial state never decays and every token stays in the
    state) over a 2048-token and a 300-token document: the slowest-decaying
    case of the chunked state path, fused and split, which agree bit for bit."""
    lengths = [2048, 300]
    T, H = sum(lengths), 2
    inp = with_gate_scale(make_inputs(T, H, 91, cu_from_lengths(lengths)), 91, 0.0)
    h0 = initial_states(len(lengths), H, 91)
    set_split("never")
    o1, s1 = _run(inp, h0)
    set_split("always")
    o2, s2 = _run(inp, h0)
    assert bool((o1 == o2).all()) and bool((s1 == s2).all())
    _check(inp, o2, s2, h0, "state, no decay")


def test_initial_state_only_and_final_state_only():
    lengths = [333, 1000]
    T, H = sum(lengths), 3
    inp = with_gate_scale(make_inputs(T, H, 53, cu_from_lengths(lengths)), 53, -0.05)
    h0 = initial_states(len(lengths), H, 53)
    log("[case] state: initial only")
    o, ht = _run(inp, h0, final=False)
    assert ht is None
    _check(inp, o, None, h0, "initial state only")
    log("[case] state: final only")
    o, ht = _run(inp, None, final=True)
    _check(inp, o, ht, None, "final state only")


def test_zero_initial_state_matches_the_stateless_kernel():
    import torch
    import linear_attention_sequence_amd as kda
    lengths = [200, 900, 17]
    T, H = sum(lengths), 4
    inp = make_inputs(T, H, 54, cu_from_lengths(lengths))
    d = to_device(inp)
    o_plain, none = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"])
    assert none is None
    z = torch.zeros(len(lengths), H, 128, 128, device="cuda")
    o_state, ht = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"],
                                initial_state=z, output_final_state=True)
    torch.cuda.synchronize()
    assert bool((o_plain == o_state).all())
    _check(inp, o_state, ht, None, "zero initial state")


def test_dense_batch_with_states():
    B, Tb, H = 3, 300, 2
    inp = with_gate_scale(make_inputs(B * Tb, H, 55, cu_from_lengths([Tb] * B)), 55, -0.1)
    h0 = initial_states(B, H, 55)
    log("[case] state dense batch")
    o, ht = _run(inp, h0, cu=False, dense_batch=B)
    assert tuple(ht.shape) == (B, H, 128, 128)
    _check(inp, o, ht, h0, "state dense batch")


def test_single_document_without_cu_seqlens():
    T, H = 515, 2
    inp = with_gate_scale(make_inputs(T, H, 56, cu_from_lengths([T])), 56, -0.05)
    h0 = initial_states(1, H, 56)
    o, ht = _run(inp, h0, cu=False)
    _check(inp, o, ht, h0, "state, cu_seqlens None")


@pytest.mark.parametrize("cut", [256, 300])
def test_chunked_prefill_equals_one_call(cut):
    """A document run in two calls, the second starting from the first's final
    state, equals one call: bit for bit when the cut is a chunk boundary (the
    same chunks, the state handed over in fp32), else within the bar."""
    import torch
    import linear_attention_sequence_amd as kda
    T, H = 1000, 4
    inp = with_gate_scale(make_inputs(T, H, 57, cu_from_lengths([T])), 57, -0.05)
    d = to_device(inp)
    h0 = torch.from_numpy(initial_states(1, H, 57)).cuda()
    o_all, s_all = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], None,
                                 initial_state=h0, output_final_state=True)
    parts = []
    s = h0
    for a, b in ((0, cut), (cut, T)):
        o_p, s = kda.chunk_fwd(*(d[x][a:b].contiguous() for x in ("q", "k", "v", "g", "beta")),
                               None, initial_state=s, output_final_state=True)
        parts.append(o_p)
    torch.cuda.synchronize()
    o_two = torch.cat(parts)
    if cut % 64 == 0:
        assert bool((o_two == o_all).all()) and bool((s == s_all).all())
    else:
        rel, mx = _rel(o_two.float().cpu().numpy(), o_all.float().cpu().numpy())
        log(f"[parity] prefill cut {cut}: o relL2 vs one call {rel:.3e}")
        assert rel <= REL_L2_TOL
        rel, mx = _rel(s.cpu().numpy(), s_all.cpu().numpy())
        assert rel <= REL_L2_TOL
    _check(inp, o_all, s_all, initial_states(1, H, 57), f"prefill reference (cut {cut})")


def test_in_place_state_update():
    """final_state may be the initial_state buffer (the C ABI allows it)."""
    import torch
    import linear_attention_sequence_amd as kda
    lengths = [129, 640]
    T, H = sum(lengths), 2
    inp = with_gate_scale(make_inputs(T, H, 58, cu_from_lengths(lengths)), 58, -0.05)
    d = to_device(inp)
    h0_np = initial_states(len(lengths), H, 58)
    buf = torch.from_numpy(h0_np.copy()).cuda()
    out = torch.empty_like(d["v"])
    stream = torch.cuda.current_stream().cuda_stream
    rc = kda.kda_chunk_fwd_state(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(),
                                 d["g"].data_ptr(), d["beta"].data_ptr(), d["cu"].data_ptr(),
                                 len(lengths), T, H, 64, -5.0, buf.data_ptr(), buf.data_ptr(),
                                 out.data_ptr(), stream)
    assert rc == 0, kda.kda_last_error()
    torch.cuda.synchronize()
    _check(inp, out, buf, h0_np, "in-place state")


def test_empty_stream_passes_states_through():
    import torch
    import linear_attention_sequence_amd as kda
    H = 3
    e = torch.empty(0, H, 128, device="cuda")
    q = e.to(torch.bfloat16)
    cu = torch.zeros(4, dtype=torch.int32, device="cuda")
    h0 = torch.from_numpy(initial_states(3, H, 59)).cuda()
    o, ht = kda.chunk_fwd(q, q, q, e, torch.empty(0, H, device="cuda"), cu, initial_state=h0,
                          output_final_state=True)
    torch.cuda.synchronize()
    assert o.numel() == 0
    assert bool((ht == h0).all())
    _, ht0 = kda.chunk_fwd(q, q, q, e, torch.empty(0, H, device="cuda"), cu,
                           output_final_state=True)
    torch.cuda.synchronize()
    assert bool((ht0 == 0).all())


def test_bad_cu_seqlens_fills_final_state_with_nan():
    import torch
    import linear_attention_sequence_amd as kda
    lengths = [100, 100]
    T, H = 200, 2
    inp = make_inputs(T, H, 60, cu_from_lengths(lengths))
    d = to_device(inp)
    kda.device_status()
    cu = torch.tensor([0, 150, 100], dtype=torch.int32, device="cuda")   # decreasing
    o, ht = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, output_final_state=True)
    st = kda.device_status()
    assert st & kda.KDA_DEV_BAD_CU_SEQLENS
    assert bool(torch.isnan(o.float()).all()) and bool(torch.isnan(ht).all())
    cu = torch.tensor([0, 100, 150], dtype=torch.int32, device="cuda")   # does not end at T
    o, ht = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, output_final_state=True)
    assert kda.device_status() & kda.KDA_DEV_BAD_CU_SEQLENS
    assert bool(torch.isnan(ht).all())


def test_packed_stream_with_states_sampled_heads():
    """The 32768-token packed lognormal stream (H = 32), every document with an
    initial state, slow decay so the state reaches far; sampled heads."""
    w, inp = workload_inputs(3)
    inp = with_gate_scale(inp, w.seed, -0.05)
    n = len(inp.cu_seqlens) - 1
    h0 = initial_states(n, w.H, w.seed)
    log(f"[case] state {w.name} docs={n}")
    o, ht = _run(inp, h0)
    _check(inp, o, ht, h0, f"state {w.name}", heads=[0, 9, 31])
