"""GPU parity of the token-recurrent entry point (kda_recurrent_fwd) against
the fp64 oracle: the same operator as the chunked forward with states,
evaluated one token at a time (decode and short documents).

Bar: output and final state within relative L2 5e-3 and max absolute error
3e-2 of the oracle.  The recurrent kernel keeps everything in fp32 except the
bf16 output, so its state is far closer to the oracle than that bar."""
import numpy as np
import pytest

import oracle
from kda_gpu_util import MAX_ABS_TOL, REL_L2_TOL, log, to_device
from kda_workloads import cu_from_lengths, initial_states, make_inputs, with_gate_scale

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_sequence_amd as kda
    kda.load_library()


def _check(inp, o, ht, h0, label, heads=None, state_tol=REL_L2_TOL):
    cu = [int(x) for x in inp.cu_seqlens]
    heads = range(inp.H) if heads is None else heads
    tasks = [(a, b, h, h + 1, d) for d, (a, b) in enumerate(zip(cu[:-1], cu[1:])) for h in heads]
    o_np = o.float().cpu().numpy().astype(np.float64)
    ht_np = None if ht is None else ht.cpu().numpy().astype(np.float64)
    acc = dict(no=0.0, do=0.0, ns=0.0, ds=0.0, mo=0.0, ms=0.0)
    for (a, b, h0_, h1_, d), ref_o, ref_s in oracle.kda_tasks(
            inp.q, inp.k, inp.v, inp.g, inp.beta, tasks, initial_state=h0, final_state=True):
        if b > a:
            diff = o_np[a:b, h0_:h1_] - ref_o
            acc["no"] += float((diff * diff).sum())
            acc["do"] += float((ref_o * ref_o).sum())
            acc["mo"] = max(acc["mo"], float(np.abs(diff).max()))
        if ht_np is not None:
            diff = ht_np[d, h0_:h1_] - ref_s
            acc["ns"] += float((diff * diff).sum())
            acc["ds"] += float((ref_s * ref_s).sum())
            acc["ms"] = max(acc["ms"], float(np.abs(diff).max()))
    if acc["do"] > 0:
        rel = np.sqrt(acc["no"] / acc["do"])
        log(f"[parity] {label}: o relL2={rel:.3e} maxabs={acc['mo']:.3e} tasks={len(tasks)}")
        assert rel <= REL_L2_TOL and acc["mo"] <= MAX_ABS_TOL, (label, rel, acc["mo"])
    if ht_np is not None:
        rel = np.sqrt(acc["ns"] / acc["ds"])
        log(f"[parity] {label}: state relL2={rel:.3e} maxabs={acc['ms']:.3e}")
        assert rel <= state_tol and acc["ms"] <= MAX_ABS_TOL, (label, rel, acc["ms"])


def _rec(d, h0=None, final=True, cu_key="cu"):
    import torch
    import linear_attention_sequence_amd as kda
    s0 = None if h0 is None else torch.from_numpy(np.ascontiguousarray(h0)).cuda()
    o, ht = kda.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                              d[cu_key] if cu_key else None, initial_state=s0,
                              output_final_state=final)
    torch.cuda.synchronize()
    return o, ht


def test_decode_step_one_token_per_document():
    N, H = 64, 4
    inp = make_inputs(N, H, 61, cu_from_lengths([1] * N))
    h0 = initial_states(N, H, 61)
    log(f"[case] recurrent decode N={N} H={H}")
    o, ht = _rec(to_device(inp), h0)
    _check(inp, o, ht, h0, "recurrent decode step", state_tol=1e-5)


@pytest.mark.parametrize("gate_scale", [-5.0, -0.05])
def test_short_documents_with_states(gate_scale):
    lengths = [1, 5, 33, 0, 64, 100, 0]
    T, H = sum(lengths), 3
    inp = make_inputs(T, H, 62, cu_from_lengths(lengths))
    if gate_scale != -5.0:
        inp = with_gate_scale(inp, 62, gate_scale)
    h0 = initial_states(len(lengths), H, 62)
    log(f"[case] recurrent short docs gate={gate_scale}")
    o, ht = _rec(to_device(inp), h0)
    _check(inp, o, ht, h0, f"recurrent short docs (gate {gate_scale})", state_tol=1e-5)
    ht_np = ht.cpu().numpy()
    np.testing.assert_array_equal(ht_np[3], h0[3])
    np.testing.assert_array_equal(ht_np[6], h0[6])


@pytest.mark.parametrize("gate", ["zero", "lowest"])
def test_extreme_gates_with_states(gate):
    """g = 0 everywhere (no decay: the state keeps every token) over a
    200-token document, and g = -5.5 everywhere (the lowest accepted gate),
    with initial and final states."""
    import dataclasses
    lengths = [200, 17, 1]
    T, H = sum(lengths), 2
    base = make_inputs(T, H, 68, cu_from_lengths(lengths))
    inp = dataclasses.replace(base, g=np.full_like(base.g, 0.0 if gate == "zero" else -5.5))
    h0 = initial_states(len(lengths), H, 68)
    log(f"[case] recurrent extreme gate {gate}")
    o, ht = _rec(to_device(inp), h0)
    _check(inp, o, ht, h0, f"recurrent gate {gate}", state_tol=1e-4)


def test_no_states_and_dense_batch():
    import torch
    import linear_attention_sequence_amd as kda
    B, Tb, H = 4, 40, 2
    inp = make_inputs(B * Tb, H, 63, cu_from_lengths([Tb] * B))
    d = to_device(inp)
    view = lambda x: x.view(B, Tb, H, -1) if x.dim() == 3 else x.view(B, Tb, H)  # noqa: E731
    o, ht = kda.recurrent_fwd(*(view(d[x]) for x in ("q", "k", "v", "g", "beta")), None)
    torch.cuda.synchronize()
    assert ht is None
    _check(inp, o.view(B * Tb, H, 128), None, None, "recurrent dense batch, zero state")


def test_in_place_decode_loop_matches_one_prefill():
    """Eight decode steps, each updating the state buffer in place, equal one
    recurrent call over the eight tokens of every document."""
    import torch
    import linear_attention_sequence_amd as kda
    N, H, steps = 16, 2, 8
    T = N * steps
    # token s of sequence n sits at row s * N + n (one decode batch per step)
    inp = with_gate_scale(make_inputs(T, H, 64, cu_from_lengths([T])), 64, -0.05)
    d = to_device(inp)
    h0 = initial_states(N, H, 64)
    state = torch.from_numpy(h0.copy()).cuda()
    cu_step = torch.arange(0, N + 1, dtype=torch.int32, device="cuda")
    outs = []
    for s in range(steps):
        rows = slice(s * N, (s + 1) * N)
        o, _ = kda.recurrent_fwd(*(d[x][rows] for x in ("q", "k", "v", "g", "beta")), cu_step,
                                 initial_state=state, final_state=state)
        outs.append(o)
    torch.cuda.synchronize()
    o_steps = torch.stack(outs)                      # [steps, N, H, 128]
    # the same tokens laid out document by document, for the oracle
    perm = np.arange(T).reshape(steps, N).T.reshape(-1)
    pin = type(inp)(inp.q[perm], inp.k[perm], inp.v[perm], inp.g[perm], inp.beta[perm],
                    cu_from_lengths([steps] * N))
    o_docs = o_steps.permute(1, 0, 2, 3).reshape(T, H, 128)
    _check(pin, o_docs, state, h0, "in-place decode loop", state_tol=1e-5)


def test_matches_the_chunked_state_path():
    import torch
    import linear_attention_sequence_amd as kda
    lengths = [70, 3, 129]
    T, H = sum(lengths), 2
    inp = with_gate_scale(make_inputs(T, H, 65, cu_from_lengths(lengths)), 65, -0.1)
    d = to_device(inp)
    h0 = torch.from_numpy(initial_states(len(lengths), H, 65)).cuda()
    o_r, s_r = kda.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"],
                                 initial_state=h0, output_final_state=True)
    o_c, s_c = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"],
                             initial_state=h0, output_final_state=True)
    torch.cuda.synchronize()
    rel_o = float(torch.linalg.norm((o_r.float() - o_c.float()).flatten())
                  / torch.linalg.norm(o_r.float().flatten()))
    rel_s = float(torch.linalg.norm((s_r - s_c).flatten()) / torch.linalg.norm(s_r.flatten()))
    log(f"[parity] recurrent vs chunked: o relL2={rel_o:.3e} state relL2={rel_s:.3e}")
    assert rel_o <= 2 * REL_L2_TOL and rel_s <= 2 * REL_L2_TOL


def test_empty_stream_and_bad_cu_seqlens():
    import torch
    import linear_attention_sequence_amd as kda
    H = 2
    e = torch.empty(0, H, 128, device="cuda")
    q = e.to(torch.bfloat16)
    h0 = torch.from_numpy(initial_states(3, H, 66)).cuda()
    o, ht = kda.recurrent_fwd(q, q, q, e, torch.empty(0, H, device="cuda"),
                              torch.zeros(4, dtype=torch.int32, device="cuda"),
                              initial_state=h0, output_final_state=True)
    torch.cuda.synchronize()
    assert bool((ht == h0).all())
    inp = make_inputs(20, H, 66, cu_from_lengths([10, 10]))
    d = to_device(inp)
    kda.device_status()
    bad = torch.tensor([0, 12, 11], dtype=torch.int32, device="cuda")
    o, ht = kda.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], bad,
                              output_final_state=True)
    assert kda.device_status() & kda.KDA_DEV_BAD_CU_SEQLENS
    assert bool(torch.isnan(o.float()).all()) and bool(torch.isnan(ht).all())


def test_decode_batch_at_serving_size_sampled_heads():
    """One decode step for 256 sequences x 32 heads (the size the decode
    benchmark times), sampled heads against the oracle."""
    N, H = 256, 32
    inp = make_inputs(N, H, 67, cu_from_lengths([1] * N))
    h0 = initial_states(N, H, 67)
    log(f"[case] recurrent decode N={N} H={H}")
    o, ht = _rec(to_device(inp), h0)
    _check(inp, o, ht, h0, "recurrent decode 256x32", heads=[0, 17, 31], state_tol=1e-5)
