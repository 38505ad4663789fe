"""GPU parity of the chunked backward (kda_chunk_bwd) against the fp64
autograd oracle (oracle/kda_oracle_bwd.py).

Bar, per gradient tensor: relative L2 error <= 5e-3 and max absolute error
<= 3e-2 times max(1, max |reference|).  The backward runs in fp32; its error
comes mostly from the forward states it differentiates around, which the
bf16/fp16 forward pipeline produces (relative error ~2e-3, the forward's own
bar)."""
import numpy as np
import pytest

from kda_gpu_util import REL_L2_TOL, log, to_device, set_split
from kda_workloads import (cu_from_lengths, initial_states, make_inputs, standard_normal,
                           round_to_bf16, with_gate_scale)
from oracle.kda_oracle_bwd import kda_backward_tasks

pytestmark = pytest.mark.gpu
ABS_TOL = 3e-2
NAMES = ("dq", "dk", "dv", "dg", "dbeta")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_sequence_amd as kda
    kda.load_library()


def _dout(T, H, seed):
    return round_to_bf16(standard_normal((T, H, 128), seed, 11))


def _run(inp, do, h0=None, dht=None, cu=True):
    import torch
    import linear_attention_sequence_amd as kda
    d = to_device(inp)
    t = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa
    r = kda.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                      torch.from_numpy(do).to(torch.bfloat16).cuda(), d["cu"] if cu else None,
                      initial_state=t(h0), d_final_state=t(dht))
    torch.cuda.synchronize()
    return [None if x is None else x.cpu().numpy().astype(np.float64) for x in r]


def _check(inp, do, got, h0, dht, label, heads=None):
    cu = [int(x) for x in inp.cu_seqlens]
    heads = range(inp.H) if heads is None else heads
    tasks = [(a, b, h, h + 1, d) for d, (a, b) in enumerate(zip(cu[:-1], cu[1:])) for h in heads]
    acc = {n: [0.0, 0.0, 0.0, 0.0] for n in NAMES + ("dh0",)}   # num, den, maxdiff, maxref
    for (a, b, h0_, h1_, d), ref in kda_backward_tasks(inp.q, inp.k, inp.v, inp.g, inp.beta, do,
                                                       tasks, h0, dht):
        for i, n in enumerate(NAMES):
            if b > a:
                x = got[i][a:b, h0_:h1_] - ref[n]
                acc[n][0] += float((x * x).sum())
                acc[n][1] += float((ref[n] * ref[n]).sum())
                acc[n][2] = max(acc[n][2], float(np.abs(x).max()))
                acc[n][3] = max(acc[n][3], float(np.abs(ref[n]).max()))
        if got[5] is not None:
            x = got[5][d, h0_:h1_] - ref["dh0"]
            acc["dh0"][0] += float((x * x).sum())
            acc["dh0"][1] += float((ref["dh0"] * ref["dh0"]).sum())
            acc["dh0"][2] = max(acc["dh0"][2], float(np.abs(x).max()))
            acc["dh0"][3] = max(acc["dh0"][3], float(np.abs(ref["dh0"]).max()))
    for n, (num, den, mx, mref) in acc.items():
        if den == 0:
            continue
        rel = np.sqrt(num / den)
        log(f"[parity] {label} {n}: relL2={rel:.3e} maxabs={mx:.3e} (max|ref| {mref:.3e})")
        assert rel <= REL_L2_TOL, (label, n, rel)
        assert mx <= ABS_TOL * max(1.0, mref), (label, n, mx)


LENGTHS = [130, 0, 37, 200, 64, 1]


@pytest.mark.parametrize("states", [False, True])
def test_backward_small_packed(states):
    T, H = sum(LENGTHS), 2
    inp = with_gate_scale(make_inputs(T, H, 71, cu_from_lengths(LENGTHS)), 71, -0.05)
    do = _dout(T, H, 71)
    h0 = initial_states(len(LENGTHS), H, 71) if states else None
    dht = initial_states(len(LENGTHS), H, 72, std=1.0) if states else None
    log(f"[case] bwd small packed states={states}")
    got = _run(inp, do, h0, dht)
    _check(inp, do, got, h0, dht, f"bwd small (states={states})")


@pytest.mark.parametrize("policy", ["never", "always"])
def test_backward_split_and_fused_forward(policy):
    set_split(policy)
    lengths = [700, 300]
    T, H = sum(lengths), 2
    inp = make_inputs(T, H, 73, cu_from_lengths(lengths))
    do = _dout(T, H, 73)
    log(f"[case] bwd forward policy={policy}")
    got = _run(inp, do)
    _check(inp, do, got, None, None, f"bwd workload gate ({policy})")


def test_backward_single_document_without_cu_seqlens():
    T, H = 515, 3
    inp = with_gate_scale(make_inputs(T, H, 74, cu_from_lengths([T])), 74, -0.3)
    do = _dout(T, H, 74)
    h0 = initial_states(1, H, 74)
    got = _run(inp, do, h0, None, cu=False)
    _check(inp, do, got, h0, None, "bwd one document, cu None")


def test_backward_empty_stream_and_bad_cu_seqlens():
    import torch
    import linear_attention_sequence_amd as kda
    H = 2
    e = torch.empty(0, H, 128, device="cuda")
    q = e.to(torch.bfloat16)
    cu = torch.zeros(3, dtype=torch.int32, device="cuda")
    h0 = torch.from_numpy(initial_states(2, H, 75)).cuda()
    dht = torch.from_numpy(initial_states(2, H, 76)).cuda()
    r = kda.chunk_bwd(q, q, q, e, torch.empty(0, H, device="cuda"), q, cu, initial_state=h0,
                      d_final_state=dht)
    torch.cuda.synchronize()
    assert bool((r[5] == dht).all())
    inp = make_inputs(100, H, 77, cu_from_lengths([50, 50]))
    d = to_device(inp)
    kda.device_status()
    bad = torch.tensor([0, 60, 40], dtype=torch.int32, device="cuda")
    r = kda.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["v"].clone(), bad)
    assert kda.device_status() & kda.KDA_DEV_BAD_CU_SEQLENS
    for x in r[:5]:
        assert bool(torch.isnan(x).all())


def test_backward_4096_token_document_sampled_heads():
    T, H = 4096, 8
    inp = make_inputs(T, H, 78, cu_from_lengths([T]))
    do = _dout(T, H, 78)
    log("[case] bwd T=4096 H=8")
    got = _run(inp, do)
    _check(inp, do, got, None, None, "bwd T=4096", heads=[0, 5])


def test_autograd_wrapper_matches_the_oracle():
    """chunk_kda through torch.autograd: q, k, v keep their bf16 dtype (their
    gradients are rounded to bf16), g and beta fp32, the initial state fp32."""
    import torch
    import linear_attention_sequence_amd as kda
    from oracle.kda_oracle_bwd import kda_backward
    lengths = [90, 200]
    T, H = sum(lengths), 2
    inp = with_gate_scale(make_inputs(T, H, 79, cu_from_lengths(lengths)), 79, -0.1)
    do = _dout(T, H, 79)
    h0 = initial_states(len(lengths), H, 79)
    d = to_device(inp)
    leaves = [d[x].detach().clone().requires_grad_(True) for x in ("q", "k", "v", "g", "beta")]
    s0 = torch.from_numpy(h0).cuda().requires_grad_(True)
    o, fin = kda.chunk_kda(*leaves, d["cu"], initial_state=s0, output_final_state=True)
    dfin = torch.from_numpy(initial_states(len(lengths), H, 80)).cuda()
    torch.autograd.backward([o, fin], [torch.from_numpy(do).to(torch.bfloat16).cuda(), dfin])
    ref = kda_backward(inp.q, inp.k, inp.v, inp.g, inp.beta, do, inp.cu_seqlens, h0,
                       dfin.cpu().numpy().astype(np.float64))
    for name, leaf in zip(NAMES + ("dh0",), leaves + [s0]):
        got = leaf.grad.float().cpu().numpy().astype(np.float64)
        rel = np.linalg.norm(got - ref[name]) / np.linalg.norm(ref[name])
        log(f"[parity] autograd {name}: relL2={rel:.3e} dtype={leaf.grad.dtype}")
        assert leaf.grad.dtype == leaf.dtype
        assert rel <= REL_L2_TOL, (name, rel)


@pytest.mark.parametrize("H", [1, 5])
def test_backward_head_counts(H):
    lengths = [65, 130]
    T = sum(lengths)
    inp = with_gate_scale(make_inputs(T, H, 81, cu_from_lengths(lengths)), 81, -0.2)
    do = _dout(T, H, 81)
    got = _run(inp, do)
    _check(inp, do, got, None, None, f"bwd H={H}")


def test_backward_special_inputs():
    """beta = 0 (nothing is written: dq = dk = dg = 0 without a state) and
    g = 0 (no decay), one-token and exactly-one-chunk documents."""
    lengths = [1, 64, 100]
    T, H = sum(lengths), 2
    inp = make_inputs(T, H, 82, cu_from_lengths(lengths))
    inp.beta[:] = 0.0
    do = _dout(T, H, 82)
    got = _run(inp, do)
    for i in (0, 1, 3):
        assert np.abs(got[i]).max() == 0.0, i
    _check(inp, do, got, None, None, "bwd beta = 0")
    inp2 = with_gate_scale(make_inputs(T, H, 83, cu_from_lengths(lengths)), 83, 0.0)
    got2 = _run(inp2, do)
    _check(inp2, do, got2, None, None, "bwd g = 0")


def test_backward_no_decay_long_document():
    """g = 0 over a 1024-token document (16 chunks) and a short one, with an
    initial state and a final-state gradient: nothing decays, so the state
    gradient of the last chunk reaches the first undiminished."""
    lengths = [1024, 40]
    T, H = sum(lengths), 1
    inp = with_gate_scale(make_inputs(T, H, 86, cu_from_lengths(lengths)), 86, 0.0)
    do = _dout(T, H, 86)
    h0 = initial_states(len(lengths), H, 86)
    dht = np.ascontiguousarray(initial_states(len(lengths), H, 87))
    log(f"[case] bwd no decay, T={T}")
    got = _run(inp, do, h0, dht)
    _check(inp, do, got, h0, dht, "bwd no decay, 1024 tokens")


def test_backward_packed_stream_sampled_heads():
    """The 32768-token packed lognormal stream (H = 32), every document, two
    sampled heads; the same launch configuration as the backward benchmark."""
    from kda_workloads import workload_inputs
    w, inp = workload_inputs(3)
    do = _dout(w.T, w.H, w.seed)
    log(f"[case] bwd {w.name}")
    got = _run(inp, do)
    _check(inp, do, got, None, None, f"bwd {w.name}", heads=[0, 31])


def test_backward_long_document_one_head():
    """The 65536-token document of the long-plus-short stream (1024 chunks
    through the state-gradient chain), one sampled head."""
    from kda_workloads import workload_inputs
    w, inp = workload_inputs(5)
    do = _dout(w.T, w.H, w.seed)
    log(f"[case] bwd {w.name} long document")
    got = _run(inp, do)
    cu = [int(x) for x in inp.cu_seqlens]
    tasks = [(cu[0], cu[1], 7, 8, 0)]
    for (a, b, h0_, h1_, d), ref in kda_backward_tasks(inp.q, inp.k, inp.v, inp.g, inp.beta, do,
                                                       tasks):
        for i, n in enumerate(NAMES):
            x = got[i][a:b, h0_:h1_] - ref[n]
            rel = float(np.sqrt((x * x).sum() / (ref[n] * ref[n]).sum()))
            mx = float(np.abs(x).max())
            log(f"[parity] bwd long document {n}: relL2={rel:.3e} maxabs={mx:.3e}")
            assert rel <= REL_L2_TOL and mx <= ABS_TOL * max(1.0, float(np.abs(ref[n]).max())), n


def test_backward_many_tiny_documents():
    """300 documents of 1 to 5 tokens with states: chunks of a few rows, most
    of every 16-row block empty, a long chunk table and many chains."""
    rng = np.random.default_rng(71)
    lengths = [int(x) for x in rng.integers(1, 6, size=300)]
    T, H = sum(lengths), 2
    inp = make_inputs(T, H, 71, cu_from_lengths(lengths))
    do = _dout(T, H, 71)
    h0 = initial_states(len(lengths), H, 71)
    dht = np.ascontiguousarray(initial_states(len(lengths), H, 72))
    log(f"[case] bwd {len(lengths)} tiny documents, T={T}")
    got = _run(inp, do, h0, dht)
    _check(inp, do, got, h0, dht, "bwd tiny documents")


def test_backward_thousands_of_one_token_documents():
    """4096 documents of one token at H = 32: a workspace slot per document
    and head would take ~54 GB in one pass, so the call runs over groups of
    documents, each within the default 16 GiB ceiling."""
    T, H = 4096, 32
    inp = make_inputs(T, H, 91, cu_from_lengths([1] * T))
    do = _dout(T, H, 91)
    log(f"[case] bwd {T} one-token documents, H={H}")
    got = _run(inp, do)
    _check(inp, do, got, None, None, "bwd 4096 one-token documents", heads=[0, 17, 31])


def test_backward_in_groups_matches_one_pass():
    """A ceiling of one byte forces one document per pass: the gradients are
    the single pass's bit for bit (documents are independent), with states,
    empty documents and both ends of the stream."""
    import linear_attention_sequence_amd as kda
    lengths = [0, 130, 0, 37, 200, 64, 1, 300, 5, 0]
    T, H = sum(lengths), 2
    inp = with_gate_scale(make_inputs(T, H, 92, cu_from_lengths(lengths)), 92, -0.05)
    do = _dout(T, H, 92)
    h0 = initial_states(len(lengths), H, 92)
    dht = np.ascontiguousarray(initial_states(len(lengths), H, 93))
    log("[case] bwd in groups of one document vs one pass")
    one = _run(inp, do, h0, dht)
    prev = kda.kda_debug_set_bwd_workspace_limit(1)
    try:
        grouped = _run(inp, do, h0, dht)
    finally:
        kda.kda_debug_set_bwd_workspace_limit(prev)
    for name, a, b in zip(NAMES + ("dh0",), one, grouped):
        assert np.array_equal(a, b), name
    _check(inp, do, grouped, h0, dht, "bwd in groups")


def test_backward_in_groups_rejects_bad_cu_seqlens():
    """The grouped path reads cu_seqlens on the host; a broken one still sets
    the device flag and fills every gradient with NaN."""
    import torch
    import linear_attention_sequence_amd as kda
    H = 2
    inp = make_inputs(100, H, 94, cu_from_lengths([50, 30, 20]))
    d = to_device(inp)
    kda.device_status()
    bad = torch.tensor([0, 60, 40, 100], dtype=torch.int32, device="cuda")
    prev = kda.kda_debug_set_bwd_workspace_limit(1)
    try:
        r = kda.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["v"].clone(), bad)
        torch.cuda.synchronize()
    finally:
        kda.kda_debug_set_bwd_workspace_limit(prev)
    assert kda.device_status() & kda.KDA_DEV_BAD_CU_SEQLENS
    for x in r[:5]:
        assert bool(torch.isnan(x).all())


def test_backward_more_documents_than_ranked():
    """1100 documents, more than the setup kernel ranks by length (their
    state-gradient chains then run in cu_seqlens order): 1 to 5 tokens each,
    two of them longer, with states."""
    rng = np.random.default_rng(73)
    lengths = [int(x) for x in rng.integers(1, 6, size=1100)]
    lengths[17], lengths[900] = 130, 70
    T, H = sum(lengths), 1
    inp = make_inputs(T, H, 73, cu_from_lengths(lengths))
    do = _dout(T, H, 73)
    h0 = initial_states(len(lengths), H, 73)
    dht = np.ascontiguousarray(initial_states(len(lengths), H, 74))
    log(f"[case] bwd {len(lengths)} documents (unranked chain order), T={T}")
    got = _run(inp, do, h0, dht)
    _check(inp, do, got, h0, dht, "bwd 1100 documents")


def test_backward_gate_at_the_lowest_bound():
    """g = -5.5 on every token and channel (the lowest bound the interface
    accepts): every decay split of the backward takes its widest factors,
    exp(+-5.5 x 8) inside a 16-row block, with an initial state and a
    final-state gradient."""
    import dataclasses
    lengths = [150, 64, 17]
    T, H = sum(lengths), 2
    base = make_inputs(T, H, 84, cu_from_lengths(lengths))
    inp = dataclasses.replace(base, g=np.full_like(base.g, -5.5))
    do = _dout(T, H, 84)
    h0 = initial_states(len(lengths), H, 84)
    dht = np.ascontiguousarray(initial_states(len(lengths), H, 85))
    import torch
    import linear_attention_sequence_amd as kda
    d = to_device(inp)
    r = kda.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                      torch.from_numpy(do).to(torch.bfloat16).cuda(), d["cu"],
                      initial_state=torch.from_numpy(h0).cuda(),
                      d_final_state=torch.from_numpy(dht).cuda(), gate_bound=-5.5)
    torch.cuda.synchronize()
    got = [x.cpu().numpy().astype(np.float64) for x in r]
    _check(inp, do, got, h0, dht, "bwd gate at -5.5")
