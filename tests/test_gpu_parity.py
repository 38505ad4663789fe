"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bar: relative L2 error <= 5e-3 and max absolute error <= 3e-2 on the same
seeded inputs.  Small cases compare every output; the full-size packed
streams compare sampled (document, head) tasks, each of which the oracle
computes in full, in the same launch configuration the benchmark times."""
import numpy as np
import pytest

import oracle
from kda_gpu_util import check, compare_tasks, doc_tasks, log, run_gpu, set_split, to_device
from kda_workloads import (Inputs, cu_from_lengths, make_inputs, one_hot_keys, with_gate_scale,
                           workload, workload_inputs)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_sequence_amd as kda
    kda.load_library()


def _small(T, H, seed, lengths, **kw):
    return make_inputs(T, H, seed, cu_from_lengths(lengths), **kw)


# ---------------------------------------------------------------- workloads

def test_workload1_single_doc_T256():
    w, inp = workload_inputs(1)
    log(f"[case] workload 1 {w.name}")
    o = run_gpu(inp)
    check(inp, o, doc_tasks(inp.cu_seqlens, w.H), w.name)


def test_workload2_single_doc_T4096():
    w, inp = workload_inputs(2)
    log(f"[case] workload 2 {w.name}")
    o = run_gpu(inp)
    check(inp, o, doc_tasks(inp.cu_seqlens, w.H), w.name)


def test_workload3_packed_lognormal_sampled_heads():
    w, inp = workload_inputs(3)
    log(f"[case] workload 3 {w.name} docs={len(w.lengths)}")
    o = run_gpu(inp)
    check(inp, o, doc_tasks(inp.cu_seqlens, w.H, heads=[0, 7, 13, 22, 31]), w.name)


def test_workload4_dense_batch_sampled():
    """Every one of the 8 documents of 8192 tokens on 4 heads, the last head
    included."""
    w, inp = workload_inputs(4)
    log(f"[case] workload 4 {w.name}")
    o = run_gpu(inp)
    check(inp, o, doc_tasks(inp.cu_seqlens, w.H, heads=[0, 9, 17, 31]), w.name)


def test_workload5_long_plus_short_sampled():
    """The 65,536-token document on 3 heads, every short document on 2."""
    w, inp = workload_inputs(5)
    log(f"[case] workload 5 {w.name} docs={len(w.lengths)}")
    o = run_gpu(inp)
    cu = inp.cu_seqlens
    tasks = [(0, int(cu[1]), h, h + 1) for h in (0, 5, 31)] + doc_tasks(cu[1:], w.H, heads=[2, 29])
    check(inp, o, tasks, w.name)


def test_long_document_slow_decay_split_and_fused():
    """One 65,536-token document (1024 chunks) with a slow decay, so that the
    state carries across chunks all the way (the workloads' gate forgets it
    within a chunk): the split path (its long sequential chain) and the fused
    path give the same bits, and both match the oracle."""
    import torch
    T, H = 65536, 1
    inp = with_gate_scale(_small(T, H, 42, [T]), 42, -0.05)
    log("[case] one 65536-token document, g = -0.05 sigmoid, split then fused")
    set_split("always")
    a = run_gpu(inp)
    set_split("never")
    b = run_gpu(inp)
    assert bool((_bits(a) == _bits(b)).all())
    assert bool(torch.isfinite(a.float()).all())
    check(inp, a, doc_tasks(inp.cu_seqlens, H), "65536 tokens, gate -0.05*sigmoid")


# ---------------------------------------------------------------- special inputs

def test_beta_zero_gives_exact_zeros():
    inp = _small(300, 3, 21, [100, 200])
    inp.beta[:] = 0.0
    o = run_gpu(inp)
    assert int((o != 0).sum()) == 0


def test_all_length_one_documents():
    T, H = 4096, 4
    inp = _small(T, H, 22, [1] * T)
    o = run_gpu(inp)
    check(inp, o, doc_tasks(inp.cu_seqlens, H, heads=[0, 3])[:600], "all length-1 documents")
    # closed form at T = 1: o = scale * beta * (qh . kh) v
    qn = oracle.l2_normalise(inp.q)
    kn = oracle.l2_normalise(inp.k)
    ref = 128 ** -0.5 * inp.beta[..., None] * (qn * kn).sum(-1, keepdims=True) * inp.v
    got = o.float().cpu().numpy()
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    log(f"[parity] length-1 closed form relL2={rel:.3e}")
    assert rel <= 5e-3


@pytest.mark.parametrize("gate_scale,T", [(-0.05, 2048), (0.0, 512), (0.0, 8192)])
def test_slow_decay_exercises_the_state(gate_scale, T):
    """The state carries across every chunk; g = 0 (no decay at all) is the
    hardest case for the bf16 copy of S in the products (relL2 grows slowly
    with the document length: ~3.8e-3 at 512 tokens, ~4.2e-3 at 8192)."""
    H = 4
    inp = with_gate_scale(_small(T, H, 23, [T]), 23, gate_scale)
    o = run_gpu(inp)
    check(inp, o, doc_tasks(inp.cu_seqlens, H), f"gate {gate_scale}*sigmoid T={T}")


def test_one_hot_keys():
    T, H = 1024, 4
    inp = _small(T, H, 24, [300, 724])
    inp.k[:] = one_hot_keys(T, H, 24)
    inp = with_gate_scale(inp, 24, -0.3)
    o = run_gpu(inp)
    check(inp, o, doc_tasks(inp.cu_seqlens, H), "one-hot keys")


def test_ragged_document_lengths():
    lengths = [1, 2, 15, 16, 17, 63, 64, 65, 0, 127, 128, 129, 200, 31]
    T, H = sum(lengths), 3
    inp = _small(T, H, 25, lengths)
    o = run_gpu(inp)
    check(inp, o, doc_tasks(inp.cu_seqlens, H), "ragged lengths")


def test_gate_at_the_bound():
    T, H = 300, 2
    inp = _small(T, H, 26, [T])
    inp.g[:] = -5.0
    inp.g[::7] = -0.001
    o = run_gpu(inp)
    check(inp, o, doc_tasks(inp.cu_seqlens, H), "gate at the bound")


# ---------------------------------------------------------------- split documents
# Long documents may be "split": their chunks' state-independent part runs on
# all CUs first and only the sequential chain stays per (document, head).
# The split policy test hook forces the choice; both paths must give
# identical bits.

def _bits(o):
    import torch
    return o.view(torch.int16)


def test_split_path_is_bit_identical_to_fused():
    lengths = [513, 64 * 8, 1000, 37, 700, 2000, 1, 450]
    T, H = sum(lengths), 3
    inp = _small(T, H, 31, lengths)
    set_split("never")
    a = run_gpu(inp)
    set_split("always")
    b = run_gpu(inp)
    assert bool((_bits(a) == _bits(b)).all())
    check(inp, b, doc_tasks(inp.cu_seqlens, H), "split documents")


@pytest.mark.parametrize("cu", [True, False])
def test_split_long_document_carries_the_state(cu):
    T, H = 2048 + 37, 4
    inp = with_gate_scale(_small(T, H, 32, [T]), 32, -0.05)
    set_split("never")
    a = run_gpu(inp, cu=cu)
    set_split("always")
    b = run_gpu(inp, cu=cu)
    assert bool((_bits(a) == _bits(b)).all())
    check(inp, b, doc_tasks(inp.cu_seqlens, H), "split, slow decay")


# ---------------------------------------------------------------- value range
# Tb X and M U run on fp16 operands; values that would not fit are brought in
# range by exact powers of two.  Large v exercise those paths: the output is
# linear in v, so GPU(2^k v) / 2^k must match the oracle on v.

def _scaled_v(inp, k):
    import dataclasses
    return dataclasses.replace(inp, v=inp.v * np.float32(2.0 ** k))


@pytest.mark.parametrize("k", [12, 20, 40])
def test_large_values_stay_in_range(k):
    import torch
    T, H = 700, 2
    base = with_gate_scale(_small(T, H, 33, [300, 400]), 33, -0.05)
    for policy in ("never", "always"):
        set_split(policy)
        o = run_gpu(_scaled_v(base, k))
        assert bool(torch.isfinite(o.float()).all())
        o1 = (o.float() * 2.0 ** -k).to(torch.bfloat16)
        check(base, o1, doc_tasks(base.cu_seqlens, H), f"v * 2^{k} ({policy})")


@pytest.mark.parametrize("v_scale,beta_scale", [(1e-6, 1.0), (1.0, 1e-5), (1e-6, 1e-5)])
def test_small_values_keep_their_precision(v_scale, beta_scale):
    """X, U and Tb are fp16 operands behind a power-of-two scale that also
    scales small values up, out of the fp16 subnormal range (v is any bf16 and
    beta any finite value)."""
    import dataclasses
    T, H = 700, 2
    base = with_gate_scale(_small(T, H, 36, [300, 400]), 36, -0.05)
    inp = dataclasses.replace(base, v=(base.v * np.float32(v_scale)),
                              beta=(base.beta * np.float32(beta_scale)))
    from kda_workloads import round_to_bf16
    inp = dataclasses.replace(inp, v=round_to_bf16(inp.v))
    for policy in ("never", "always"):
        set_split(policy)
        o = run_gpu(inp)
        rel, mx = compare_tasks(inp, o, doc_tasks(inp.cu_seqlens, H))
        ref_scale = float(np.abs(oracle.kda_forward(inp.q, inp.k, inp.v, inp.g, inp.beta,
                                                    inp.cu_seqlens)).max())
        log(f"[parity] v*{v_scale} beta*{beta_scale} ({policy}): relL2={rel:.3e} "
            f"maxabs={mx:.3e} (output scale {ref_scale:.3e})")
        assert rel <= 5e-3, rel
        assert mx <= 3e-2 * ref_scale, mx


def test_large_beta():
    T, H = 640, 2
    inp = with_gate_scale(_small(T, H, 34, [T]), 34, -0.3)
    inp.beta[:] = 1.9
    for policy in ("never", "always"):
        set_split(policy)
        o = run_gpu(inp)
        check(inp, o, doc_tasks(inp.cu_seqlens, H), f"beta 1.9 ({policy})")


@pytest.mark.parametrize("H", [1, 5, 64])
def test_head_counts(H):
    lengths = [37, 600, 64, 129]
    T = sum(lengths)
    inp = with_gate_scale(_small(T, H, 35 + H, lengths), 35 + H, -0.5)
    set_split("never")
    a = run_gpu(inp)
    set_split("always")
    b = run_gpu(inp)
    assert bool((_bits(a) == _bits(b)).all())
    heads = sorted({0, H // 2, H - 1})
    check(inp, b, doc_tasks(inp.cu_seqlens, H, heads=heads), f"H={H}")


def test_gate_at_the_lowest_bound():
    import torch
    import linear_attention_sequence_amd as kda
    T, H = 300, 2
    inp = _small(T, H, 40, [T])
    inp.g[:] = -5.5
    inp.g[::5] = -0.01
    d = to_device(inp)
    o, _ = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], gate_bound=-5.5)
    torch.cuda.synchronize()
    assert kda.device_status() == 0
    check(inp, o, doc_tasks(inp.cu_seqlens, H), "gate at -5.5")


def test_more_splittable_documents_than_candidates():
    # 1100 documents of 9 chunks: the scheduler examines the longest 1024 for
    # splitting, the rest stay fused; the output is the same bit for bit
    lengths = [515] * 1100
    T, H = sum(lengths), 1
    inp = _small(T, H, 41, lengths)
    set_split("never")
    a = run_gpu(inp)
    set_split("always")
    b = run_gpu(inp)
    assert bool((_bits(a) == _bits(b)).all())
    cu = inp.cu_seqlens
    check(inp, b, [(int(cu[i]), int(cu[i + 1]), 0, 1) for i in (0, 555, 1099)], "1100 split candidates")


# ---------------------------------------------------------------- layouts

def test_cu_none_is_one_document():
    T, H = 333, 2
    inp = _small(T, H, 27, [T])
    a = run_gpu(inp, cu=True)
    b = run_gpu(inp, cu=False)
    assert bool((a == b).all())
    check(inp, b, doc_tasks(inp.cu_seqlens, H), "cu_seqlens=None")


def test_dense_batch_is_packed_documents():
    import torch
    import linear_attention_sequence_amd as kda
    B, T, H = 3, 100, 2
    inp = _small(B * T, H, 28, [T] * B)
    d = to_device(inp)
    packed, _ = kda.chunk_fwd(d["q"][None], d["k"][None], d["v"][None], d["g"][None],
                              d["beta"][None], d["cu"])
    dense, _ = kda.chunk_fwd(d["q"].view(B, T, H, 128), d["k"].view(B, T, H, 128),
                             d["v"].view(B, T, H, 128), d["g"].view(B, T, H, 128),
                             d["beta"].view(B, T, H))
    torch.cuda.synchronize()
    assert bool((packed.view(B, T, H, 128) == dense).all())


def test_deterministic():
    import torch
    import linear_attention_sequence_amd as kda
    w, inp = workload_inputs(3)
    d = to_device(inp)
    a, _ = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"])
    b, _ = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"])
    torch.cuda.synchronize()
    assert bool((a.view(torch.int16) == b.view(torch.int16)).all())


def test_empty_stream():
    import torch
    import linear_attention_sequence_amd as kda
    z = torch.zeros(0, 2, 128, dtype=torch.bfloat16, device="cuda")
    o, none = kda.chunk_fwd(z, z, z, z.float(), torch.zeros(0, 2, device="cuda"), None)
    assert o.numel() == 0 and none is None


# ---------------------------------------------------------------- device-side errors

def test_bad_cu_seqlens_sets_status_and_nan():
    import torch
    import linear_attention_sequence_amd as kda
    T, H = 128, 2
    inp = _small(T, H, 29, [T])
    d = to_device(inp)
    assert kda.device_status() == 0
    for bad in ([0, 100, 90, 128], [1, 128], [0, 130, 128]):
        cu = torch.tensor(bad, dtype=torch.int32, device="cuda")
        o, _ = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], cu)
        st = kda.device_status()
        assert st & kda.KDA_DEV_BAD_CU_SEQLENS, bad
        assert bool(torch.isnan(o.float()).all()), bad
    assert kda.device_status() == 0


def test_gate_out_of_range_is_flagged():
    import linear_attention_sequence_amd as kda
    T, H = 64, 1
    inp = _small(T, H, 30, [T])
    d = to_device(inp)
    assert kda.device_status() == 0
    kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"])
    assert kda.device_status() == 0
    d["g"][5, 0, 3] = 0.5
    kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"])
    assert kda.device_status() & kda.KDA_DEV_GATE_RANGE


def test_binding_rejects_bad_tensors():
    import torch
    import linear_attention_sequence_amd as kda
    q = torch.zeros(1, 64, 2, 128, dtype=torch.bfloat16, device="cuda")
    g = torch.zeros(1, 64, 2, 128, device="cuda")
    beta = torch.zeros(1, 64, 2, device="cuda")
    with pytest.raises(ValueError, match="k must be"):
        kda.chunk_fwd(q, q.float(), q, g, beta)
    with pytest.raises(ValueError, match="head dim"):
        kda.chunk_fwd(q[..., :64].contiguous(), q[..., :64].contiguous(), q[..., :64].contiguous(),
                      g[..., :64].contiguous(), beta)
    with pytest.raises(ValueError, match="cu_seqlens must be an int32"):
        kda.chunk_fwd(q, q, q, g, beta, torch.tensor([0, 64], device="cuda"))
