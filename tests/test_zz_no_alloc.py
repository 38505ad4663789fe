"""kda_chunk_fwd_noalloc (the entry point for callers that cannot allocate)
against kda_chunk_fwd, through the C ABI: the same output bit for bit, on two
calls in a row, the second with a smaller input (the scratch array keeps the
first call's contents), and T beyond the scratch rejected before anything runs."""
import numpy as np
import pytest

from kda_gpu_util import check, doc_tasks, log, to_device
from kda_workloads import cu_from_lengths, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_sequence_amd as kda
    kda.load_library()


def _run(entry, d, T, H, out, with_cu=True):
    import torch
    import linear_attention_sequence_amd as kda
    stream = torch.cuda.current_stream().cuda_stream
    rc = entry(d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["g"].data_ptr(),
               d["beta"].data_ptr(), d["cu"].data_ptr() if with_cu else None, T, H, 64, -5.0,
               out.data_ptr(), stream)
    assert rc == kda.KDA_OK, kda.kda_last_error()
    torch.cuda.synchronize()


def test_no_alloc_matches_the_allocating_entry_point_on_two_calls():
    import torch
    import linear_attention_sequence_amd as kda
    cases = [
        # long documents (split by the allocating call), ragged tails, an empty one
        ([3000, 37, 0, 1500, 700, 64, 129], 8, 51),
        # then a smaller stream: the scratch still holds the first call's lists
        ([200, 1, 63, 65], 3, 52),
    ]
    for lengths, H, seed in cases:
        T = sum(lengths)
        log(f"[case] no-alloc T={T} H={H} docs={len(lengths)}")
        inp = make_inputs(T, H, seed, cu_from_lengths(lengths))
        d = to_device(inp)
        ref = torch.empty_like(d["v"])
        got = torch.full_like(d["v"], float("nan"))
        _run(kda.kda_chunk_fwd, d, T, H, ref)
        _run(kda.kda_chunk_fwd_noalloc, d, T, H, got)
        assert kda.device_status() == 0
        assert bool((got.view(torch.int16) == ref.view(torch.int16)).all())
        check(inp, got, doc_tasks(inp.cu_seqlens, H, heads=[0, H - 1]), f"no-alloc T={T}")


def test_no_alloc_single_document_without_cu_seqlens():
    import torch
    import linear_attention_sequence_amd as kda
    T, H = 1000, 2
    inp = make_inputs(T, H, 53, cu_from_lengths([T]))
    d = to_device(inp)
    ref = torch.empty_like(d["v"])
    got = torch.empty_like(d["v"])
    _run(kda.kda_chunk_fwd, d, T, H, ref, with_cu=False)
    _run(kda.kda_chunk_fwd_noalloc, d, T, H, got, with_cu=False)
    assert bool((got.view(torch.int16) == ref.view(torch.int16)).all())


def test_no_alloc_rejects_a_stream_beyond_its_scratch():
    import linear_attention_sequence_amd as kda
    P = 1 << 20  # never dereferenced: the call fails on the host first
    rc = kda.kda_chunk_fwd_noalloc(P, P, P, P, P, None, 9_000_000, 1, 64, -5.0, P, None)
    assert rc == kda.KDA_ERR_BAD_SHAPE
    assert "scratch" in kda.kda_last_error()
    log(f"[case] no-alloc rejects T=9e6: {kda.kda_last_error()}")
