"""Shared helpers of the GPU parity tests: move seeded inputs to the GPU, run
the library, and compare against the fp64 oracle task by task."""
import sys

import numpy as np

import oracle

REL_L2_TOL = 5e-3
MAX_ABS_TOL = 3e-2


def set_split(policy):
    """Force the split-document policy of the library ("never", "auto",
    "always"); the conftest fixture puts it back to "auto" after each test."""
    import linear_attention_sequence_amd as kda
    kda.set_split_policy(policy)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp):
    import torch
    dev = torch.device("cuda:0")
    return dict(
        q=torch.from_numpy(inp.q).to(torch.bfloat16).to(dev),
        k=torch.from_numpy(inp.k).to(torch.bfloat16).to(dev),
        v=torch.from_numpy(inp.v).to(torch.bfloat16).to(dev),
        g=torch.from_numpy(inp.g).to(dev),
        beta=torch.from_numpy(inp.beta).to(dev),
        cu=torch.from_numpy(np.ascontiguousarray(inp.cu_seqlens, np.int32)).to(dev),
    )


def run_gpu(inp, cu=True):
    import torch
    import linear_attention_sequence_amd as kda
    d = to_device(inp)
    o, _ = kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"] if cu else None)
    torch.cuda.synchronize()
    return o


def compare_tasks(inp, o_gpu, tasks, workers=None):
    """Compare the GPU output against the oracle on (a, b, h0, h1) tasks.
    Returns (relL2, maxabs) over all tasks together."""
    num = den = 0.0
    mx = 0.0
    for (a, b, h0, h1), ref in oracle.kda_tasks(inp.q, inp.k, inp.v, inp.g, inp.beta, tasks,
                                                workers=workers):
        got = o_gpu[a:b, h0:h1].float().cpu().numpy().astype(np.float64)
        d = got - ref
        num += float((d * d).sum())
        den += float((ref * ref).sum())
        mx = max(mx, float(np.abs(d).max()) if d.size else 0.0)
    rel = np.sqrt(num / den) if den > 0 else np.sqrt(num)
    return rel, mx


def doc_tasks(cu, H, heads=None):
    heads = range(H) if heads is None else heads
    out = []
    for a, b in zip(cu[:-1], cu[1:]):
        if b > a:
            for h in heads:
                out.append((int(a), int(b), h, h + 1))
    return out


def check(inp, o_gpu, tasks, label, rel_tol=REL_L2_TOL, abs_tol=MAX_ABS_TOL):
    rel, mx = compare_tasks(inp, o_gpu, tasks)
    log(f"[parity] {label}: relL2={rel:.3e} maxabs={mx:.3e} tasks={len(tasks)}")
    assert rel <= rel_tol, (label, rel)
    assert mx <= abs_tol, (label, mx)
    return rel, mx
