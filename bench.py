"""Benchmark of the KDA chunked forward on one MI355X.

One step = one kda_chunk_fwd call (scheduler, pre and main kernels) over the
packed 32768-token stream with H = 32, K = V = 128 and lognormal document
lengths (median 1024, clipped to [17, 8192]).  Inputs are resident in HBM
before the timed region.  Prints ONE JSON line on stdout.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--copy-probe]
                    [--with-state] [--decode N] [--backward] [--peaks]

``--peaks`` measures the practical ceilings instead: a 1 GiB device-to-device
copy (GB/s) and a large bf16 GEMM through the vendor library (TFLOP/s).
``--backward`` times the chunked backward (kda_chunk_bwd) on the same packed
stream instead: gradients of q, k, v, g, beta for a seeded d_out.
``--decode N`` times one decode step instead: N sequences of one token each
through the token-recurrent entry point, every state updated in place (the
state read and write, 128 KiB per sequence and head, are the algorithmic
bytes).  ``--with-state`` times the state-carrying variant instead (every document
starts from a given fp32 state and returns its final state; the state bytes
are added to the algorithmic bytes).  ``--copy-probe`` adds, after the timed region, two plain device-to-device
copies of 1 GiB: under ``rocprofv3 --pmc FETCH_SIZE`` / ``WRITE_SIZE`` their
counter readings calibrate the chunk kernel's readings to bytes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

H = 32
DK = DV = 128
CHUNK = 64
BYTES_PER_TOKEN_HEAD = 2 * DK + 2 * DK + 2 * DV + 4 * DK + 4 + 2 * DV  # q k v g beta o = 1540
PEAK_BF16_TFLOPS = 2516.6   # dense bf16 MFMA, 256 CU x 2.4 GHz x 4096 flop/clk/CU
PEAK_HBM_GBS = 8000.0       # HBM3E
METRIC_WORKLOAD = 3
KERNEL_SOURCES = [os.path.join(ROOT, "linear_attention_sequence_amd", "csrc", f)
                  for f in ("kda_kernels.h", "kda_fwd.hip", "kda_fwd_state.hip")]
COPY_PROBE_BYTES = 1 << 30

# HBM traffic of one call on the packed 32768-token stream, from two rocprofv3
# --pmc passes (FETCH_SIZE, WRITE_SIZE; KiB per dispatch, mean of 3 calls) per
# kernel of the call, scaled by the same counters' reading for a 1 GiB device
# copy (FETCH_SIZE reads half the bytes a copy moves, WRITE_SIZE all of them).
# Valid only for the kernel sources with this sha256 (kda_kernels.h,
# kda_fwd.hip, kda_fwd_state.hip in that order); otherwise null.
TRAFFIC = {
    "workload": "packed_lognormal_T32768_H32",
    "kernel_sha256": "a78c47199cfe2a636382eb70c2f8258f1d32497dc67fca2e98f5db0e1ff9d0e6",
    "fetch_kib": {"kda_schedule_kernel": 8.4, "kda_pre_kernel": 266835.0, "kda_pc_kernel": 646775.5},
    "write_kib": {"kda_schedule_kernel": 2.3, "kda_pre_kernel": 497732.2, "kda_pc_kernel": 262173.5},
    "fetch_scale": 2.0,
    "write_scale": 1.0,
}


def chunk_flops(c: int, K: int = DK, V: int = DV) -> int:
    """Algorithmic flops of one chunk of c tokens for one head: A and M (lower
    triangles), the two triangular solves, W S / Q S / K^T U (c x K x V each) and
    M U (lower triangle), doubled for multiply + add."""
    return 2 * (3 * c * K * V + K * (3 * c * c - c) // 2 + V * c * c)


def algorithmic_flops(lengths, heads: int) -> int:
    f = 0
    for L in lengths:
        full, tail = divmod(int(L), CHUNK)
        f += full * chunk_flops(CHUNK) + (chunk_flops(tail) if tail else 0)
    return f * heads


def kernel_source_sha256() -> str:
    """sha256 over the kernel sources, in a fixed order."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload_name: str):
    """HBM bytes per launch from the stored counter readings, or None when they
    were taken on another kernel source or workload."""
    t = TRAFFIC
    if t is None or t["workload"] != workload_name or t["kernel_sha256"] != kernel_source_sha256():
        return None
    return (sum(t["fetch_kib"].values()) * t["fetch_scale"] +
            sum(t["write_kib"].values()) * t["write_scale"]) * 1024.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def cpu_baseline(inp, lengths, sample_heads):
    """fp64 oracle on (every document) x (sample_heads), all host cores."""
    import oracle
    cu = np.asarray(inp.cu_seqlens)
    tasks = [(int(a), int(b), h, h + 1) for a, b in zip(cu[:-1], cu[1:]) if b > a
             for h in sample_heads]
    workers = oracle.default_workers()
    try:
        host_cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        host_cores = os.cpu_count()
    t0 = time.perf_counter()
    n = 0
    for (a, b, h0, h1), _ in oracle.kda_tasks(inp.q, inp.k, inp.v, inp.g, inp.beta, tasks,
                                              workers=workers):
        n += (b - a) * (h1 - h0)
    wall = time.perf_counter() - t0
    token_heads_per_s = n / wall
    return {
        "value": token_heads_per_s / H,
        "unit": "tokens/s",
        "cores": workers,
        "host_cores": host_cores,
        "kind": "oracle",
        "sample": (f"fp64 token-by-token oracle on all {len(lengths)} documents x "
                   f"{len(sample_heads)} of {H} heads ({n} token-heads, {wall:.1f} s wall) on "
                   f"{workers} worker processes, one per core up to 12 of the {host_cores} "
                   f"cores this process may use; tokens/s = token-heads/s / {H}"),
    }


def time_steps(step, steps, warmup):
    """Mean ms per step over ``steps`` calls after ``warmup``, HIP events on the
    current stream (the stream the library launches on)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def time_calls(step, steps, warmup, flush=None):
    """Per-call ms of ``steps`` calls after ``warmup``: a pair of HIP events on
    the launch stream around each call.  ``flush`` (untimed, before each call)
    evicts the caches.  Returns (per-call ms list, wall seconds of the timed
    loop)."""
    import torch
    for _ in range(warmup):
        if flush is not None:
            flush()
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        if flush is not None:
            flush()
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [a.elapsed_time(b) for a, b in evs], wall


def cache_flusher(dev):
    """A 1 GiB device write: larger than the 256 MB Infinity Cache and the L2s."""
    import torch
    buf = torch.empty(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)

    def flush():
        buf.fill_(1.0)
    return flush


PEAK_FP32_MFMA_TFLOPS = 157.3  # dense fp32 MFMA
BWD_BYTES_PER_TOKEN_HEAD = 2 * DK + 2 * DK + 2 * DV + 4 * DK + 4 + 2 * DV + 4 * (2 * DK + DV + DK) + 4


def bwd_chunk_flops(c: int, K: int = DK, V: int = DV) -> int:
    """Flops of the products of the chunked backward for one chunk of c tokens
    of one head (fp32 MACs x 2): per-chunk factors (Kk, M, Tb^T Kbar, M^T dO,
    Tb^T P1, F^T, R), the reverse state chain (F^T dS), and the gradient
    products (X, U, dU, dX, dQt, dKt, dKbar, dM, dTb, the inverse's backward,
    the bilinear terms, dD)."""
    tri = c * c // 2
    prep = c * c * K + tri * K + tri * V + tri * V + K * K * c + 2 * K * V * c + c ** 3 // 6
    chain = K * K * V
    grads = (c * K * V + tri * V + (tri * V + c * K * V) + tri * V + 3 * c * V * K + tri * V
             + tri * V + c ** 3 + 3 * tri * K + K * V)
    return 2 * (prep + chain + grads)


def backward_bench(args):
    """kda_chunk_bwd on the packed stream (default workload), d_out seeded."""
    import torch
    import linear_attention_sequence_amd as kda
    from kda_workloads import round_to_bf16, standard_normal, workload_inputs
    w, inp = workload_inputs(args.workload)
    dev = torch.device("cuda:0")
    t = {n: torch.from_numpy(getattr(inp, n)).to(dev) for n in ("q", "k", "v", "g", "beta")}
    for n in ("q", "k", "v"):
        t[n] = t[n].to(torch.bfloat16)
    cu = torch.from_numpy(np.asarray(inp.cu_seqlens, np.int32)).to(dev)
    do = torch.from_numpy(round_to_bf16(standard_normal(inp.v.shape, w.seed, 11))).to(
        torch.bfloat16).to(dev)

    def step():
        kda.chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], do, cu)

    steps = min(args.steps, 10)
    ms = time_steps(step, steps, min(args.warmup, 2))
    status = kda.device_status()
    sec = ms / 1e3
    flops = 0
    for L in w.lengths:
        full, tail = divmod(int(L), CHUNK)
        flops += full * bwd_chunk_flops(CHUNK) + (bwd_chunk_flops(tail) if tail else 0)
    flops *= H
    tflops = flops / sec / 1e12
    bytes_alg = BWD_BYTES_PER_TOKEN_HEAD * w.T * H
    log(f"[bench] backward {w.name}: {ms:.3f} ms/call, {w.T / sec:.4g} tokens/s, "
        f"{tflops:.1f} TFLOP/s fp32 ({100 * tflops / PEAK_FP32_MFMA_TFLOPS:.1f}% fp32 MFMA), "
        f"{bytes_alg / sec / 1e9:.0f} GB/s, status {status}")
    print(json.dumps({
        "metric": "KDA chunk bwd tokens/sec (H=32, K=V=128)",
        "value": w.T / sec, "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": min(args.warmup, 2), "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "H": H, "K": DK, "V": DV, "chunk": CHUNK,
                   "documents": len(w.lengths), "seed": w.seed,
                   "d_out": "bf16 N(0,1), stream 11 of the same seed"},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": PEAK_FP32_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / PEAK_FP32_MFMA_TFLOPS, "traffic": None,
                     "algorithmic_flops": flops, "algorithmic_bytes": bytes_alg,
                     "kernel": "kda_chunk_bwd call (forward with chunk states + setup, prep, "
                               "chain, grads kernels)"},
        "device_status": status,
    }), flush=True)


def peaks_bench():
    """Practical ceilings on this GPU: device copy bandwidth and bf16 GEMM rate."""
    import torch
    dev = torch.device("cuda:0")
    n = COPY_PROBE_BYTES // 2
    src = torch.ones(n, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    ms_copy = time_steps(lambda: dst.copy_(src), 20, 3)
    copy_gbs = 2 * COPY_PROBE_BYTES / (ms_copy / 1e3) / 1e9
    del src, dst
    m = 8192
    a = torch.randn(m, m, device=dev).to(torch.bfloat16)
    b = torch.randn(m, m, device=dev).to(torch.bfloat16)
    c = torch.empty(m, m, device=dev, dtype=torch.bfloat16)
    ms_mm = time_steps(lambda: torch.matmul(a, b, out=c), 20, 3)
    tflops = 2 * m ** 3 / (ms_mm / 1e3) / 1e12
    log(f"[bench] peaks: 1 GiB copy {copy_gbs:.0f} GB/s ({100 * copy_gbs / PEAK_HBM_GBS:.1f}% of "
        f"{PEAK_HBM_GBS:.0f}); bf16 GEMM {m}^3 {tflops:.0f} TFLOP/s "
        f"({100 * tflops / PEAK_BF16_TFLOPS:.1f}% of {PEAK_BF16_TFLOPS:.0f})")
    print(json.dumps({"copy_gbs": copy_gbs, "copy_bytes": 2 * COPY_PROBE_BYTES,
                      "bf16_gemm_tflops": tflops, "gemm_shape": [m, m, m],
                      "peak_hbm_gbs": PEAK_HBM_GBS, "peak_bf16_tflops": PEAK_BF16_TFLOPS}),
          flush=True)


def decode_bench(args):
    """One decode step of N sequences (one token each, H = 32) through
    kda_recurrent_fwd, the state of every sequence updated in place."""
    import torch
    import linear_attention_sequence_amd as kda
    from kda_workloads import cu_from_lengths, initial_states, make_inputs
    N = args.decode
    seed = 7
    inp = make_inputs(N, H, seed, cu_from_lengths([1] * N))
    dev = torch.device("cuda:0")
    t = {name: torch.from_numpy(getattr(inp, name)).to(dev) for name in ("q", "k", "v", "g", "beta")}
    for name in ("q", "k", "v"):
        t[name] = t[name].to(torch.bfloat16)
    cu = torch.from_numpy(np.asarray(inp.cu_seqlens, np.int32)).to(dev)
    state = torch.from_numpy(initial_states(N, H, seed)).to(dev)
    out = torch.empty_like(t["v"])

    def step():
        kda.recurrent_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], cu, initial_state=state,
                          final_state=state, out=out)

    ms = time_steps(step, args.steps, args.warmup)
    status = kda.device_status()
    sec = ms / 1e3
    bytes_alg = N * H * (2 * DK * DV * 4 + BYTES_PER_TOKEN_HEAD) + 4 * (N + 1)
    gbs = bytes_alg / sec / 1e9
    log(f"[bench] decode N={N} H={H}: {ms * 1e3:.1f} us/step, {N / sec:.4g} tokens/s, "
        f"{gbs:.0f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% HBM), status {status}")
    print(json.dumps({
        "metric": f"KDA decode step tokens/sec (N={N} sequences, H={H}, K=V=128)",
        "value": N / sec, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"decode_N{N}_H{H}", "N": N, "H": H, "K": DK, "V": DV,
                   "state": "fp32, updated in place", "seed": seed},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": None,
                     "algorithmic_bytes": bytes_alg,
                     "kernel": "kda_recurrent_fwd call (check + recurrent kernels)"},
        "device_status": status,
    }), flush=True)


def forward_bench(args):
    """kda_chunk_fwd on workload ``args.workload``: one JSON line."""
    import torch
    import linear_attention_sequence_amd as kda
    from kda_workloads import initial_states, workload_inputs
    w, inp = workload_inputs(args.workload)
    T = w.T
    Hw = w.H  # this workload's head count (the headline stream has 32)
    dev = torch.device("cuda:0")
    q = torch.from_numpy(inp.q).to(torch.bfloat16).to(dev)
    k = torch.from_numpy(inp.k).to(torch.bfloat16).to(dev)
    v = torch.from_numpy(inp.v).to(torch.bfloat16).to(dev)
    g = torch.from_numpy(inp.g).to(dev)
    beta = torch.from_numpy(inp.beta).to(dev)
    cu = torch.from_numpy(np.asarray(inp.cu_seqlens, np.int32)).to(dev)
    out = torch.empty_like(v)
    n_docs = len(w.lengths)
    state_kw = {}
    if args.with_state:
        state_kw = dict(initial_state=torch.from_numpy(initial_states(n_docs, Hw, w.seed)).to(dev),
                        output_final_state=True)
    torch.cuda.synchronize()

    def step():
        kda.chunk_fwd(q, k, v, g, beta, cu, out=out, **state_kw)

    per_call, wall = time_calls(step, args.steps, args.warmup)
    ms = float(np.median(per_call))
    flushed = None
    if args.workload in (1, 2):
        # these fit in the Infinity Cache: also time them with it flushed
        fl, _ = time_calls(step, args.steps, args.warmup, flush=cache_flusher(dev))
        flushed = {"median_ms": float(np.median(fl)), "mean_ms": float(np.mean(fl)),
                   "tokens_per_s": T / (float(np.median(fl)) / 1e3),
                   "flush": "1 GiB device write before each call (untimed)"}
    status = kda.device_status()

    if args.copy_probe:
        src = torch.ones(COPY_PROBE_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: 2 x {COPY_PROBE_BYTES} B read + {COPY_PROBE_BYTES} B written")
        del src, dst

    sec = ms / 1e3
    tokens_per_s = T / sec
    flops = algorithmic_flops(w.lengths, Hw)
    bytes_alg = BYTES_PER_TOKEN_HEAD * T * Hw + 4 * (n_docs + 1)
    if args.with_state:
        bytes_alg += 2 * n_docs * Hw * DK * DV * 4   # initial state read, final state written
    tflops = flops / sec / 1e12
    gbs = bytes_alg / sec / 1e9
    log(f"[bench] {w.name}: median {ms * 1e3:.1f} us/call (mean {np.mean(per_call) * 1e3:.1f}, "
        f"min {np.min(per_call) * 1e3:.1f}), {tokens_per_s:.4g} tokens/s, "
        f"{tflops:.1f} TFLOP/s ({100 * tflops / PEAK_BF16_TFLOPS:.1f}% bf16 MFMA), "
        f"{gbs:.0f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% HBM), wall {wall:.3f}s, status {status}")
    if flushed is not None:
        log(f"[bench] {w.name} flushed: median {flushed['median_ms'] * 1e3:.1f} us/call")

    result = {
        "metric": "KDA chunk fwd tokens/sec (H=32, K=V=128) + % bf16 MFMA peak",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "statistic": "median of per-call HIP-event times (warm caches)",
        "mean_ms": float(np.mean(per_call)),
        "min_ms": float(np.min(per_call)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "T": T, "H": Hw, "K": DK, "V": DV, "chunk": CHUNK,
            "documents": len(w.lengths),
            "seed": w.seed,
            "description": w.description,
            **({"state": "initial and final fp32 state per document"} if args.with_state else {}),
        },
        "tflops": tflops,
        "mfma_frac": tflops / PEAK_BF16_TFLOPS,
        "hbm_gbs": gbs,
        "roofline": {
            "bound": "hbm",
            "achieved": gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": gbs / PEAK_HBM_GBS,
            "traffic": None if args.with_state else measured_traffic(w.name),
            "algorithmic_bytes": bytes_alg,
            "kernel": "kda_chunk_fwd call (kda_schedule_kernel + kda_pre_kernel + kda_pc_kernel)",
            "timing": "HIP events on the launch stream around each call",
        },
        "device_status": status,
    }
    if flushed is not None:
        result["flushed"] = flushed
    if not args.no_cpu_baseline and args.workload == METRIC_WORKLOAD:
        result["cpu_baseline"] = cpu_baseline(inp, w.lengths, sample_heads=list(range(0, H, 2)))
    print(json.dumps(result), flush=True)

    del q, k, v, g, beta, cu, out, state_kw
    torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--sweep", action="store_true",
                    help="one JSON line per workload 1..5 (warm; workloads 1-2 also flushed)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", type=int, default=METRIC_WORKLOAD)
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--with-state", action="store_true")
    ap.add_argument("--decode", type=int, default=0, metavar="N")
    ap.add_argument("--backward", action="store_true")
    ap.add_argument("--peaks", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the KDA forward here is a single-GPU "
              "operator (multi-GPU sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)

    import linear_attention_sequence_amd as kda

    kda.load_library()
    if args.decode:
        decode_bench(args)
        return
    if args.backward:
        backward_bench(args)
        return
    if args.peaks:
        peaks_bench()
        return
    if args.sweep:
        for idx in range(1, 6):
            args.workload = idx
            forward_bench(args)
        return
    forward_bench(args)


if __name__ == "__main__":
    main()
