"""Benchmark of the KDA chunked forward on one MI355X.

One step = one kda_chunk_fwd call (scheduler, pre and main kernels) over the
packed 32768-token stream with H = 32, K = V = 128 and lognormal document
lengths (median 1024, clipped to [17, 8192]).  Inputs are resident in HBM
before the timed region.  Prints ONE JSON line on stdout.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--copy-probe]

``--copy-probe`` adds, after the timed region, two plain device-to-device
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
# Valid only for the kernel source with this sha256; otherwise null.
TRAFFIC = {
    "workload": "packed_lognormal_T32768_H32",
    "kernel_sha256": "0c2a35ce9f2d671b836643ad37f21d63fd9b8c49099ff9b1bb9efdaa47ada5e5",
    "fetch_kib": {"kda_schedule_kernel": 7.2, "kda_pre_kernel": 268263.6, "kda_chunk_fwd_kernel": 686187.5},
    "write_kib": {"kda_schedule_kernel": 2.2, "kda_pre_kernel": 573797.3, "kda_chunk_fwd_kernel": 262174.9},
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
        "kind": "oracle",
        "sample": (f"fp64 token-by-token oracle on all {len(lengths)} documents x "
                   f"{len(sample_heads)} of {H} heads ({n} token-heads, {wall:.1f} s wall); "
                   f"tokens/s = token-heads/s / {H}"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", type=int, default=METRIC_WORKLOAD)
    ap.add_argument("--copy-probe", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the KDA forward here is a single-GPU "
              "operator (multi-GPU sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_attention_sequence_amd as kda
    from kda_workloads import workload_inputs

    kda.load_library()
    w, inp = workload_inputs(args.workload)
    T = w.T
    dev = torch.device("cuda:0")
    q = torch.from_numpy(inp.q).to(torch.bfloat16).to(dev)
    k = torch.from_numpy(inp.k).to(torch.bfloat16).to(dev)
    v = torch.from_numpy(inp.v).to(torch.bfloat16).to(dev)
    g = torch.from_numpy(inp.g).to(dev)
    beta = torch.from_numpy(inp.beta).to(dev)
    cu = torch.from_numpy(np.asarray(inp.cu_seqlens, np.int32)).to(dev)
    out = torch.empty_like(v)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        kda.chunk_fwd(q, k, v, g, beta, cu, out=out)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        kda.chunk_fwd(q, k, v, g, beta, cu, out=out)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
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
    flops = algorithmic_flops(w.lengths, H)
    bytes_alg = BYTES_PER_TOKEN_HEAD * T * H + 4 * (len(w.lengths) + 1)
    tflops = flops / sec / 1e12
    gbs = bytes_alg / sec / 1e9
    log(f"[bench] {w.name}: {ms * 1e3:.1f} us/call, {tokens_per_s:.4g} tokens/s, "
        f"{tflops:.1f} TFLOP/s ({100 * tflops / PEAK_BF16_TFLOPS:.1f}% bf16 MFMA), "
        f"{gbs:.0f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% HBM), wall {wall:.3f}s, status {status}")

    result = {
        "metric": "KDA chunk fwd tokens/sec (H=32, K=V=128) + % bf16 MFMA peak",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "T": T, "H": H, "K": DK, "V": DV, "chunk": CHUNK,
            "documents": len(w.lengths),
            "seed": w.seed,
            "description": w.description,
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
            "traffic": measured_traffic(w.name),
            "algorithmic_bytes": bytes_alg,
            "kernel": "kda_chunk_fwd call (kda_schedule_kernel + kda_pre_kernel + kda_chunk_fwd_kernel)",
            "timing": "HIP events on the launch stream around each call",
        },
        "device_status": status,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, w.lengths, sample_heads=list(range(0, H, 2)))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
