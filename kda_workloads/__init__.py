"""Seeded synthetic inputs for the KDA chunked forward.

This module only draws random numbers and lays out documents. It holds none
of the method's arithmetic, so both the fp64 oracle (``oracle/``) and the HIP
path (``linear_attention_sequence_amd``) may consume what it produces without
sharing any computation.

Recipe (one place, used everywhere):

* Every tensor is filled in blocks of ``BLOCK`` elements.  Block ``j`` of
  stream ``s`` under seed ``seed`` is drawn from
  ``PCG64(SeedSequence(seed, spawn_key=(s, j)))``.  The result therefore does
  not depend on how many threads fill it.
* Streams: 0 document lengths, 1 q, 2 k, 3 v, 4 the gate pre-activation
  ``z_g``, 5 the beta pre-activation ``z_b``, 6 initial states.
* ``q, k, v ~ N(0, 1)`` drawn in fp32 and rounded to bf16 (round to nearest
  even) before anyone sees them; both sides consume the same bf16 values.
* ``g = gate_scale * sigmoid(z_g)`` in fp32 with ``gate_scale = -5``: a log
  decay in ``(-5, 0)`` per token, head and key channel.
* ``beta = sigmoid(z_b)`` in fp32, one value per token and head.
* Initial states (for the state-carrying variant): ``0.2 * N(0, 1)`` in fp32,
  one K x V matrix per document and head (0.2 is about the spread of a state
  a document leaves behind under a slow decay).

The five workloads are the packed streams the Kimi Delta Attention pages
specialise the fused forward for (head dims K = V = 128, packed batch-1
layout with int32 ``cu_seqlens``, a dense batch viewed as packed documents;
kda_fused page, package docstring).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HEAD_DIM = 128
BLOCK = 1 << 22

STREAM_LENGTHS = 0
STREAM_Q = 1
STREAM_K = 2
STREAM_V = 3
STREAM_ZG = 4
STREAM_ZB = 5
STREAM_STATE = 6


def _rng(seed: int, stream: int, block: int = 0) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream, block))))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def standard_normal(shape, seed: int, stream: int) -> np.ndarray:
    """fp32 N(0,1) array of ``shape``, filled block-wise (thread-count independent)."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    nblk = (n + BLOCK - 1) // BLOCK

    def fill(j):
        _rng(seed, stream, j).standard_normal(out=out[j * BLOCK:(j + 1) * BLOCK],
                                              dtype=np.float32)

    if nblk <= 1:
        for j in range(nblk):
            fill(j)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def sigmoid_f32(z: np.ndarray) -> np.ndarray:
    """Logistic function evaluated in fp64 and stored as fp32 (input shaping only)."""
    out = np.empty(z.shape, np.float32)
    flat_in = z.reshape(-1)
    flat_out = out.reshape(-1)
    step = BLOCK

    def work(j):
        s = slice(j * step, (j + 1) * step)
        flat_out[s] = (1.0 / (1.0 + np.exp(-flat_in[s].astype(np.float64)))).astype(np.float32)

    nblk = (flat_in.size + step - 1) // step
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(nblk)))
    return out


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returned as fp32 holding bf16 values."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    out = np.empty_like(u)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)

    def work(j):
        s = slice(j * BLOCK, (j + 1) * BLOCK)
        a = flat_u[s].astype(np.uint64)
        r = (a + 0x7FFF + ((a >> 16) & 1)) >> 16
        flat_o[s] = (r << 16).astype(np.uint32)

    nblk = (flat_u.size + BLOCK - 1) // BLOCK
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(nblk)))
    return out.view(np.float32).reshape(x.shape)


# ----------------------------------------------------------------------------
# document layouts
# ----------------------------------------------------------------------------

def cu_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, np.int64)
    cu = np.zeros(len(lengths) + 1, np.int64)
    np.cumsum(lengths, out=cu[1:])
    return cu.astype(np.int32)


def lognormal_lengths(total: int, seed: int, median: int = 1024, lo: int = 17,
                      hi: int = 8192, sigma: float = 1.0) -> list[int]:
    """Lengths ``clip(rint(median*exp(sigma*z)), lo, hi)`` drawn until they reach
    ``total``; the last one is trimmed so they sum to ``total`` exactly."""
    rng = _rng(seed, STREAM_LENGTHS)
    out, acc = [], 0
    while acc < total:
        z = rng.standard_normal()
        L = int(np.clip(np.rint(median * np.exp(sigma * z)), lo, hi))
        L = min(L, total - acc)
        out.append(L)
        acc += L
    return out


def long_plus_short_lengths(total: int, long_len: int, seed: int, lo: int = 1,
                            hi: int = 200) -> list[int]:
    """One ``long_len`` document, then uniform ``[lo, hi]`` lengths filling the rest
    (the last one trimmed)."""
    rng = _rng(seed, STREAM_LENGTHS)
    out, acc = [long_len], long_len
    while acc < total:
        L = int(rng.integers(lo, hi + 1))
        L = min(L, total - acc)
        out.append(L)
        acc += L
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    seed: int
    lengths: tuple
    description: str

    @property
    def cu_seqlens(self) -> np.ndarray:
        return cu_from_lengths(self.lengths)


def workload(idx: int) -> Workload:
    """The five packed streams, 1-based like the configuration list they come from."""
    if idx == 1:
        return Workload("single_doc_T256_H2", 256, 2, 0, (256,),
                        "one document, T=256, H=2; fp32 draws rounded to bf16")
    if idx == 2:
        return Workload("single_doc_T4096_H32", 4096, 32, 1, (4096,),
                        "one document, T=4096, H=32")
    if idx == 3:
        L = lognormal_lengths(32768, seed=2)
        return Workload("packed_lognormal_T32768_H32", 32768, 32, 2, tuple(L),
                        "packed stream, lognormal lengths (median 1024, clip [17, 8192])")
    if idx == 4:
        return Workload("dense_B8_T8192_H32", 65536, 32, 3, (8192,) * 8,
                        "dense batch of 8 x 8192 viewed as packed documents")
    if idx == 5:
        L = long_plus_short_lengths(131072, 65536, seed=4)
        return Workload("long_plus_short_T131072_H32", 131072, 32, 4, tuple(L),
                        "one 65536-token document then U[1,200] documents")
    raise ValueError(f"no workload {idx}")


@dataclasses.dataclass
class Inputs:
    """Host-side inputs. q, k, v hold bf16 values stored as fp32."""
    q: np.ndarray      # [T, H, K] fp32 (bf16-exact)
    k: np.ndarray      # [T, H, K] fp32 (bf16-exact)
    v: np.ndarray      # [T, H, V] fp32 (bf16-exact)
    g: np.ndarray      # [T, H, K] fp32
    beta: np.ndarray   # [T, H] fp32
    cu_seqlens: np.ndarray  # [N+1] int32

    @property
    def T(self) -> int:
        return self.q.shape[0]

    @property
    def H(self) -> int:
        return self.q.shape[1]


def make_inputs(T: int, H: int, seed: int, cu_seqlens, K: int = HEAD_DIM, V: int = HEAD_DIM,
                gate_scale: float = -5.0) -> Inputs:
    q = round_to_bf16(standard_normal((T, H, K), seed, STREAM_Q))
    k = round_to_bf16(standard_normal((T, H, K), seed, STREAM_K))
    v = round_to_bf16(standard_normal((T, H, V), seed, STREAM_V))
    zg = standard_normal((T, H, K), seed, STREAM_ZG)
    g = sigmoid_f32(zg)
    del zg
    g *= np.float32(gate_scale)
    zb = standard_normal((T, H), seed, STREAM_ZB)
    beta = sigmoid_f32(zb)
    return Inputs(q, k, v, g, beta, np.asarray(cu_seqlens, np.int32))


def workload_inputs(idx: int) -> tuple[Workload, Inputs]:
    w = workload(idx)
    return w, make_inputs(w.T, w.H, w.seed, w.cu_seqlens)


# ----------------------------------------------------------------------------
# special-case variants (parity only)
# ----------------------------------------------------------------------------

def with_gate_scale(inp: Inputs, seed: int, gate_scale: float) -> Inputs:
    """Same draws, gate ``gate_scale*sigmoid(z_g)`` (e.g. -0.05 for a slow decay)."""
    zg = standard_normal(inp.g.shape, seed, STREAM_ZG)
    g = sigmoid_f32(zg)
    g *= np.float32(gate_scale)
    return dataclasses.replace(inp, g=g)


def initial_states(n_docs: int, H: int, seed: int, std: float = 0.2, K: int = HEAD_DIM,
                   V: int = HEAD_DIM) -> np.ndarray:
    """fp32 [n_docs, H, K, V] states ``std * N(0, 1)``."""
    s = standard_normal((n_docs, H, K, V), seed, STREAM_STATE)
    s *= np.float32(std)
    return s


def one_hot_keys(T: int, H: int, seed: int, K: int = HEAD_DIM) -> np.ndarray:
    """Keys that are a random positive multiple of a random unit vector e_c."""
    rng = _rng(seed, 17)
    ch = rng.integers(0, K, size=(T, H))
    mag = rng.uniform(0.5, 2.0, size=(T, H)).astype(np.float32)
    k = np.zeros((T, H, K), np.float32)
    np.put_along_axis(k, ch[..., None], mag[..., None], axis=-1)
    return round_to_bf16(k)
