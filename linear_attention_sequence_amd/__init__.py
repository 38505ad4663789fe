"""Kimi Delta Attention (KDA) chunked forward on MI355X (gfx950).

Thin Python binding over the C ABI in ``include/kda.h`` (``libkda.so``, built
in-tree).  Torch is used only for device memory and streams: every step of
the forward runs in the library's HIP kernels.  There is no CPU or PyTorch
fallback: if the library is missing, importing works but every call raises.

The tensor-level entry point mirrors the fused path of the K3 model
(page "nemo_automodel.components.models.kimi_k3.kda_fused"):
``chunk_fwd(q, k, v, g, beta, cu_seqlens)`` returns ``(o, None)`` like
``fused_chunk_kda``; ``unsupported_reason`` names the first violated condition
like ``fused_kda_unsupported_reason``.  ``initial_state`` /
``output_final_state`` add the state input and output of FLA's ``chunk_kda``
(through ``kda_chunk_fwd_state``); ``recurrent_fwd`` is the token-recurrent
form of the same operator (``kda_recurrent_fwd``) for decoding.
"""
from __future__ import annotations

import ctypes
import math
import os

HEAD_DIM = 128
CHUNK = 64
DEFAULT_GATE_BOUND = -5.0

KDA_OK = 0
KDA_ERR_NULL_PTR = -1
KDA_ERR_BAD_SHAPE = -2
KDA_ERR_UNSUPPORTED = -3
KDA_ERR_ALIGN = -4
KDA_ERR_HIP = -5
KDA_ERR_ALLOC = -6
KDA_DEV_BAD_CU_SEQLENS = 1
KDA_DEV_GATE_RANGE = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")
_lib = None


class KDAError(RuntimeError):
    """A non-zero return of the C ABI."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"kda_chunk_fwd failed ({code}): {msg}")
        self.code = code


def load_library():
    """Load ``libkda.so`` (raises if it was not built)."""
    global _lib
    if _lib is None:
        # torch first: its HIP runtime and the one libkda.so links carry the same
        # soname, and the library must use the runtime torch's tensors live in
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                "(there is no fallback implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        lib.kda_chunk_fwd.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
        lib.kda_chunk_fwd.restype = ctypes.c_int
        lib.kda_chunk_fwd_noalloc.argtypes = lib.kda_chunk_fwd.argtypes
        lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
        lib.kda_chunk_fwd_state.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p]
        lib.kda_chunk_fwd_state.restype = ctypes.c_int
        lib.kda_recurrent_fwd.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.kda_recurrent_fwd.restype = ctypes.c_int
        lib.kda_chunk_bwd.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
            ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p]
        lib.kda_chunk_bwd.restype = ctypes.c_int
        lib.kda_last_error.argtypes = []
        lib.kda_last_error.restype = ctypes.c_char_p
        lib.kda_device_status.argtypes = [ctypes.c_void_p]
        lib.kda_device_status.restype = ctypes.c_int
        lib.kda_debug_set_split_policy.argtypes = [ctypes.c_int]
        lib.kda_debug_set_split_policy.restype = ctypes.c_int
        lib.kda_debug_set_bwd_workspace_limit.argtypes = [ctypes.c_uint64]
        lib.kda_debug_set_bwd_workspace_limit.restype = ctypes.c_uint64
        _lib = lib
    return _lib


# ---------------------------------------------------------------------------
# same-name wrappers of the C entry points (argument marshalling only)
# ---------------------------------------------------------------------------

def kda_chunk_fwd(q, k, v, g, beta, cu_seqlens, T, H, chunk, gate_bound, out, stream) -> int:
    """Call the C entry point with raw addresses (ints or None); returns its status."""
    lib = load_library()
    return lib.kda_chunk_fwd(q, k, v, g, beta, cu_seqlens, int(T), int(H), int(chunk),
                             float(gate_bound), out, stream)


def kda_chunk_fwd_noalloc(q, k, v, g, beta, cu_seqlens, T, H, chunk, gate_bound, out,
                          stream) -> int:
    """Call the C entry point with raw addresses (ints or None); returns its status."""
    lib = load_library()
    return lib.kda_chunk_fwd_noalloc(q, k, v, g, beta, cu_seqlens, int(T), int(H), int(chunk),
                                     float(gate_bound), out, stream)


def kda_chunk_fwd_state(q, k, v, g, beta, cu_seqlens, n_docs, T, H, chunk, gate_bound,
                        initial_state, final_state, out, stream) -> int:
    """Call the C entry point with raw addresses (ints or None); returns its status."""
    lib = load_library()
    return lib.kda_chunk_fwd_state(q, k, v, g, beta, cu_seqlens, int(n_docs), int(T), int(H),
                                   int(chunk), float(gate_bound), initial_state, final_state,
                                   out, stream)


def kda_recurrent_fwd(q, k, v, g, beta, cu_seqlens, n_docs, T, H, initial_state, final_state,
                      out, stream) -> int:
    """Call the C entry point with raw addresses (ints or None); returns its status."""
    lib = load_library()
    return lib.kda_recurrent_fwd(q, k, v, g, beta, cu_seqlens, int(n_docs), int(T), int(H),
                                 initial_state, final_state, out, stream)


def kda_chunk_bwd(q, k, v, g, beta, cu_seqlens, n_docs, T, H, chunk, gate_bound, initial_state,
                  d_out, d_final_state, dq, dk, dv, dg, dbeta, d_initial_state, stream) -> int:
    """Call the C entry point with raw addresses (ints or None); returns its status."""
    lib = load_library()
    return lib.kda_chunk_bwd(q, k, v, g, beta, cu_seqlens, int(n_docs), int(T), int(H),
                             int(chunk), float(gate_bound), initial_state, d_out, d_final_state,
                             dq, dk, dv, dg, dbeta, d_initial_state, stream)


def kda_last_error() -> str:
    return load_library().kda_last_error().decode()


def kda_device_status(stream=None) -> int:
    return load_library().kda_device_status(stream)


def kda_debug_set_split_policy(policy: int) -> int:
    return load_library().kda_debug_set_split_policy(int(policy))


def kda_debug_set_bwd_workspace_limit(n_bytes: int) -> int:
    return int(load_library().kda_debug_set_bwd_workspace_limit(int(n_bytes)))


SPLIT_POLICIES = {"never": 0, "auto": 1, "always": 2}


def set_split_policy(name: str) -> str:
    """Force the choice of split documents (test hook): ``"never"``,
    ``"auto"`` (the default) or ``"always"``.  Returns the previous name."""
    prev = kda_debug_set_split_policy(SPLIT_POLICIES[name])
    if prev < 0:
        raise KDAError(prev, "bad split policy")
    return {v: k for k, v in SPLIT_POLICIES.items()}[prev]


# ---------------------------------------------------------------------------
# tensor-level API
# ---------------------------------------------------------------------------

def _layout(q):
    """Return (B, T) of a [B, T, H, D] or [T, H, D] tensor."""
    if q.dim() == 4:
        return q.shape[0], q.shape[1]
    if q.dim() == 3:
        return 1, q.shape[0]
    return None


def unsupported_reason(q, k, v, g, beta, cu_seqlens=None, *, chunk: int = CHUNK,
                       gate_bound: float = DEFAULT_GATE_BOUND, mode: str = "chunk",
                       use_qk_l2norm_in_kernel: bool = True, safe_gate: bool = True,
                       initial_state=None, output_final_state: bool = False,
                       cp_context=None) -> str | None:
    """Why this call cannot run on the library's kernels, or None when it can.

    Checked in order: mode, l2 norm, safe gate, context parallelism, chunk,
    gate bound, dtypes, devices, layout, shapes, contiguity, cu_seqlens,
    initial state."""
    import torch
    if mode != "chunk":
        return f"kda_mode must be 'chunk' (got {mode!r})"
    if not use_qk_l2norm_in_kernel:
        return "q/k must be l2-normalised inside the kernel"
    if not safe_gate:
        return "the gate must be the bounded (safe) log gate"
    if cp_context is not None:
        return "context parallelism is not supported"
    if chunk != CHUNK:
        return f"chunk must be {CHUNK}"
    if not (isinstance(gate_bound, (int, float)) and math.isfinite(gate_bound)
            and -5.5 <= gate_bound < 0):
        return "gate_bound must be finite and in [-5.5, 0)"
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16),
                        ("v", v, torch.bfloat16), ("g", g, torch.float32),
                        ("beta", beta, torch.float32)):
        if not isinstance(t, torch.Tensor):
            return f"{name} must be a tensor"
        if t.dtype != dt:
            return f"{name} must be {dt} (got {t.dtype})"
        if t.device.type != "cuda":
            return f"{name} must be on a GPU"
        if t.device != q.device:
            return f"{name} is on {t.device}, q on {q.device}"
    lay = _layout(q)
    if lay is None:
        return "q must be [B, T, H, 128] or [T, H, 128]"
    B, T = lay
    if q.shape[-1] != HEAD_DIM:
        return f"head dim must be {HEAD_DIM} (got {q.shape[-1]})"
    H = q.shape[-2]
    if k.shape != q.shape:
        return f"k shape {tuple(k.shape)} != q shape {tuple(q.shape)}"
    if g.shape != q.shape:
        return f"g shape {tuple(g.shape)} != q shape {tuple(q.shape)}"
    if v.shape != q.shape:
        return f"v shape {tuple(v.shape)} must equal q shape {tuple(q.shape)} (V = K = 128)"
    if tuple(beta.shape) != tuple(q.shape[:-1]):
        return f"beta shape {tuple(beta.shape)} must be {tuple(q.shape[:-1])}"
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        if not t.is_contiguous():
            return f"{name} must be contiguous"
    if cu_seqlens is not None:
        if B != 1:
            return "packed input (cu_seqlens given) must have batch 1"
        if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32:
            return "cu_seqlens must be an int32 tensor"
        if cu_seqlens.device != q.device:
            return "cu_seqlens must be on the same GPU as q"
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            return "cu_seqlens must be 1-D with at least 2 entries"
        if cu_seqlens.numel() > T + 1 and initial_state is None and not output_final_state:
            return "cu_seqlens has more than T + 1 entries"
        if not cu_seqlens.is_contiguous():
            return "cu_seqlens must be contiguous"
    if B * T > 2**31 - 1:
        return "too many tokens (T must be <= INT32_MAX)"
    if H > 4096:
        return "too many heads"
    if initial_state is not None:
        N = cu_seqlens.numel() - 1 if cu_seqlens is not None else B
        if not isinstance(initial_state, torch.Tensor) or initial_state.dtype != torch.float32:
            return "initial_state must be an fp32 tensor"
        if initial_state.device != q.device:
            return "initial_state must be on the same GPU as q"
        if tuple(initial_state.shape) != (N, H, HEAD_DIM, HEAD_DIM):
            return (f"initial_state shape {tuple(initial_state.shape)} must be "
                    f"{(N, H, HEAD_DIM, HEAD_DIM)} (documents, heads, K, V)")
        if not initial_state.is_contiguous():
            return "initial_state must be contiguous"
    return None


def chunk_fwd(q, k, v, g, beta, cu_seqlens=None, *, chunk: int = CHUNK,
              gate_bound: float = DEFAULT_GATE_BOUND, out=None, initial_state=None,
              output_final_state: bool = False):
    """KDA chunked forward.  Returns ``(o, final_state)``.

    Packed input: ``q, k, v, g`` of shape [1, T, H, 128] (or [T, H, 128]),
    ``beta`` [1, T, H], int32 ``cu_seqlens`` [N+1] on the same GPU.  Dense
    input (``cu_seqlens=None``): [B, T, H, 128] is viewed as B packed
    documents of T tokens (no copy).

    Without states (the fused K3 call) ``final_state`` is None and the list
    ends at its first entry equal to T.  With ``initial_state`` (fp32
    [N, H, 128, 128], document d starts from ``initial_state[d]``) or
    ``output_final_state``, all N + 1 entries of ``cu_seqlens`` delimit
    documents (N = B for dense input) and, when ``output_final_state`` is set,
    ``final_state`` [N, H, 128, 128] fp32 holds each document's last state
    (FLA's ``chunk_kda`` convention).  Raises ValueError for an unsupported
    call and KDAError if the library reports an error."""
    import torch
    reason = unsupported_reason(q, k, v, g, beta, cu_seqlens, chunk=chunk, gate_bound=gate_bound,
                                initial_state=initial_state,
                                output_final_state=output_final_state)
    if reason is not None:
        raise ValueError(reason)
    B, T = _layout(q)
    H = q.shape[-2]
    n_tok = B * T
    if out is None:
        out = torch.empty_like(v)
    elif out.shape != v.shape or out.dtype != torch.bfloat16 or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous bf16 tensor shaped like v on q's device")
    stateful = initial_state is not None or output_final_state
    cu = cu_seqlens
    if cu is None and B > 1:
        cu = torch.arange(0, n_tok + 1, T, dtype=torch.int32, device=q.device)
    if not stateful:
        if n_tok == 0:
            return out, None
        with torch.cuda.device(q.device):
            stream = torch.cuda.current_stream(q.device).cuda_stream
            rc = kda_chunk_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                               beta.data_ptr(), None if cu is None else cu.data_ptr(), n_tok, H,
                               chunk, gate_bound, out.data_ptr(), stream)
        if rc != KDA_OK:
            raise KDAError(rc, kda_last_error())
        return out, None
    n_docs = cu.numel() - 1 if cu is not None else 1
    final = None
    if output_final_state:
        final = torch.empty((n_docs, H, HEAD_DIM, HEAD_DIM), dtype=torch.float32, device=q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = kda_chunk_fwd_state(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(),
            None if cu is None else cu.data_ptr(), n_docs, n_tok, H, chunk, gate_bound,
            None if initial_state is None else initial_state.data_ptr(),
            None if final is None else final.data_ptr(), out.data_ptr(), stream)
    if rc != KDA_OK:
        raise KDAError(rc, kda_last_error())
    return out, final


def recurrent_fwd(q, k, v, g, beta, cu_seqlens=None, *, initial_state=None,
                  output_final_state: bool = False, final_state=None, out=None):
    """Token-recurrent KDA forward (decode, short documents).  Returns
    ``(o, final_state)``.

    Same tensors and document convention as ``chunk_fwd`` with states: all
    N + 1 ``cu_seqlens`` entries delimit documents (N = B for a dense
    [B, T, H, 128] batch).  ``final_state`` may be passed in (fp32
    [N, H, 128, 128], possibly ``initial_state`` itself for an in-place decode
    step); otherwise one is allocated when ``output_final_state`` is set."""
    import torch
    reason = unsupported_reason(q, k, v, g, beta, cu_seqlens, initial_state=initial_state,
                                output_final_state=True)
    if reason is not None:
        raise ValueError(reason)
    B, T = _layout(q)
    H = q.shape[-2]
    n_tok = B * T
    if out is None:
        out = torch.empty_like(v)
    elif out.shape != v.shape or out.dtype != torch.bfloat16 or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous bf16 tensor shaped like v on q's device")
    cu = cu_seqlens
    if cu is None and B > 1:
        cu = torch.arange(0, n_tok + 1, T, dtype=torch.int32, device=q.device)
    n_docs = cu.numel() - 1 if cu is not None else 1
    if final_state is not None:
        if (not isinstance(final_state, torch.Tensor) or final_state.dtype != torch.float32
                or tuple(final_state.shape) != (n_docs, H, HEAD_DIM, HEAD_DIM)
                or not final_state.is_contiguous() or final_state.device != q.device):
            raise ValueError(f"final_state must be a contiguous fp32 tensor of shape "
                             f"{(n_docs, H, HEAD_DIM, HEAD_DIM)} on q's device")
    elif output_final_state:
        final_state = torch.empty((n_docs, H, HEAD_DIM, HEAD_DIM), dtype=torch.float32,
                                  device=q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = kda_recurrent_fwd(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(),
            None if cu is None else cu.data_ptr(), n_docs, n_tok, H,
            None if initial_state is None else initial_state.data_ptr(),
            None if final_state is None else final_state.data_ptr(), out.data_ptr(), stream)
    if rc != KDA_OK:
        raise KDAError(rc, kda_last_error())
    return out, final_state


def chunk_bwd(q, k, v, g, beta, d_out, cu_seqlens=None, *, initial_state=None,
              d_final_state=None, chunk: int = CHUNK, gate_bound: float = DEFAULT_GATE_BOUND):
    """Gradients of ``chunk_fwd(..., initial_state=initial_state,
    output_final_state=True)`` for ``d_out`` (bf16, shaped like v) and
    ``d_final_state`` (fp32 [N, H, 128, 128] or None).  Returns fp32
    ``(dq, dk, dv, dg, dbeta, d_initial_state)`` shaped like the inputs
    (``d_initial_state`` is None when ``initial_state`` is None)."""
    import torch
    reason = unsupported_reason(q, k, v, g, beta, cu_seqlens, chunk=chunk, gate_bound=gate_bound,
                                initial_state=initial_state, output_final_state=True)
    if reason is not None:
        raise ValueError(reason)
    if (not isinstance(d_out, torch.Tensor) or d_out.dtype != torch.bfloat16
            or d_out.shape != v.shape or not d_out.is_contiguous() or d_out.device != q.device):
        raise ValueError("d_out must be a contiguous bf16 tensor shaped like v on q's device")
    B, T = _layout(q)
    H = q.shape[-2]
    n_tok = B * T
    cu = cu_seqlens
    if cu is None and B > 1:
        cu = torch.arange(0, n_tok + 1, T, dtype=torch.int32, device=q.device)
    n_docs = cu.numel() - 1 if cu is not None else 1
    if d_final_state is not None:
        if (not isinstance(d_final_state, torch.Tensor) or d_final_state.dtype != torch.float32
                or tuple(d_final_state.shape) != (n_docs, H, HEAD_DIM, HEAD_DIM)
                or not d_final_state.is_contiguous() or d_final_state.device != q.device):
            raise ValueError(f"d_final_state must be a contiguous fp32 tensor of shape "
                             f"{(n_docs, H, HEAD_DIM, HEAD_DIM)} on q's device")
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty(q.shape, **f32)
    dk = torch.empty(q.shape, **f32)
    dv = torch.empty(v.shape, **f32)
    dg = torch.empty(g.shape, **f32)
    dbeta = torch.empty(beta.shape, **f32)
    dh0 = torch.empty((n_docs, H, HEAD_DIM, HEAD_DIM), **f32) if initial_state is not None else None
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = kda_chunk_bwd(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(),
            None if cu is None else cu.data_ptr(), n_docs, n_tok, H, chunk, gate_bound,
            None if initial_state is None else initial_state.data_ptr(), d_out.data_ptr(),
            None if d_final_state is None else d_final_state.data_ptr(), dq.data_ptr(),
            dk.data_ptr(), dv.data_ptr(), dg.data_ptr(), dbeta.data_ptr(),
            None if dh0 is None else dh0.data_ptr(), stream)
    if rc != KDA_OK:
        raise KDAError(rc, kda_last_error())
    return dq, dk, dv, dg, dbeta, dh0


def _autograd_function():
    import torch

    class _ChunkKDAFunction(torch.autograd.Function):
        """Autograd over the library's forward and backward: saves only q, k, v,
        g, beta, cu_seqlens and the initial state; the backward recomputes every
        intermediate (page "nemo_automodel.components.models.kimi_k3.kda_fused",
        package docstring)."""

        @staticmethod
        def forward(ctx, q, k, v, g, beta, cu_seqlens, initial_state, gate_bound,
                    output_final_state):
            o, final = chunk_fwd(q, k, v, g, beta, cu_seqlens, gate_bound=gate_bound,
                                 initial_state=initial_state,
                                 output_final_state=output_final_state)
            ctx.save_for_backward(q, k, v, g, beta, cu_seqlens, initial_state)
            ctx.gate_bound = gate_bound
            if final is None:
                return o
            return o, final

        @staticmethod
        def backward(ctx, d_o, *rest):
            q, k, v, g, beta, cu, h0 = ctx.saved_tensors
            d_final = rest[0] if rest else None
            if d_final is not None:
                d_final = d_final.float().contiguous()
            dq, dk, dv, dg, dbeta, dh0 = chunk_bwd(
                q, k, v, g, beta, d_o.to(torch.bfloat16).contiguous(), cu, initial_state=h0,
                d_final_state=d_final, gate_bound=ctx.gate_bound)
            return (dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), dg.to(g.dtype),
                    dbeta.to(beta.dtype), None, dh0, None, None)

    return _ChunkKDAFunction


def chunk_kda(q, k, v, g, beta, cu_seqlens=None, *, initial_state=None,
              output_final_state: bool = False, gate_bound: float = DEFAULT_GATE_BOUND):
    """Differentiable KDA chunked forward: ``(o, final_state or None)``, with
    the gradients of q, k, v, g, beta (and of ``initial_state``) from
    ``kda_chunk_bwd``.  Same tensors and document convention as ``chunk_fwd``."""
    fn = _autograd_function()
    r = fn.apply(q, k, v, g, beta, cu_seqlens, initial_state, gate_bound, output_final_state)
    if output_final_state:
        return r
    return r, None


def device_status(device=None) -> int:
    """Synchronise the current stream and return / clear the sticky device flags."""
    import torch
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        rc = kda_device_status(torch.cuda.current_stream().cuda_stream)
    if rc < 0:
        raise KDAError(rc, "kda_device_status failed")
    return rc
