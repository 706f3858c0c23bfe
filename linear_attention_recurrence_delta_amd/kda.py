"""Python binding of the KDA C ABI (``include/kda.h``): argument marshalling only.

torch supplies device memory and the current HIP stream; every step of the
computation runs in the HIP kernels of libkda.so.  Nothing here computes on
tensor values, and nothing falls back to another implementation: a missing
library or a non-OK status raises.
"""
from __future__ import annotations

import torch

from ._lib import lib

KDA_DTYPE_F32 = 0
KDA_DTYPE_BF16 = 1
_DTYPES = {torch.float32: KDA_DTYPE_F32, torch.bfloat16: KDA_DTYPE_BF16}


class KdaError(RuntimeError):
    """A kda_* call returned a status other than KDA_OK."""

    def __init__(self, status: int):
        self.status = int(status)
        super().__init__(lib().kda_status_string(self.status).decode())


def _check(status: int) -> None:
    if status != 0:
        raise KdaError(status)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device (cuda/hip) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, got %d" % (name, ndim, t.dim()))


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def kda_abi_version() -> int:
    return int(lib().kda_abi_version())


def kda_prefill_supported(dtype: torch.dtype, d_k: int, d_v: int, chunk_size: int = 0) -> bool:
    return bool(lib().kda_prefill_supported(_DTYPES.get(dtype, -1), d_k, d_v, chunk_size))


def kda_decode_supported(dtype: torch.dtype, d_k: int, d_v: int) -> bool:
    return bool(lib().kda_decode_supported(_DTYPES.get(dtype, -1), d_k, d_v))


def kda_prefill_workspace_bytes(num_seqs, total_tokens, num_heads, d_k, d_v, dtype, chunk_size=0) -> int:
    return int(lib().kda_prefill_workspace_bytes(num_seqs, total_tokens, num_heads, d_k, d_v,
                                                 _DTYPES.get(dtype, -1), chunk_size))


def kda_prefill(q, k, v, g, beta, initial_state=None, cu_seqlens=None, *, chunk_size: int = 0,
                scale: float = 1.0, output_final_state: bool = True, num_seqs: int | None = None,
                out=None, final_state=None):
    """Chunked KDA prefill over a packed batch.

    q, k, g: [T, H, d_k]; v: [T, H, d_v]; beta: [T, H].  A dense batch may be
    passed as [B, T, H, d] (and beta [B, T, H]); it is the packed layout with
    B equal-length sequences.  cu_seqlens: int32 device tensor [N + 1] or None.
    initial_state: fp32 [N, H, d_k, d_v] or None (zeros).
    Returns (o, final_state); final_state is None if output_final_state is False.
    """
    dense_batch = q.dim() == 4
    if dense_batch:
        B = q.shape[0]
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens needs the packed [T, H, d] layout")
        q, k, v, g = (x.view(-1, *x.shape[2:]) if x.is_contiguous() else x for x in (q, k, v, g))
        beta = beta.view(-1, beta.shape[-1]) if beta.is_contiguous() else beta
        num_seqs = B
    qdt = q.dtype
    if qdt not in _DTYPES:
        raise TypeError("q must be bfloat16 or float32")
    _need(q, "q", qdt, 3)
    T, H, dk = q.shape
    _need(k, "k", qdt, 3)
    _need(v, "v", qdt, 3)
    _need(g, "g", torch.float32, 3)
    _need(beta, "beta", torch.float32, 2)
    dv = v.shape[-1]
    if k.shape != (T, H, dk) or g.shape != (T, H, dk) or v.shape[:2] != (T, H) or beta.shape != (T, H):
        raise ValueError("inconsistent q/k/v/g/beta shapes")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
        N = cu_seqlens.shape[0] - 1
    else:
        N = 1 if num_seqs is None else int(num_seqs)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, 4)
        if tuple(initial_state.shape) != (N, H, dk, dv):
            raise ValueError("initial_state must be [N, H, d_k, d_v]")
    dev = q.device
    o = out if out is not None else torch.empty((T, H, dv), dtype=qdt, device=dev)
    _need(o, "out", qdt, 3)
    fs = None
    if output_final_state:
        fs = final_state if final_state is not None else torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
        _need(fs, "final_state", torch.float32, 4)
    dt = _DTYPES[qdt]
    ws_bytes = int(lib().kda_prefill_workspace_bytes(N, T, H, dk, dv, dt, chunk_size))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    with torch.cuda.device(dev):
        _check(lib().kda_prefill(N, T, H, dk, dv, dt, chunk_size, float(scale),
                                 _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 _ptr(initial_state), _ptr(cu_seqlens), _ptr(o), _ptr(fs),
                                 _ptr(ws), ws_bytes, _stream(dev)))
    if dense_batch:
        o = o.view(N, T // max(N, 1), H, dv)
    return o, fs


def kda_decode_step(q, k, v, g, beta, state, *, scale: float = 1.0, out=None):
    """One token per sequence.  q, k, g: [N, H, d_k]; v: [N, H, d_v];
    beta: [N, H]; state: fp32 [N, H, d_k, d_v], updated in place.  Returns o."""
    qdt = q.dtype
    if qdt not in _DTYPES:
        raise TypeError("q must be bfloat16 or float32")
    _need(q, "q", qdt, 3)
    N, H, dk = q.shape
    _need(k, "k", qdt, 3)
    _need(v, "v", qdt, 3)
    _need(g, "g", torch.float32, 3)
    _need(beta, "beta", torch.float32, 2)
    _need(state, "state", torch.float32, 4)
    dv = v.shape[-1]
    if k.shape != (N, H, dk) or g.shape != (N, H, dk) or beta.shape != (N, H) or \
            tuple(state.shape) != (N, H, dk, dv):
        raise ValueError("inconsistent decode shapes")
    dev = q.device
    o = out if out is not None else torch.empty((N, H, dv), dtype=qdt, device=dev)
    _need(o, "out", qdt, 3)
    with torch.cuda.device(dev):
        _check(lib().kda_decode_step(N, H, dk, dv, _DTYPES[qdt], float(scale),
                                     _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(state), _ptr(o), _stream(dev)))
    return o
