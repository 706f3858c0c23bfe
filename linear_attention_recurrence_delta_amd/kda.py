"""Python binding of the KDA C ABI (``include/kda.h``): argument marshalling only.

torch supplies device memory and the current HIP stream; every step of the
computation runs in the HIP kernels of libkda.so.  Nothing here computes on
tensor values, and nothing falls back to another implementation: a missing
library or a non-OK status raises.
"""
from __future__ import annotations

import torch

from ._lib import PrefillDesc, PrefillTensors, lib

KDA_DTYPE_F32 = 0
KDA_DTYPE_BF16 = 1
_DTYPES = {torch.float32: KDA_DTYPE_F32, torch.bfloat16: KDA_DTYPE_BF16}

# Kernel plans (kda_prefill_desc.kernel in include/kda.h)
KDA_KERNEL_AUTO = 0
KDA_KERNEL_PIPELINED = 1
KDA_KERNEL_CHUNK_STAGED = 2


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


def _prefill_args(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, out, output_final_state, final_state,
                  g_dtype=torch.float32, need_out=True):
    """Shared argument handling of the prefill entry points (shapes, dtypes,
    output allocation).  Returns a dict of the marshalled arguments."""
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
    _need(g, "g" if g_dtype == torch.float32 else "z", g_dtype, 3)
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
    for name, t in (("k", k), ("v", v), ("g" if g_dtype == torch.float32 else "z", g), ("beta", beta),
                    ("initial_state", initial_state), ("cu_seqlens", cu_seqlens)):
        if t is not None and t.device != dev:
            raise ValueError("%s must be on q's device (%s), got %s" % (name, dev, t.device))
    o = None
    if need_out:
        o = out if out is not None else torch.empty((T, H, dv), dtype=qdt, device=dev)
        _need(o, "out", qdt)
        if tuple(o.shape) != (T, H, dv) and not (dense_batch and o.numel() == T * H * dv and o.dim() == 4
                                                 and tuple(o.shape) == (num_seqs, T // max(num_seqs, 1), H, dv)):
            raise ValueError("out must be [T, H, d_v] = %s, got %s" % ((T, H, dv), tuple(o.shape)))
        if o.device != dev:
            raise ValueError("out must be on q's device")
        o = o.view(T, H, dv)
    fs = None
    if output_final_state:
        fs = final_state if final_state is not None else torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
        _need(fs, "final_state", torch.float32, 4)
        if tuple(fs.shape) != (N, H, dk, dv):
            raise ValueError("final_state must be [N, H, d_k, d_v] = %s, got %s" % ((N, H, dk, dv), tuple(fs.shape)))
        if fs.device != dev:
            raise ValueError("final_state must be on q's device")
    return dict(dense_batch=dense_batch, q=q, k=k, v=v, g=g, beta=beta, T=T, H=H, dk=dk, dv=dv, N=N, dev=dev,
                o=o, fs=fs, dt=_DTYPES[qdt])


def _desc(a, chunk_size, scale, fused=False, interval=0, capacity=0, plan=None):
    plan = plan or {}
    unknown = set(plan) - {"kernel", "slab_columns", "segments"}
    if unknown:
        raise ValueError("unknown plan keys %s" % sorted(unknown))
    return PrefillDesc(num_seqs=a["N"], total_tokens=a["T"], num_heads=a["H"], d_k=a["dk"], d_v=a["dv"],
                       qkv_dtype=a["dt"], chunk_size=int(chunk_size), scale=float(scale), fused=int(fused),
                       checkpoint_interval=int(interval), checkpoint_capacity=int(capacity),
                       kernel=int(plan.get("kernel", 0)), slab_columns=int(plan.get("slab_columns", 0)),
                       segments=int(plan.get("segments", 0)))


def _workspace(a, desc, packed):
    """Workspace of the call (the segment scan's maps; packed batches need none)."""
    if packed:
        ws_bytes = 0
    else:
        with torch.cuda.device(a["dev"]):  # the plan depends on the device's compute units
            ws_bytes = int(lib().kda_prefill_ex_workspace_bytes(desc))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=a["dev"]) if ws_bytes else None
    return ws, ws_bytes


def _run_ex(a, desc, initial_state, cu_seqlens, z=None, a_log=None, checkpoints=None, noalloc=False):
    """kda_prefill_ex (or, noalloc, kda_prefill_ex_noalloc: no workspace
    allocated, the library's static buffer instead) with the marshalled
    arguments."""
    t = PrefillTensors(q=_ptr(a["q"]), k=_ptr(a["k"]), v=_ptr(a["v"]), g=None if z is not None else _ptr(a["g"]),
                       z=_ptr(z), a_log=_ptr(a_log), beta=_ptr(a["beta"]), initial_state=_ptr(initial_state),
                       cu_seqlens=_ptr(cu_seqlens), o=_ptr(a["o"]), final_state=_ptr(a["fs"]),
                       checkpoints=_ptr(checkpoints))
    if noalloc:
        with torch.cuda.device(a["dev"]):
            _check(lib().kda_prefill_ex_noalloc(desc, t, _stream(a["dev"])))
        return
    ws, ws_bytes = _workspace(a, desc, cu_seqlens is not None)
    with torch.cuda.device(a["dev"]):
        _check(lib().kda_prefill_ex(desc, t, _ptr(ws), ws_bytes, _stream(a["dev"])))


def kda_noalloc_scratch_bytes() -> int:
    return int(lib().kda_noalloc_scratch_bytes())


def kda_prefill_ex_workspace_bytes(num_seqs, total_tokens, num_heads, d_k, d_v, dtype, chunk_size=0, *,
                                   fused=False, checkpoint_interval=0, checkpoint_capacity=0, plan=None) -> int:
    a = dict(N=num_seqs, T=total_tokens, H=num_heads, dk=d_k, dv=d_v, dt=_DTYPES.get(dtype, -1))
    return int(lib().kda_prefill_ex_workspace_bytes(_desc(a, chunk_size, 1.0, fused, checkpoint_interval,
                                                          checkpoint_capacity, plan)))


def kda_prefill(q, k, v, g, beta, initial_state=None, cu_seqlens=None, *, chunk_size: int = 0,
                scale: float = 1.0, output_final_state: bool = True, num_seqs: int | None = None,
                out=None, final_state=None, plan=None, noalloc: bool = False):
    """Chunked KDA prefill over a packed batch.

    q, k, g: [T, H, d_k]; v: [T, H, d_v]; beta: [T, H].  A dense batch may be
    passed as [B, T, H, d] (and beta [B, T, H]); it is the packed layout with
    B equal-length sequences.  cu_seqlens: int32 device tensor [N + 1] or None.
    initial_state: fp32 [N, H, d_k, d_v] or None (zeros).
    plan: None (the library's choice, through kda_prefill) or a dict with
    any of kernel (KDA_KERNEL_*), slab_columns, segments (through
    kda_prefill_ex; include/kda.h describes the fields).
    noalloc: through kda_prefill_ex_noalloc (no workspace is allocated; the
    library's static device buffer serves instead; outputs are allocated here
    unless out / final_state are given).
    Returns (o, final_state); final_state is None if output_final_state is False.
    """
    a = _prefill_args(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, out, output_final_state, final_state)
    desc = _desc(a, chunk_size, scale, plan=plan)
    if plan is not None or noalloc:
        _run_ex(a, desc, initial_state, cu_seqlens, noalloc=noalloc)
    else:
        ws, ws_bytes = _workspace(a, desc, cu_seqlens is not None)
        with torch.cuda.device(a["dev"]):
            _check(lib().kda_prefill(a["N"], a["T"], a["H"], a["dk"], a["dv"], a["dt"], chunk_size, float(scale),
                                     _ptr(a["q"]), _ptr(a["k"]), _ptr(a["v"]), _ptr(a["g"]), _ptr(a["beta"]),
                                     _ptr(initial_state), _ptr(cu_seqlens), _ptr(a["o"]), _ptr(a["fs"]),
                                     _ptr(ws), ws_bytes, _stream(a["dev"])))
    o = a["o"]
    if a["dense_batch"]:
        o = o.view(a["N"], a["T"] // max(a["N"], 1), a["H"], a["dv"])
    return o, a["fs"]


def kda_prefill_checkpointed(q, k, v, g, beta, initial_state=None, cu_seqlens=None, *, checkpoint_interval: int,
                             chunk_size: int = 0, scale: float = 1.0, output_final_state: bool = True,
                             num_seqs: int | None = None, out=None, final_state=None, checkpoints=None,
                             plan=None):
    """kda_prefill that also returns the state after every checkpoint_interval
    tokens of each sequence (a multiple of the chunk size in use).

    Returns (o, final_state, checkpoints, first_slot): checkpoints is fp32
    [T // checkpoint_interval, H, d_k, d_v]; first_slot is an int64 device
    tensor [N + 1] whose entry n is the slot of sequence n's first checkpoint
    (sequence n owns slots first_slot[n] .. first_slot[n + 1] - 1, checkpoint j
    being the state after its first (j + 1) * checkpoint_interval tokens).
    Slots from first_slot[N] on are not written.
    """
    a = _prefill_args(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, out, output_final_state, final_state)
    interval = int(checkpoint_interval)
    if interval < 1:
        raise ValueError("checkpoint_interval must be positive")
    cap = a["T"] // interval
    ck = checkpoints if checkpoints is not None else torch.empty((cap, a["H"], a["dk"], a["dv"]),
                                                                  dtype=torch.float32, device=a["dev"])
    _need(ck, "checkpoints", torch.float32, 4)
    if ck.shape[1:] != (a["H"], a["dk"], a["dv"]) or ck.shape[0] < cap:
        raise ValueError("checkpoints must be [>= T // checkpoint_interval, H, d_k, d_v]")
    # slot bookkeeping for the caller (the kernels derive the same offsets from cu_seqlens)
    if cu_seqlens is not None:
        counts = (cu_seqlens[1:] - cu_seqlens[:-1]).to(torch.int64) // interval
    else:
        counts = torch.full((a["N"],), (a["T"] // max(a["N"], 1)) // interval, dtype=torch.int64, device=a["dev"])
    first_slot = torch.zeros(a["N"] + 1, dtype=torch.int64, device=a["dev"])
    if a["N"] > 0:
        first_slot[1:] = torch.cumsum(counts, 0)
    if ck.device != a["dev"]:
        raise ValueError("checkpoints must be on q's device")
    desc = _desc(a, chunk_size, scale, interval=interval, capacity=int(ck.shape[0]), plan=plan)
    if plan is not None:
        _run_ex(a, desc, initial_state, cu_seqlens, checkpoints=ck if ck.numel() else None)
    else:
        ws, ws_bytes = _workspace(a, desc, cu_seqlens is not None)
        with torch.cuda.device(a["dev"]):
            _check(lib().kda_prefill_checkpointed(
                a["N"], a["T"], a["H"], a["dk"], a["dv"], a["dt"], chunk_size, float(scale),
                _ptr(a["q"]), _ptr(a["k"]), _ptr(a["v"]), _ptr(a["g"]), _ptr(a["beta"]),
                _ptr(initial_state), _ptr(cu_seqlens), _ptr(a["o"]), _ptr(a["fs"]),
                interval, _ptr(ck) if ck.numel() else None, int(ck.shape[0]),
                _ptr(ws), ws_bytes, _stream(a["dev"])))
    o = a["o"]
    if a["dense_batch"]:
        o = o.view(a["N"], a["T"] // max(a["N"], 1), a["H"], a["dv"])
    return o, a["fs"], ck, first_slot


def kda_prefill_fused_supported(dtype: torch.dtype, d_k: int, d_v: int, chunk_size: int = 0) -> bool:
    return bool(lib().kda_prefill_fused_supported(_DTYPES.get(dtype, -1), d_k, d_v, chunk_size))


def kda_prefill_fused(q, k, v, z, a_log, beta, initial_state=None, cu_seqlens=None, *, chunk_size: int = 0,
                      scale: float = 1.0, output_final_state: bool = True, num_seqs: int | None = None,
                      out=None, final_state=None, plan=None):
    """kda_prefill with the gate and the q/k L2 norm computed in the kernel.

    q, k: unnormalised [T, H, d_k] (bf16); z: decay logits [T, H, d_k] (same
    dtype); a_log: fp32 [H] per-head log-scale.  g = -5 Sigmoid(exp(a_log) z)
    is formed in the kernel (no g argument).  Returns (o, final_state)."""
    # the shared marshalling checks shapes and dtypes; z takes g's place
    a = _prefill_args(q, k, v, z, beta, initial_state, cu_seqlens, num_seqs, out, output_final_state,
                      final_state, g_dtype=q.dtype)
    _need(a_log, "a_log", torch.float32, 1)
    if a_log.shape[0] != a["H"]:
        raise ValueError("a_log must have one entry per head")
    if a_log.device != a["dev"]:
        raise ValueError("a_log must be on q's device")
    desc = _desc(a, chunk_size, scale, fused=True, plan=plan)
    if plan is not None:
        _run_ex(a, desc, initial_state, cu_seqlens, z=a["g"], a_log=a_log)
    else:
        ws, ws_bytes = _workspace(a, desc, cu_seqlens is not None)
        with torch.cuda.device(a["dev"]):
            _check(lib().kda_prefill_fused(a["N"], a["T"], a["H"], a["dk"], a["dv"], a["dt"], chunk_size,
                                           float(scale), _ptr(a["q"]), _ptr(a["k"]), _ptr(a["v"]), _ptr(a["g"]),
                                           _ptr(a_log), _ptr(a["beta"]), _ptr(initial_state), _ptr(cu_seqlens),
                                           _ptr(a["o"]), _ptr(a["fs"]), _ptr(ws), ws_bytes, _stream(a["dev"])))
    o = a["o"]
    if a["dense_batch"]:
        o = o.view(a["N"], a["T"] // max(a["N"], 1), a["H"], a["dv"])
    return o, a["fs"]


def kda_output_gate_supported(dtype: torch.dtype, d_v: int) -> bool:
    return bool(lib().kda_output_gate_supported(_DTYPES.get(dtype, -1), d_v))


def kda_output_gate(o, gate, weight, *, eps: float = 1e-6, out=None):
    """y = sigmoid(gate) * RMSNorm(o) * weight over the last axis (d_v).

    o, gate: [..., H, d_v] in bfloat16 or float32 (same dtype); weight: fp32
    [d_v].  out may be o or gate (in place).  Returns y."""
    if o.dtype not in _DTYPES or gate.dtype != o.dtype:
        raise TypeError("o and gate must both be bfloat16 or both float32")
    if o.dim() < 2 or gate.shape != o.shape:
        raise ValueError("o and gate must have the same shape [..., H, d_v]")
    _need(o, "o", o.dtype)
    _need(gate, "gate", o.dtype)
    _need(weight, "weight", torch.float32, 1)
    H, dv = o.shape[-2], o.shape[-1]
    if weight.shape[0] != dv:
        raise ValueError("weight must have d_v entries")
    T = o.numel() // max(1, H * dv)
    y = out if out is not None else torch.empty_like(o)
    _need(y, "out", o.dtype)
    if y.shape != o.shape:
        raise ValueError("out must have the shape of o")
    with torch.cuda.device(o.device):
        _check(lib().kda_output_gate(T, H, dv, _DTYPES[o.dtype], float(eps), _ptr(o), _ptr(gate), _ptr(weight),
                                     _ptr(y), _stream(o.device)))
    return y


def kda_prefill_output_gated(q, k, v, g, beta, gate, weight, initial_state=None, cu_seqlens=None, *,
                             eps: float = 1e-6, chunk_size: int = 0, scale: float = 1.0,
                             output_final_state: bool = True, num_seqs: int | None = None, out=None,
                             final_state=None):
    """kda_prefill followed by y = sigmoid(gate) * RMSNorm(o) * weight, with y
    returned in place of o (fused into the o store where a workgroup holds a
    whole head).  gate: [T, H, d_v] in q's dtype; weight: fp32 [d_v].
    Returns (y, final_state)."""
    a = _prefill_args(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, out, output_final_state, final_state)
    if a["dense_batch"]:
        gate = gate.view(-1, *gate.shape[2:]) if gate.is_contiguous() else gate
    _need(gate, "gate", a["q"].dtype, 3)
    _need(weight, "weight", torch.float32, 1)
    if tuple(gate.shape) != (a["T"], a["H"], a["dv"]) or gate.device != a["dev"]:
        raise ValueError("gate must be [T, H, d_v] on q's device")
    if weight.shape[0] != a["dv"] or weight.device != a["dev"]:
        raise ValueError("weight must have d_v entries on q's device")
    desc = _desc(a, chunk_size, scale)
    ws, ws_bytes = _workspace(a, desc, cu_seqlens is not None)
    with torch.cuda.device(a["dev"]):
        _check(lib().kda_prefill_output_gated(
            a["N"], a["T"], a["H"], a["dk"], a["dv"], a["dt"], chunk_size, float(scale),
            _ptr(a["q"]), _ptr(a["k"]), _ptr(a["v"]), _ptr(a["g"]), _ptr(a["beta"]), _ptr(initial_state),
            _ptr(cu_seqlens), _ptr(gate), _ptr(weight), float(eps), _ptr(a["o"]), _ptr(a["fs"]),
            _ptr(ws), ws_bytes, _stream(a["dev"])))
    y = a["o"]
    if a["dense_batch"]:
        y = y.view(a["N"], a["T"] // max(a["N"], 1), a["H"], a["dv"])
    return y, a["fs"]


def kda_prefill_backward_supported(dtype: torch.dtype, d_k: int, d_v: int) -> bool:
    return bool(lib().kda_prefill_backward_supported(_DTYPES[dtype], d_k, d_v)) if dtype in _DTYPES else False


def kda_prefill_backward(q, k, v, g, beta, d_o, initial_state=None, d_final_state=None, cu_seqlens=None, *,
                         scale: float = 1.0, num_seqs: int | None = None, need_d_initial_state: bool = True):
    """Gradients of kda_prefill: for a loss with gradient d_o [T, H, d_v] with
    respect to o and d_final_state [N, H, d_k, d_v] (or None) with respect to
    the final states, returns (dq, dk, dv, dg, dbeta, d_initial_state) shaped
    like q, k, v, g, beta and [N, H, d_k, d_v] (None if not requested).  q, k,
    v and d_o are bf16 with d_k = d_v = 128; the other arguments are as in
    kda_prefill (packed [T, H, d] layout)."""
    if q.dim() != 3:
        raise ValueError("kda_prefill_backward takes the packed [T, H, d] layout")
    a = _prefill_args(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, None, False, None, need_out=False)
    _need(d_o, "d_o", a["q"].dtype, 3)
    if d_o.shape != (a["T"], a["H"], a["dv"]) or d_o.device != a["dev"]:
        raise ValueError("d_o must be [T, H, d_v] on q's device")
    if d_final_state is not None:
        _need(d_final_state, "d_final_state", torch.float32, 4)
        if tuple(d_final_state.shape) != (a["N"], a["H"], a["dk"], a["dv"]) or d_final_state.device != a["dev"]:
            raise ValueError("d_final_state must be [N, H, d_k, d_v] on q's device")
    dev = a["dev"]
    dq = torch.empty_like(a["q"])
    dk = torch.empty_like(a["k"])
    dv = torch.empty_like(a["v"])
    dg = torch.empty_like(a["g"])
    dbeta = torch.empty_like(a["beta"])
    dS0 = torch.empty((a["N"], a["H"], a["dk"], a["dv"]), dtype=torch.float32, device=dev) \
        if need_d_initial_state else None
    ws_bytes = int(lib().kda_prefill_backward_workspace_bytes(a["N"], a["T"], a["H"], a["dk"], a["dv"], a["dt"]))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    with torch.cuda.device(dev):
        _check(lib().kda_prefill_backward(
            a["N"], a["T"], a["H"], a["dk"], a["dv"], a["dt"], float(scale),
            _ptr(a["q"]), _ptr(a["k"]), _ptr(a["v"]), _ptr(a["g"]), _ptr(a["beta"]), _ptr(initial_state),
            _ptr(cu_seqlens), _ptr(d_o), _ptr(d_final_state), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
            _ptr(dbeta), _ptr(dS0), _ptr(ws), ws_bytes, _stream(dev)))
    return dq, dk, dv, dg, dbeta, dS0


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
    for name, t in (("k", k), ("v", v), ("g", g), ("beta", beta), ("state", state)):
        if t.device != dev:
            raise ValueError("%s must be on q's device (%s), got %s" % (name, dev, t.device))
    o = out if out is not None else torch.empty((N, H, dv), dtype=qdt, device=dev)
    _need(o, "out", qdt, 3)
    if tuple(o.shape) != (N, H, dv) or o.device != dev:
        raise ValueError("out must be [N, H, d_v] = %s on q's device, got %s" % ((N, H, dv), tuple(o.shape)))
    with torch.cuda.device(dev):
        _check(lib().kda_decode_step(N, H, dk, dv, _DTYPES[qdt], float(scale),
                                     _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(state), _ptr(o), _stream(dev)))
    return o
