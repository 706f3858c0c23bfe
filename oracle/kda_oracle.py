"""ctypes wrapper of the C fp64 oracle (test infrastructure only).

Inputs are converted to contiguous float64 numpy arrays (bf16 and fp32 values
convert exactly), the C routine runs the token-by-token recurrence, and the
results come back as float64 arrays.  See ``kda_oracle.c`` for the definition
and its sources.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lock = threading.Lock()
_lib = None


def lib_path() -> str:
    return _LIB


def compile_source(src: str, out: str) -> str:
    """gcc -O2, OpenMP, no fast-math: C source file -> shared library."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-I", _HERE, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle library next to its source."""
    if force or not os.path.exists(_LIB):
        compile_source(_SRC, _LIB)
    return _LIB


def _bind(path: str):
    lib = ctypes.CDLL(path)
    i64, dbl, ip = ctypes.c_int64, ctypes.c_double, ctypes.c_int
    vp = ctypes.c_void_p
    lib.kda_oracle_prefill_f64.argtypes = [
        i64, vp, i64, i64, i64, dbl, ip,
        vp, vp, vp, vp, vp, vp, vp, vp, ip]
    lib.kda_oracle_prefill_f64.restype = ip
    lib.kda_oracle_decode_step_f64.argtypes = [
        i64, i64, i64, i64, dbl, vp, vp, vp, vp, vp, vp, vp, ip]
    lib.kda_oracle_decode_step_f64.restype = ip
    lib.kda_oracle_prefill_backward_f64.argtypes = [
        i64, vp, i64, i64, i64, dbl,
        vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, ip]
    lib.kda_oracle_prefill_backward_f64.restype = ip
    lib.kda_oracle_max_threads.restype = ip
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=False)
            _lib = _bind(_LIB)
    return _lib


class OracleLib:
    """The same API bound to another build of an oracle source (used by the
    test that plants mistakes in copies of the oracle)."""

    def __init__(self, path: str):
        self._l = _bind(path)

    def prefill(self, *a, **kw):
        return prefill(*a, _lib=self._l, **kw)

    def decode_step(self, *a, **kw):
        return decode_step(*a, _lib=self._l, **kw)

    def prefill_backward(self, *a, **kw):
        return prefill_backward(*a, _lib=self._l, **kw)


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor: exact widening on the host
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def prefill(q, k, v, g, beta, initial_state=None, cu_seqlens=None,
            scale: float = 1.0, delta: bool = True, nthreads: int = 0,
            _lib=None):
    """Token-by-token fp64 KDA over a packed batch.

    Shapes: q, k, g [T, H, dk]; v [T, H, dv]; beta [T, H];
    initial_state [N, H, dk, dv] or None; cu_seqlens [N + 1] or None (one
    sequence of length T).  Returns (o [T, H, dv], final_state [N, H, dk, dv]).
    """
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
            dtype=np.int64))
    N = cu.shape[0] - 1
    assert k.shape == (T, H, dk) and g.shape == (T, H, dk)
    assert v.shape == (T, H, dv) and beta.shape == (T, H)
    assert int(cu[-1]) == T
    S0 = None if initial_state is None else _f64(initial_state)
    if S0 is not None:
        assert S0.shape == (N, H, dk, dv)
    o = np.zeros((T, H, dv), dtype=np.float64)
    S = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = (_lib or _load()).kda_oracle_prefill_f64(
        N, _ptr(cu), H, dk, dv, float(scale), 1 if delta else 0,
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0),
        _ptr(o), _ptr(S), int(nthreads))
    if rc != 0:
        raise ValueError("kda_oracle_prefill_f64 failed with %d" % rc)
    return o, S


def prefill_checkpoints(q, k, v, g, beta, initial_state=None, cu_seqlens=None, *,
                        interval: int, scale: float = 1.0, nthreads: int = 0):
    """States at token boundaries, by definition: checkpoint j of sequence n
    is the final state of the token-by-token recurrence (prefill above) over
    that sequence's first (j + 1) * interval tokens, from its initial state.
    The KDA state restored at a token boundary for prefix reuse ("Inside
    Kimi K3", section "Sequence mixing").

    Returns (checkpoints [sum_n floor(L_n / interval), H, dk, dv],
    first_slot [N + 1]) with sequence n's checkpoints in slots
    first_slot[n] .. first_slot[n + 1] - 1.  Slow on purpose: one prefill per
    checkpoint."""
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.asarray(cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    S0 = None if initial_state is None else _f64(initial_state)
    counts = [int(cu[n + 1] - cu[n]) // int(interval) for n in range(N)]
    first_slot = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    ck = np.zeros((int(first_slot[-1]), H, dk, dv), dtype=np.float64)
    for n in range(N):
        a = int(cu[n])
        for j in range(counts[n]):
            b = a + (j + 1) * int(interval)
            init = None if S0 is None else S0[n:n + 1]
            _, S = prefill(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], initial_state=init,
                           scale=scale, nthreads=nthreads)
            ck[first_slot[n] + j] = S[0]
    return ck, first_slot


def l2norm(x):
    """L2Norm over the last axis (the head dimension) in fp64: each (token,
    head) vector divided by its Euclidean norm; the zero vector stays zero
    (the pages do not define L2Norm(0); this reading keeps a zero query or
    key inert).  q_t and k_t are L2-normalised in the symbol table of
    "Understanding Kimi K3's attention"."""
    x = _f64(x)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.divide(x, n, out=np.zeros_like(x), where=n > 0)


def gate(z, a_log, g_min: float = -5.0):
    """Log-decay from the decay logits, in fp64: g = g_min Sigmoid(e^{A_h} z)
    ("Understanding Kimi K3's attention", gate equation; g_min = -5, A_h a
    per-head log-scale).  z [T, H, dk], a_log [H]."""
    z = _f64(z)
    a = np.exp(_f64(a_log))[None, :, None]
    return g_min / (1.0 + np.exp(-a * z))


def prefill_fused(q, k, v, z, a_log, beta, initial_state=None, cu_seqlens=None,
                  scale: float = 1.0, nthreads: int = 0):
    """The recurrence with its inputs prepared as the pages define them:
    L2-normalised q and k and the gated log-decay from z (l2norm, gate
    above), then prefill.  Returns (o, final_state)."""
    return prefill(l2norm(q), l2norm(k), v, gate(z, a_log), beta, initial_state=initial_state,
                   cu_seqlens=cu_seqlens, scale=scale, nthreads=nthreads)


def output_gate(o, gate, weight, eps: float):
    """Gated output before the output projection, in fp64: Sigmoid(gate) times
    RMSNorm(o) over the last axis, RMSNorm(x) = x / sqrt(mean(x^2) + eps) *
    weight ("Understanding Kimi K3's attention", output equation; the pages
    give no eps, so it is an argument).  o, gate [..., d_v], weight [d_v]."""
    o = _f64(o)
    gate = _f64(gate)
    w = _f64(weight)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return o / np.sqrt(ms + float(eps)) * w * (1.0 / (1.0 + np.exp(-gate)))


def decode_step(q, k, v, g, beta, state, scale: float = 1.0,
                nthreads: int = 0, _lib=None):
    """One token per (n, h).  Returns (o [N, H, dv], new_state) without
    touching the caller's arrays."""
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    S = _f64(state).copy()
    N, H, dk, dv = S.shape
    assert q.shape == (N, H, dk) and k.shape == (N, H, dk)
    assert v.shape == (N, H, dv) and g.shape == (N, H, dk)
    assert beta.shape == (N, H)
    o = np.zeros((N, H, dv), dtype=np.float64)
    rc = (_lib or _load()).kda_oracle_decode_step_f64(
        N, H, dk, dv, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
        _ptr(beta), _ptr(S), _ptr(o), int(nthreads))
    if rc != 0:
        raise ValueError("kda_oracle_decode_step_f64 failed with %d" % rc)
    return o, S


def prefill_backward(q, k, v, g, beta, d_o, initial_state=None, d_final_state=None,
                     cu_seqlens=None, scale: float = 1.0, seg_len: int = 0,
                     nthreads: int = 0, _lib=None):
    """Gradients of prefill (delta = True) for a loss whose gradients with
    respect to o and to the final states are d_o [T, H, dv] and d_final_state
    [N, H, dk, dv] (None = zeros): the token recurrence differentiated in
    reverse, in fp64 (kda_oracle.c).  Returns (dq, dk, dv, dg, dbeta, dS0)
    with the shapes of q, k, v, g, beta and [N, H, dk, dv]."""
    q, k, v, g, beta, d_o = (_f64(a) for a in (q, k, v, g, beta, d_o))
    T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
            dtype=np.int64))
    N = cu.shape[0] - 1
    assert k.shape == (T, H, dk) and g.shape == (T, H, dk)
    assert v.shape == (T, H, dv) and beta.shape == (T, H) and d_o.shape == (T, H, dv)
    assert int(cu[-1]) == T
    S0 = None if initial_state is None else _f64(initial_state)
    dST = None if d_final_state is None else _f64(d_final_state)
    for x in (S0, dST):
        if x is not None:
            assert x.shape == (N, H, dk, dv)
    dq = np.zeros((T, H, dk))
    dkey = np.zeros((T, H, dk))
    dval = np.zeros((T, H, dv))
    dg = np.zeros((T, H, dk))
    dbeta = np.zeros((T, H))
    dS0 = np.zeros((N, H, dk, dv))
    rc = (_lib or _load()).kda_oracle_prefill_backward_f64(
        N, _ptr(cu), H, dk, dv, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(S0), _ptr(d_o), _ptr(dST), _ptr(dq), _ptr(dkey), _ptr(dval), _ptr(dg), _ptr(dbeta),
        _ptr(dS0), int(seg_len), int(nthreads))
    if rc != 0:
        raise ValueError("kda_oracle_prefill_backward_f64 failed with %d" % rc)
    return dq, dkey, dval, dg, dbeta, dS0
