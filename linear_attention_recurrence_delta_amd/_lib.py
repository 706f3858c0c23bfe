"""Load libkda.so (built in-tree by ``build_lib.py``) and declare its C ABI.

There is no fallback: if the library is missing or fails to load, every
entry point raises.  The symbols and signatures mirror ``include/kda.h``.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")

_lock = threading.Lock()
_lib = None

# name -> (restype, argtypes)
_i32, _i64, _f32, _sz, _vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                              ctypes.c_size_t, ctypes.c_void_p)


class PrefillDesc(ctypes.Structure):
    """kda_prefill_desc (include/kda.h), same field order and C layout."""
    _fields_ = [("num_seqs", _i32), ("total_tokens", _i64), ("num_heads", _i32), ("d_k", _i32),
                ("d_v", _i32), ("qkv_dtype", _i32), ("chunk_size", _i32), ("scale", _f32), ("fused", _i32),
                ("checkpoint_interval", _i32), ("checkpoint_capacity", _i64), ("kernel", _i32),
                ("slab_columns", _i32), ("segments", _i32)]


class PrefillTensors(ctypes.Structure):
    """kda_prefill_tensors (include/kda.h): device pointers."""
    _fields_ = [(n, _vp) for n in ("q", "k", "v", "g", "z", "a_log", "beta", "initial_state", "cu_seqlens",
                                   "o", "final_state", "checkpoints")]


_pdesc, _ptens = ctypes.POINTER(PrefillDesc), ctypes.POINTER(PrefillTensors)
SIGNATURES = {
    "kda_abi_version": (_i32, []),
    "kda_status_string": (ctypes.c_char_p, [_i32]),
    "kda_prefill_supported": (_i32, [_i32, _i32, _i32, _i32]),
    "kda_decode_supported": (_i32, [_i32, _i32, _i32]),
    "kda_prefill_workspace_bytes": (_sz, [_i32, _i64, _i32, _i32, _i32, _i32, _i32]),
    "kda_prefill": (_i32, [_i32, _i64, _i32, _i32, _i32, _i32, _i32, _f32,
                           _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kda_prefill_checkpointed": (_i32, [_i32, _i64, _i32, _i32, _i32, _i32, _i32, _f32,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _i32, _vp, _i64, _vp, _sz, _vp]),
    "kda_prefill_ex_workspace_bytes": (_sz, [_pdesc]),
    "kda_prefill_ex": (_i32, [_pdesc, _ptens, _vp, _sz, _vp]),
    "kda_noalloc_scratch_bytes": (_sz, []),
    "kda_prefill_ex_noalloc": (_i32, [_pdesc, _ptens, _vp]),
    "kda_prefill_fused_supported": (_i32, [_i32, _i32, _i32, _i32]),
    "kda_prefill_fused": (_i32, [_i32, _i64, _i32, _i32, _i32, _i32, _i32, _f32,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kda_prefill_output_gated": (_i32, [_i32, _i64, _i32, _i32, _i32, _i32, _i32, _f32,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f32, _vp, _vp,
                                        _vp, _sz, _vp]),
    "kda_output_gate_supported": (_i32, [_i32, _i32]),
    "kda_output_gate": (_i32, [_i64, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _vp, _vp]),
    "kda_prefill_backward_supported": (_i32, [_i32, _i32, _i32]),
    "kda_prefill_backward_workspace_bytes": (_sz, [_i32, _i64, _i32, _i32, _i32, _i32]),
    "kda_prefill_backward": (_i32, [_i32, _i64, _i32, _i32, _i32, _i32, _f32,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "kda_decode_step": (_i32, [_i32, _i32, _i32, _i32, _i32, _f32,
                               _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
}


class LibraryMissing(RuntimeError):
    pass


def lib():
    """The loaded library (ctypes.CDLL) with argument types declared."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise LibraryMissing(
                    "libkda.so is not built (%s); run __graft_entry__.build() or "
                    "python -m linear_attention_recurrence_delta_amd.build_lib" % LIB_PATH)
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib
