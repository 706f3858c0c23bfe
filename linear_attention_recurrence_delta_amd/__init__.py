"""MI355X-native Kimi Delta Attention (KDA) core.

The compute lives in libkda.so (hand-written HIP for gfx950, C ABI in
``include/kda.h``); this package is its thin Python binding.
"""
from ._lib import LIB_PATH, LibraryMissing  # noqa: F401
from .kda import (  # noqa: F401
    KDA_DTYPE_BF16,
    KDA_DTYPE_F32,
    KDA_KERNEL_AUTO,
    KDA_KERNEL_CHUNK_STAGED,
    KDA_KERNEL_PIPELINED,
    KdaError,
    kda_abi_version,
    kda_decode_step,
    kda_decode_supported,
    kda_prefill,
    kda_prefill_backward,
    kda_prefill_backward_supported,
    kda_prefill_checkpointed,
    kda_prefill_ex_workspace_bytes,
    kda_prefill_fused,
    kda_prefill_fused_supported,
    kda_prefill_output_gated,
    kda_output_gate,
    kda_noalloc_scratch_bytes,
    kda_output_gate_supported,
    kda_prefill_supported,
    kda_prefill_workspace_bytes,
)
