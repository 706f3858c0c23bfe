"""CPU fp64 oracle for the KDA core -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it and shares no code with it.
"""
from .kda_oracle import (  # noqa: F401
    OracleLib,
    compile_source,
    build,
    decode_step,
    gate,
    l2norm,
    lib_path,
    max_threads,
    output_gate,
    prefill,
    prefill_backward,
    prefill_checkpoints,
    prefill_fused,
)
