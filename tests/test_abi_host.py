"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every function include/kda.h declares, and
reject bad arguments on the host before any HIP call.  The fake device
pointers used here are never dereferenced: every call below returns from
validation (or is a no-op) before anything is launched.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, NULLP, BAD, UNSUP, MISAL, WS, HIP = 0, 1, 2, 3, 4, 5, 6
BF16, F32 = 1, 0
FAKE = 0x10000  # aligned, never dereferenced


@pytest.fixture(scope="module")
def lib():
    from linear_attention_recurrence_delta_amd._lib import lib as _lib
    return _lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = header_functions()
    for must in ("kda_prefill", "kda_decode_step", "kda_prefill_workspace_bytes",
                 "kda_status_string", "kda_abi_version"):
        assert must in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in header_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_declares_every_header_function():
    from linear_attention_recurrence_delta_amd._lib import SIGNATURES
    assert sorted(SIGNATURES) == header_functions()


def header_statuses():
    text = open(HEADER).read()
    body = re.search(r"typedef enum \{([^}]*)\} kda_status;", text).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    return {int(v): n for n, v in re.findall(r"(KDA_[A-Z_]+)\s*=\s*(\d+)", body)}


def test_version_and_status_strings(lib):
    assert lib.kda_abi_version() == 4
    statuses = header_statuses()
    assert sorted(statuses) == list(range(9))
    for s, name in statuses.items():
        txt = lib.kda_status_string(s).decode()
        assert txt.startswith(name + ":"), (s, txt)
    assert "unknown" in lib.kda_status_string(99).decode()


def test_validate_mode_keeps_host_checks_first(lib, monkeypatch):
    # KDA_VALIDATE=1 adds a device check after the host checks: invalid
    # arguments still fail on the host, before any HIP call.
    monkeypatch.setenv("KDA_VALIDATE", "1")
    v = ctypes.c_void_p
    assert lib.kda_prefill(1, 64, 2, 128, 128, BF16, 0, 1.0, v(FAKE), v(FAKE), v(FAKE), v(FAKE + 8), v(FAKE),
                           None, None, v(FAKE * 2), None, None, 0, None) == MISAL
    assert lib.kda_prefill(1, 64, 2, 128, 128, BF16, 0, 1.0, None, v(FAKE), v(FAKE), v(FAKE), v(FAKE),
                           None, None, v(FAKE * 2), None, None, 0, None) == NULLP
    assert lib.kda_decode_step(0, 4, 128, 128, BF16, 1.0, None, None, None, None, None, None, None, None) == OK


def test_supported_sets(lib):
    for c in (0, 16, 32, 64):
        assert lib.kda_prefill_supported(BF16, 128, 128, c) == 1
    for d in (16, 32, 64, 128):
        assert lib.kda_prefill_supported(F32, d, d, 16) == 1
        assert lib.kda_decode_supported(F32, d, d) == 1
        assert lib.kda_decode_supported(BF16, d, d) == 1
    assert lib.kda_prefill_supported(BF16, 128, 64, 64) == 0
    assert lib.kda_prefill_supported(BF16, 100, 100, 64) == 0
    assert lib.kda_prefill_supported(BF16, 128, 128, 48) == 0
    assert lib.kda_prefill_supported(7, 128, 128, 64) == 0
    assert lib.kda_decode_supported(BF16, 128, 64) == 0
    assert lib.kda_decode_supported(3, 128, 128) == 0


def _prefill(lib, N=1, T=64, H=2, dk=128, dv=128, dt=BF16, C=64, q=FAKE, k=FAKE, v=FAKE, g=FAKE,
             beta=FAKE, S0=None, cu=None, o=FAKE + 0x100000, fs=None, ws=None, wsb=0):
    return lib.kda_prefill(N, T, H, dk, dv, dt, C, 1.0, q, k, v, g, beta, S0, cu, o, fs, ws, wsb, None)


def test_prefill_validation(lib):
    assert _prefill(lib, N=-1) == BAD
    assert _prefill(lib, T=-5) == BAD
    assert _prefill(lib, H=0) == BAD
    assert _prefill(lib, N=0, T=10) == BAD            # tokens without sequences
    assert _prefill(lib, N=3, T=64) == BAD            # dense length must divide
    assert _prefill(lib, dk=100, dv=100) == UNSUP
    assert _prefill(lib, dk=128, dv=64) == UNSUP
    assert _prefill(lib, C=48) == UNSUP
    assert _prefill(lib, dt=5) == UNSUP
    assert _prefill(lib, T=1 << 31) == UNSUP
    # 16 token rows of every head (fp32, d = 128) must stay below 2^31 bytes
    # (q = NULL: the call stops at the pointer checks, which come after the size checks)
    assert _prefill(lib, N=1, T=16, H=262143, q=None) == NULLP
    assert _prefill(lib, N=1, T=16, H=262144, q=None) == UNSUP
    assert _prefill(lib, q=None) == NULLP
    assert _prefill(lib, beta=None) == NULLP
    assert _prefill(lib, o=None) == NULLP
    assert _prefill(lib, k=FAKE + 8) == MISAL
    assert _prefill(lib, S0=FAKE + 4) == MISAL
    assert _prefill(lib, cu=FAKE + 2, N=2) == MISAL
    assert _prefill(lib, beta=FAKE + 2) == MISAL
    assert _prefill(lib, g=FAKE + 4) == MISAL
    assert _prefill(lib, o=FAKE) == BAD               # o == q
    # no-ops that launch nothing
    assert _prefill(lib, N=0, T=0) == OK
    assert _prefill(lib, N=0, T=0, q=None, k=None, v=None, g=None, beta=None, o=None) == OK
    assert _prefill(lib, N=2, T=0, q=None, k=None, v=None, g=None, beta=None, o=None) == OK


def test_workspace_query(lib):
    assert lib.kda_prefill_workspace_bytes(1, 4096, 8, 128, 128, BF16, 64) == 0
    # direct chains: many (sequence, head) units, or short sequences
    assert lib.kda_prefill_workspace_bytes(1, 32768, 96, 128, 128, BF16, 0) == 0
    assert lib.kda_prefill_workspace_bytes(1, 4096, 8, 128, 128, BF16, 0) == 0
    assert lib.kda_prefill_workspace_bytes(1, 1 << 20, 16, 128, 128, F32, 0) == 0  # no pipeline for fp32


def _desc(**kw):
    from linear_attention_recurrence_delta_amd._lib import PrefillDesc
    base = dict(num_seqs=1, total_tokens=1 << 20, num_heads=16, d_k=128, d_v=128, qkv_dtype=BF16, chunk_size=0,
                scale=1.0, fused=0, checkpoint_interval=0, checkpoint_capacity=0, kernel=0, slab_columns=0,
                segments=0)
    base.update(kw)
    return PrefillDesc(**base)


def test_desc_layout_matches_header():
    # the ctypes mirror of kda_prefill_desc has the C layout (int64 fields
    # 8-byte aligned): 72 bytes, total_tokens at 8, checkpoint_capacity at 48
    from linear_attention_recurrence_delta_amd._lib import PrefillDesc, PrefillTensors
    import ctypes as ct
    assert ct.sizeof(PrefillDesc) == 72
    assert PrefillDesc.total_tokens.offset == 8 and PrefillDesc.checkpoint_capacity.offset == 48
    assert ct.sizeof(PrefillTensors) == 12 * 8
    text = open(HEADER).read()
    body = re.search(r"typedef struct \{(.*?)\} kda_prefill_desc;", text, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    assert re.findall(r"(\w+);", body) == [f[0] for f in PrefillDesc._fields_]
    body = re.search(r"typedef struct \{(.*?)\} kda_prefill_tensors;", text, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    names = re.findall(r"\*\s*(\w+)", body)
    assert names == [f[0] for f in PrefillTensors._fields_]


def test_segment_scan_workspace(lib):
    # One 1,048,576-token sequence of 16 heads on a 256-CU device (the count
    # used when no device answers): 17 segments (16 workgroups per head in
    # both launches), 16 slots of 2 x 64 KiB per head.  Packed or checkpointed
    # or fp32 calls need none.
    import ctypes as ct
    ex = lambda **kw: lib.kda_prefill_ex_workspace_bytes(ct.byref(_desc(**kw)))
    assert ex() == 16 * 16 * 2 * 128 * 128 * 4
    assert ex(segments=1) == 0
    assert ex(segments=5) == 16 * 4 * 2 * 128 * 128 * 4
    assert ex(segments=300) == 0                      # beyond the built maximum
    assert ex(checkpoint_interval=1024, checkpoint_capacity=1024) == 0
    assert ex(fused=1) == 0
    assert ex(qkv_dtype=F32) == 0
    assert ex(kernel=2) == 0                          # chunk-staged: no scan
    assert ex(num_heads=96, total_tokens=32768) == 0  # 96 units: no room
    assert lib.kda_prefill_ex_workspace_bytes(None) == 0


def test_prefill_ex_validation(lib):
    import ctypes as ct
    from linear_attention_recurrence_delta_amd._lib import PrefillTensors
    t = PrefillTensors(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, o=FAKE + 0x100000)
    run = lambda d, tens=t, ws=None, wsb=0: lib.kda_prefill_ex(ct.byref(d), ct.byref(tens), ws, wsb, None)
    small = dict(total_tokens=4096, num_heads=2)
    assert lib.kda_prefill_ex(None, ct.byref(t), None, 0, None) == NULLP
    assert lib.kda_prefill_ex(ct.byref(_desc()), None, None, 0, None) == NULLP
    assert run(_desc(kernel=3, **small)) == BAD
    assert run(_desc(slab_columns=-1, **small)) == BAD
    assert run(_desc(segments=-2, **small)) == BAD
    assert run(_desc(slab_columns=48, segments=1, num_seqs=0, total_tokens=0)) == OK  # nothing to run
    assert run(_desc(kernel=1, chunk_size=32, **small)) == UNSUP     # the pipeline is chunk 16 only
    tf = PrefillTensors(q=FAKE, k=FAKE, v=FAKE, z=FAKE, a_log=FAKE, beta=FAKE, o=FAKE + 0x100000)
    assert run(_desc(kernel=2, fused=1, **small), tf) == UNSUP       # the fused gate is pipelined only
    assert run(_desc(kernel=1, fused=1, **small)) == NULLP           # fused without z / a_log
    assert run(_desc(segments=4, **small), PrefillTensors(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE,
                                                          cu_seqlens=FAKE, o=FAKE + 0x100000)) == UNSUP
    assert run(_desc(segments=4, qkv_dtype=F32, **small)) == UNSUP
    assert run(_desc(segments=300, **small)) == UNSUP
    assert run(_desc(segments=300, num_seqs=1, total_tokens=64, num_heads=2)) == UNSUP  # 4 chunks < 301
    assert run(_desc(segments=4, **small)) == WS                     # the maps need a workspace
    assert run(_desc(segments=4, **small), ws=FAKE, wsb=1 << 40) == BAD  # workspace == q


def test_offset_clamp_rule(tmp_path):
    """kda_bounds.h, the rule every kernel applies to cu_seqlens offsets,
    compiled with g++ and driven over well-formed and malformed offsets:
    ranges stay inside [0, T] with end >= start, and well-formed offsets
    pass unchanged."""
    src = tmp_path / "clamp.cpp"
    src.write_text(r"""
#include "kda_bounds.h"
#include <cstdio>
#include <cstdlib>
int main() {
    unsigned s = 12345;
    auto rnd = [&]() { s = s * 1103515245u + 12345u; return (int64_t)((s >> 8) % 4001) - 2000; };
    for (int i = 0; i < 200000; ++i) {
        const int64_t T = (rnd() + 2000) / 2, x = rnd(), y = rnd();
        const kda::SeqRange r = kda::clamp_seq(x, y, T);
        if (!(0 <= r.a && r.a <= r.b && r.b <= T)) { std::puts("bad"); return 1; }
        if (0 <= x && x <= y && y <= T && (r.a != x || r.b != y)) { std::puts("changed"); return 1; }
    }
    static_assert(kda::clamp_seq(-3, 5, 4).a == 0 && kda::clamp_seq(-3, 5, 4).b == 4, "");
    static_assert(kda::clamp_seq(3, 1, 10).a == 3 && kda::clamp_seq(3, 1, 10).b == 3, "");
    std::puts("ok");
    return 0;
}
""")
    import subprocess
    exe = tmp_path / "clamp"
    csrc = os.path.join(ROOT, "linear_attention_recurrence_delta_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", csrc, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout


def _decode(lib, N=4, H=2, d=128, dt=BF16, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE,
            S=FAKE + 0x200000, o=FAKE + 0x100000):
    return lib.kda_decode_step(N, H, d, d, dt, 1.0, q, k, v, g, beta, S, o, None)


def test_decode_validation(lib):
    assert _decode(lib, N=-1) == BAD
    assert _decode(lib, H=0) == BAD
    assert _decode(lib, d=100) == UNSUP
    assert _decode(lib, dt=9) == UNSUP
    assert _decode(lib, S=None) == NULLP
    assert _decode(lib, q=None) == NULLP
    assert _decode(lib, v=FAKE + 4) == MISAL
    assert _decode(lib, S=FAKE + 0x200008) == MISAL
    assert _decode(lib, beta=FAKE + 1) == MISAL
    assert _decode(lib, o=FAKE + 0x200000) == BAD     # o == state
    assert _decode(lib, N=0, q=None, k=None, v=None, g=None, beta=None, S=None, o=None) == OK


def test_python_binding_rejects_host_tensors():
    import torch
    from linear_attention_recurrence_delta_amd import kda_prefill, kda_decode_step
    x = torch.zeros(4, 1, 16)
    b = torch.zeros(4, 1)
    with pytest.raises(ValueError):
        kda_prefill(x, x, x, x, b)
    with pytest.raises(ValueError):
        kda_decode_step(x, x, x, x, b, torch.zeros(4, 1, 16, 16))


def test_varlen_recipe():
    from linear_attention_recurrence_delta_amd.synth import varlen_lengths
    L = varlen_lengths()
    assert len(L) == 16 and sum(L) == 32768
    assert min(L) >= 256 and max(L) <= 8192
    assert any(x % 64 for x in L)  # ragged tails are exercised
    assert varlen_lengths() == L   # seeded


def test_library_has_no_oracle_dependency():
    """The product library must not link or name the oracle."""
    from linear_attention_recurrence_delta_amd._lib import LIB_PATH
    blob = open(LIB_PATH, "rb").read()
    assert b"kda_oracle" not in blob
    src_dir = os.path.join(ROOT, "linear_attention_recurrence_delta_amd")
    for dirpath, _, files in os.walk(src_dir):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, f
                assert "kda_oracle" not in txt, f


def _prefill_ck(lib, N=1, T=64, H=2, d=128, C=0, interval=16, ck=FAKE + 0x400000, cap=4, o=FAKE + 0x100000,
                fs=None, cu=None):
    return lib.kda_prefill_checkpointed(N, T, H, d, d, BF16, C, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, None, cu, o, fs,
                                        interval, ck, cap, None, 0, None)


def test_prefill_checkpointed_validation(lib):
    assert _prefill_ck(lib, interval=0) == BAD          # no interval
    assert _prefill_ck(lib, interval=-16) == BAD
    assert _prefill_ck(lib, interval=24) == BAD         # not a multiple of the default chunk 16
    assert _prefill_ck(lib, C=64, interval=32) == BAD   # not a multiple of chunk 64
    assert _prefill_ck(lib, cap=3) == BAD               # floor(64 / 16) = 4 slots needed
    assert _prefill_ck(lib, cap=-1) == BAD
    assert _prefill_ck(lib, ck=None) == NULLP
    assert _prefill_ck(lib, ck=FAKE + 0x400008) == MISAL
    assert _prefill_ck(lib, ck=FAKE) == BAD             # checkpoints == q
    assert _prefill_ck(lib, ck=FAKE + 0x100000) == BAD  # checkpoints == o
    assert _prefill_ck(lib, d=100) == UNSUP
    # checks shared with kda_prefill still come first
    assert _prefill_ck(lib, o=None) == NULLP
    assert _prefill_ck(lib, N=3) == BAD
    # no checkpoint fits: capacity 0 and a NULL buffer are fine (nothing launched for N = 0)
    assert _prefill_ck(lib, N=0, T=0, interval=16, ck=None, cap=0) == OK


def _prefill_fused(lib, N=1, T=64, H=2, d=128, dt=BF16, C=0, q=FAKE, z=FAKE + 0x300000, a=FAKE + 0x500000,
                   o=FAKE + 0x100000):
    return lib.kda_prefill_fused(N, T, H, d, d, dt, C, 1.0, q, FAKE, FAKE, z, a, FAKE, None, None, o, None,
                                 None, 0, None)


def test_prefill_fused_supported_set(lib):
    assert lib.kda_prefill_fused_supported(BF16, 128, 128, 0) == 1
    assert lib.kda_prefill_fused_supported(BF16, 128, 128, 16) == 1
    assert lib.kda_prefill_fused_supported(BF16, 128, 128, 64) == 0
    assert lib.kda_prefill_fused_supported(F32, 128, 128, 16) == 0
    assert lib.kda_prefill_fused_supported(BF16, 64, 64, 16) == 0


def test_prefill_fused_validation(lib):
    assert _prefill_fused(lib, z=None) == NULLP
    assert _prefill_fused(lib, a=None) == NULLP
    assert _prefill_fused(lib, z=FAKE + 0x300008) == MISAL
    assert _prefill_fused(lib, a=FAKE + 0x500002) == MISAL
    assert _prefill_fused(lib, o=FAKE + 0x300000) == BAD   # o == z
    assert _prefill_fused(lib, dt=F32) == UNSUP
    assert _prefill_fused(lib, C=64) == UNSUP
    assert _prefill_fused(lib, d=64) == UNSUP
    assert _prefill_fused(lib, N=3) == BAD
    assert _prefill_fused(lib, N=0, T=0, q=None, z=None, a=None, o=None) == OK


def _gate(lib, T=10, H=2, dv=128, dt=BF16, eps=1e-6, o=FAKE, g=FAKE + 0x100000, w=FAKE + 0x200000,
          y=FAKE + 0x300000):
    return lib.kda_output_gate(T, H, dv, dt, eps, o, g, w, y, None)


def test_output_gate_validation(lib):
    for d in (16, 32, 64, 128):
        assert lib.kda_output_gate_supported(BF16, d) == 1 and lib.kda_output_gate_supported(F32, d) == 1
    assert lib.kda_output_gate_supported(BF16, 96) == 0 and lib.kda_output_gate_supported(5, 128) == 0
    assert _gate(lib, T=-1) == BAD
    assert _gate(lib, H=0) == BAD
    assert _gate(lib, eps=-1.0) == BAD
    assert _gate(lib, eps=float("nan")) == BAD
    assert _gate(lib, dv=96) == UNSUP
    assert _gate(lib, dt=7) == UNSUP
    assert _gate(lib, o=None) == NULLP
    assert _gate(lib, w=None) == NULLP
    assert _gate(lib, y=FAKE + 0x300008) == MISAL
    assert _gate(lib, w=FAKE + 0x200002) == MISAL
    assert _gate(lib, y=FAKE + 0x200000) == BAD   # y == weight
    assert _gate(lib, T=0, o=None, g=None, w=None, y=None) == OK


def _bwd(lib, N=1, T=32, H=2, d=128, dt=BF16, q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, g=FAKE + 0x300000,
         b=FAKE + 0x400000, S0=None, cu=None, do=FAKE + 0x500000, dST=None, dq=FAKE + 0x600000,
         dk=FAKE + 0x700000, dv=FAKE + 0x800000, dg=FAKE + 0x900000, db=FAKE + 0xa00000, dS0=None,
         ws=FAKE + 0x1000000, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.kda_prefill_backward_workspace_bytes(N, T, H, d, d, dt)
    return lib.kda_prefill_backward(N, T, H, d, d, dt, 1.0, q, k, v, g, b, S0, cu, do, dST, dq, dk, dv, dg, db,
                                    dS0, ws, ws_bytes, None)


def test_prefill_backward_supported_set_and_workspace(lib):
    assert lib.kda_prefill_backward_supported(BF16, 128, 128) == 1
    assert lib.kda_prefill_backward_supported(F32, 128, 128) == 0
    assert lib.kda_prefill_backward_supported(BF16, 64, 64) == 0
    assert lib.kda_prefill_backward_supported(BF16, 128, 64) == 0
    # one bf16 state per head for every full 16 tokens, the two value halves'
    # fp32 partials of dq, dk, dg and dbeta, the bf16 initial states
    r256 = lambda b: -(-b // 256) * 256
    want = lambda N, T, H: (r256((T // 16) * H * 128 * 128 * 2) + r256(2 * T * H * (3 * 128 + 1) * 4) +
                            r256(N * H * 128 * 128 * 2))
    assert lib.kda_prefill_backward_workspace_bytes(2, 100, 3, 128, 128, BF16) == want(2, 100, 3)
    assert lib.kda_prefill_backward_workspace_bytes(1, 15, 3, 128, 128, BF16) == want(1, 15, 3)
    assert lib.kda_prefill_backward_workspace_bytes(0, 0, 3, 128, 128, BF16) == want(0, 0, 3)
    assert lib.kda_prefill_backward_workspace_bytes(1, 64, 3, 128, 128, F32) == 0


def test_prefill_backward_validation(lib):
    assert _bwd(lib, T=-1) == BAD
    assert _bwd(lib, H=0) == BAD
    assert _bwd(lib, dt=F32) == UNSUP
    assert _bwd(lib, d=64) == UNSUP
    assert _bwd(lib, N=3) == BAD                        # 32 tokens do not split into 3 equal sequences
    assert _bwd(lib, N=0) == BAD                        # tokens without sequences
    assert _bwd(lib, H=262144, q=None) == UNSUP         # 16 rows of the heads exceed 2^31 bytes
    assert _bwd(lib, H=262143, q=None) == NULLP
    for name in ("q", "k", "v", "g", "b", "do", "dq", "dk", "dv", "dg", "db"):
        assert _bwd(lib, **{name: None}) == NULLP, name
    assert _bwd(lib, dq=FAKE + 0x600008) == MISAL
    assert _bwd(lib, db=FAKE + 0xa00002) == MISAL
    assert _bwd(lib, dS0=FAKE + 0xb00008) == MISAL
    assert _bwd(lib, dq=FAKE) == BAD                    # dq == q
    assert _bwd(lib, dv=FAKE + 0x600000) == BAD         # dv == dq
    assert _bwd(lib, dS0=FAKE + 0x1000000) == BAD       # d_initial_state == workspace
    assert _bwd(lib, ws=None) == WS
    assert _bwd(lib, ws_bytes=100) == WS
    assert _bwd(lib, N=0, T=0, q=None, k=None, v=None, g=None, b=None, do=None, dq=None, dk=None, dv=None,
                dg=None, db=None, ws=None, ws_bytes=0) == OK


def test_prefill_ex_noalloc_host_checks(lib):
    """kda_prefill_ex_noalloc refuses, before any HIP call, a plan whose
    workspace exceeds the static buffer (64 MiB), and validates like
    kda_prefill_ex."""
    import ctypes as ct
    from linear_attention_recurrence_delta_amd._lib import PrefillTensors
    assert lib.kda_noalloc_scratch_bytes() == 64 << 20
    t = PrefillTensors(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, o=FAKE + 0x100000)
    SCRATCH = 8
    big = _desc(total_tokens=8192, num_heads=4, segments=256)  # 4 x 255 maps of 128 KiB = 127.5 MiB
    assert lib.kda_prefill_ex_workspace_bytes(ct.byref(big)) == 4 * 255 * 2 * 128 * 128 * 4
    assert lib.kda_prefill_ex_noalloc(ct.byref(big), ct.byref(t), None) == SCRATCH
    assert lib.kda_prefill_ex_noalloc(None, ct.byref(t), None) == NULLP
    assert lib.kda_prefill_ex_noalloc(ct.byref(_desc(num_heads=0)), ct.byref(t), None) == BAD
    assert lib.kda_prefill_ex_noalloc(ct.byref(_desc(kernel=7)), ct.byref(t), None) == BAD
    bad_q = PrefillTensors(q=FAKE + 8, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, o=FAKE + 0x100000)
    assert lib.kda_prefill_ex_noalloc(ct.byref(_desc()), ct.byref(bad_q), None) == MISAL
    assert lib.kda_prefill_ex_noalloc(ct.byref(_desc(num_seqs=0, total_tokens=0)), ct.byref(t), None) == OK
