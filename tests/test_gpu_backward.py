"""kda_prefill_backward against the fp64 oracle's reverse-mode gradients.

The oracle differentiates the token recurrence (pinned by finite differences
and autograd in test_oracle_pins); the GPU differentiates the chunked form
with bf16 MFMA operands.  Each gradient tensor is compared with the bf16 rule
used for the forward outputs: max |difference| <= 2e-2 * max |reference|.
Cases: ragged packed batches with an empty and a one-token sequence, initial
states and final-state gradients, a readout scale, the three decay regimes of
the synthetic workloads (K3-strength, mild and zero decay), beta at 0 and 1,
a dense batch, determinism, and the dense 32K x 96 workload on every head.
"""
import numpy as np
import pytest
import torch

from gpu_common import TOL, f64, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16 = torch.bfloat16
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


@pytest.fixture(scope="module")
def kda():
    import linear_attention_recurrence_delta_amd as m
    return m


def _case(lengths, H, seed, g_mode="k3", init_std=0.05, dst_std=0.05):
    from linear_attention_recurrence_delta_amd import synth
    T = sum(lengths)
    q, k, v, g, beta, gen = synth.token_inputs(T, H, 128, 128, BF16, seed, DEV, g_mode)
    N = len(lengths)
    S0 = synth.initial_state(N, H, 128, 128, init_std, gen, DEV) if init_std else None
    dST = synth.initial_state(N, H, 128, 128, dst_std, gen, DEV) if dst_std else None
    d_o = torch.randn((T, H, 128), generator=gen, device=DEV).to(BF16)
    cu_list = [0] + [int(x) for x in np.cumsum(lengths)]
    cu = torch.tensor(cu_list, dtype=torch.int32, device=DEV)
    return dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0, dST=dST, d_o=d_o, cu=cu, cu_list=cu_list)


def _check(kda, oracle_mod, w, label, scale=1.0, cu=True):
    got = kda.kda_prefill_backward(w["q"], w["k"], w["v"], w["g"], w["beta"], w["d_o"], w["S0"], w["dST"],
                                   w["cu"] if cu else None, scale=scale,
                                   num_seqs=None if cu else len(w["cu_list"]) - 1)
    torch.cuda.synchronize()
    ref = oracle_mod.prefill_backward(f64(w["q"]), f64(w["k"]), f64(w["v"]), f64(w["g"]), f64(w["beta"]),
                                      f64(w["d_o"]), None if w["S0"] is None else f64(w["S0"]),
                                      None if w["dST"] is None else f64(w["dST"]),
                                      np.array(w["cu_list"]), scale=scale)
    errs = {}
    for name, a, b in zip(NAMES, got, ref):
        a = f64(a)
        assert np.isfinite(a).all(), name
        errs[name] = rel_err(a, b)
    say("  %s: " % label + " ".join("%s=%.2e" % kv for kv in errs.items()))
    for name, e in errs.items():
        assert e <= TOL[BF16], (name, e)
    return got


def test_ragged_varlen_with_states(kda, oracle_mod):
    say("CASE backward varlen [37, 0, 64, 1, 130, 16] H=2, S0 and dS_T, scale 0.9")
    w = _case([37, 0, 64, 1, 130, 16], 2, 601)
    _check(kda, oracle_mod, w, "varlen", scale=0.9)


def test_single_sequence_no_states(kda, oracle_mod):
    say("CASE backward T=300 H=3, no S0, no dS_T")
    w = _case([300], 3, 602, init_std=None, dst_std=None)
    _check(kda, oracle_mod, w, "plain")


@pytest.mark.parametrize("g_mode", ["mild", "zero"])
def test_long_memory_decay(kda, oracle_mod, g_mode):
    """Weak or no decay: state gradients travel across many chunks."""
    say("CASE backward g_mode=%s [200, 77] H=2" % g_mode)
    w = _case([200, 77], 2, 603, g_mode=g_mode)
    _check(kda, oracle_mod, w, g_mode)


def test_beta_limits(kda, oracle_mod):
    """beta = 0 for a stretch (no writes) and beta = 1 elsewhere."""
    say("CASE backward beta in {0, 1}")
    w = _case([96, 45], 2, 604)
    b = w["beta"]
    b[:20] = 0.0
    b[20:] = 1.0
    _check(kda, oracle_mod, w, "beta 0/1")


def test_dense_batch_layout(kda, oracle_mod):
    say("CASE backward dense N=3 x 64 H=2 (no cu_seqlens)")
    w = _case([64, 64, 64], 2, 605)
    _check(kda, oracle_mod, w, "dense", cu=False)


def test_deterministic(kda):
    say("CASE backward determinism")
    w = _case([150, 90], 2, 606)
    a = kda.kda_prefill_backward(w["q"], w["k"], w["v"], w["g"], w["beta"], w["d_o"], w["S0"], w["dST"], w["cu"])
    b = kda.kda_prefill_backward(w["q"], w["k"], w["v"], w["g"], w["beta"], w["d_o"], w["S0"], w["dST"], w["cu"])
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_dense_k3_all_heads(kda, oracle_mod):
    """B=1 T=32768 H=96: every head's gradients against the oracle's adjoint,
    16 heads per oracle call."""
    from linear_attention_recurrence_delta_amd import synth
    say("CASE backward k3 dense 32K x 96, every head")
    T, H = 32768, 96
    q, k, v, g, beta, gen = synth.token_inputs(T, H, 128, 128, BF16, 607, DEV)
    d_o = torch.randn((T, H, 128), generator=gen, device=DEV).to(BF16)
    got = kda.kda_prefill_backward(q, k, v, g, beta, d_o)
    torch.cuda.synchronize()
    for x in got:
        assert torch.isfinite(x.float()).all()
    errs = {name: 0.0 for name in NAMES[:5] + ("dS0",)}
    for h0 in range(0, H, 16):
        heads = torch.arange(h0, h0 + 16, device=DEV)
        sl = lambda x: f64(x.index_select(1, heads))
        ref = oracle_mod.prefill_backward(sl(q), sl(k), sl(v), sl(g), sl(beta), sl(d_o))
        for name, a, b in zip(NAMES[:5], got[:5], ref[:5]):
            errs[name] = max(errs[name], rel_err(sl(a), b))
        errs["dS0"] = max(errs["dS0"], rel_err(f64(got[5][0].index_select(0, heads)), ref[5][0]))
        say("  heads %d..%d done" % (h0, h0 + 15))
    say("  dense, all 96 heads: " + " ".join("%s=%.2e" % kv for kv in errs.items()))
    for name, e in errs.items():
        assert e <= TOL[BF16], (name, e)


@pytest.mark.parametrize("cu_list", [[0, 500, 100, 300], [-50, 200, 10000], [0, 300, 0, 300]])
def test_malformed_offsets_stay_in_bounds(kda, monkeypatch, cu_list):
    """Malformed cu_seqlens without KDA_VALIDATE: the backward clamps each
    sequence to [0, T_total] as the forward kernels do, so it changes numbers
    but touches no memory outside its buffers.  Each output and the
    workspace sit inside a larger allocation whose guard tail must come back
    untouched.  ([0, 300, 0, 300]: overlapping sequences whose 16-token
    state slots add up past the workspace's T_total / 16.)"""
    import ctypes as ct
    from linear_attention_recurrence_delta_amd._lib import lib
    from linear_attention_recurrence_delta_amd import synth
    monkeypatch.delenv("KDA_VALIDATE", raising=False)
    T, H, N = 300, 2, len(cu_list) - 1
    say("CASE backward malformed cu_seqlens %s" % cu_list)
    q, k, v, g, beta, gen = synth.token_inputs(T, H, 128, 128, BF16, 880, DEV)
    d_o = torch.randn((T, H, 128), generator=gen, device=DEV).to(BF16)
    cu = torch.tensor(cu_list, dtype=torch.int32, device=DEV)
    GUARD = 4096

    def guarded(n, dtype):
        buf = torch.full((n + GUARD,), 7, dtype=dtype, device=DEV)
        return buf, buf[:n]

    outs = {}
    for name, n, dt in (("dq", T * H * 128, BF16), ("dk", T * H * 128, BF16), ("dv", T * H * 128, BF16),
                        ("dg", T * H * 128, torch.float32), ("dbeta", T * H, torch.float32),
                        ("dS0", N * H * 128 * 128, torch.float32)):
        outs[name] = guarded(n, dt)
    wsb = int(lib().kda_prefill_backward_workspace_bytes(N, T, H, 128, 128, 1))
    ws_buf, ws = guarded(wsb, torch.uint8)
    p = lambda t: t.data_ptr()
    st = lib().kda_prefill_backward(N, T, H, 128, 128, 1, 1.0, p(q), p(k), p(v), p(g), p(beta), None, p(cu),
                                    p(d_o), None, p(outs["dq"][1]), p(outs["dk"][1]), p(outs["dv"][1]),
                                    p(outs["dg"][1]), p(outs["dbeta"][1]), p(outs["dS0"][1]), p(ws), wsb,
                                    torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    for name, (buf, _) in outs.items():
        assert bool((buf[-GUARD:] == 7).all()), name
    assert bool((ws_buf[-GUARD:] == 7).all())
