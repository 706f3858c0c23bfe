"""kda_prefill_fused: gate and q/k L2 norm computed in the kernel.

The oracle prepares its inputs as the pages define them (L2Norm of q and k,
g = -5 Sigmoid(e^{A_h} z)) in fp64 from the very bf16/fp32 values handed to
the GPU, then runs its token recurrence.  Cases: ragged varlen with raw q/k
of varied norms and per-head A, zero query/key vectors, an initial state,
bitwise invariance across value-slab widths, and the dense K3 workload on
every head.
"""
import numpy as np
import pytest
import torch

from gpu_common import TOL, f64, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16 = torch.bfloat16


@pytest.fixture(scope="module")
def kda():
    import linear_attention_recurrence_delta_amd as m
    return m


def _inputs(lengths, H, seed, a_log_std=0.3, init_std=None):
    from linear_attention_recurrence_delta_amd import synth
    T = sum(lengths)
    q, k, v, z, a_log, beta, gen = synth.fused_inputs(T, H, 128, BF16, seed, DEV, a_log_std=a_log_std)
    S0 = synth.initial_state(len(lengths), H, 128, 128, init_std, gen, DEV) if init_std else None
    cu_list = [0] + [int(x) for x in np.cumsum(lengths)]
    cu = torch.tensor(cu_list, dtype=torch.int32, device=DEV) if len(lengths) > 1 else None
    return dict(q=q, k=k, v=v, z=z, a_log=a_log, beta=beta, S0=S0, cu=cu, cu_list=cu_list)


def _check(kda, oracle_mod, w, label):
    o, S = kda.kda_prefill_fused(w["q"], w["k"], w["v"], w["z"], w["a_log"], w["beta"], w["S0"], w["cu"])
    torch.cuda.synchronize()
    ro, rs = oracle_mod.prefill_fused(f64(w["q"]), f64(w["k"]), f64(w["v"]), f64(w["z"]), f64(w["a_log"]),
                                      f64(w["beta"]), None if w["S0"] is None else f64(w["S0"]),
                                      np.array(w["cu_list"]))
    eo, es = rel_err(f64(o), ro), rel_err(f64(S), rs)
    say("  %s: rel err o=%.3e S=%.3e" % (label, eo, es))
    assert np.isfinite(f64(o)).all() and np.isfinite(f64(S)).all()
    assert eo <= TOL[BF16] and es <= TOL[BF16]
    return o, S


def test_ragged_varlen(kda, oracle_mod):
    say("CASE fused varlen [37, 0, 64, 1, 130, 200, 16] H=3")
    w = _inputs([37, 0, 64, 1, 130, 200, 16], 3, 401)
    _check(kda, oracle_mod, w, "varlen")


def test_initial_state_single_sequence(kda, oracle_mod):
    say("CASE fused T=300 H=2 with S0")
    w = _inputs([300], 2, 402, init_std=0.05)
    _check(kda, oracle_mod, w, "S0")


def test_zero_query_and_key_vectors(kda, oracle_mod):
    """L2Norm of a zero vector is taken as zero: a zero key writes nothing,
    a zero query reads zero."""
    say("CASE fused zero q/k rows")
    w = _inputs([90], 2, 403)
    w["q"][5, 0].zero_()
    w["q"][40:43, 1].zero_()
    w["k"][7, 1].zero_()
    w["k"][60, 0].zero_()
    o, _ = _check(kda, oracle_mod, w, "zero rows")
    assert bool((o[5, 0] == 0).all()) and bool((o[40:43, 1] == 0).all())


def test_gate_scale_extremes(kda, oracle_mod):
    """Large |A_h| drive the gate to its limits (g near -5 or 0 per sign of z)."""
    say("CASE fused extreme a_log")
    w = _inputs([150, 70], 4, 404)
    w["a_log"] = torch.tensor([-4.0, 0.0, 2.0, 3.5], device=DEV)
    _check(kda, oracle_mod, w, "a_log extremes")


@pytest.mark.parametrize("cols", [16, 32, 64, 128])
def test_slab_width_invariance(kda, cols):
    say("CASE fused slab width %d columns" % cols)
    w = _inputs([120, 77], 2, 405)
    ref = kda.kda_prefill_fused(w["q"], w["k"], w["v"], w["z"], w["a_log"], w["beta"], None, w["cu"])
    got = kda.kda_prefill_fused(w["q"], w["k"], w["v"], w["z"], w["a_log"], w["beta"], None, w["cu"],
                                plan=dict(slab_columns=cols))
    torch.cuda.synchronize()
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])


def test_dense_k3_all_heads(kda, oracle_mod):
    """B=1 T=32768 H=96, a_log = 0 (the g distribution of the other
    workloads): every head against the oracle, 16 heads per oracle call;
    the outputs start as NaN so that a head the kernel missed fails."""
    from linear_attention_recurrence_delta_amd import synth
    say("CASE fused k3 dense 32K x 96, every head")
    T, H = 32768, 96
    q, k, v, z, a_log, beta, _ = synth.fused_inputs(T, H, 128, BF16, 406, DEV, a_log_std=0.0)
    o = torch.full((T, H, 128), float("nan"), dtype=BF16, device=DEV)
    S = torch.full((1, H, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
    kda.kda_prefill_fused(q, k, v, z, a_log, beta, out=o, final_state=S)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    worst_o = worst_s = 0.0
    for h0 in range(0, H, 16):
        heads = torch.arange(h0, h0 + 16, device=DEV)
        sl = lambda x: f64(x.index_select(1, heads))
        ro, rs = oracle_mod.prefill_fused(sl(q), sl(k), sl(v), sl(z), f64(a_log.index_select(0, heads)), sl(beta))
        worst_o = max(worst_o, rel_err(sl(o), ro))
        worst_s = max(worst_s, rel_err(f64(S[0].index_select(0, heads)), rs[0]))
    say("  dense fused, all 96 heads: rel err o=%.3e S=%.3e" % (worst_o, worst_s))
    assert worst_o <= TOL[BF16] and worst_s <= TOL[BF16]


def test_varlen_k3_all_units(kda, oracle_mod):
    """The 16-sequence K3 varlen pack (32768 tokens, H=96, a_log = 0), which
    runs whole-head workgroups: every (sequence, head) unit against the
    oracle, 16 heads per oracle call; outputs start as NaN."""
    from linear_attention_recurrence_delta_amd import synth
    L = synth.varlen_lengths()
    T, H = int(sum(L)), 96
    say("CASE fused k3 varlen 32K x 96, 16 sequences, every unit")
    q, k, v, z, a_log, beta, _ = synth.fused_inputs(T, H, 128, BF16, 407, DEV, a_log_std=0.0)
    cu_list = [0] + [int(x) for x in np.cumsum(L)]
    cu = torch.tensor(cu_list, dtype=torch.int32, device=DEV)
    o = torch.full((T, H, 128), float("nan"), dtype=BF16, device=DEV)
    S = torch.full((len(L), H, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
    kda.kda_prefill_fused(q, k, v, z, a_log, beta, None, cu, out=o, final_state=S)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    worst_o = worst_s = 0.0
    for h0 in range(0, H, 16):
        heads = torch.arange(h0, h0 + 16, device=DEV)
        sl = lambda x: f64(x.index_select(1, heads))
        ro, rs = oracle_mod.prefill_fused(sl(q), sl(k), sl(v), sl(z), f64(a_log.index_select(0, heads)), sl(beta),
                                          None, np.array(cu_list))
        worst_o = max(worst_o, rel_err(sl(o), ro))
        worst_s = max(worst_s, rel_err(f64(S.index_select(1, heads)), rs))
    say("  varlen fused, all %d units: rel err o=%.3e S=%.3e" % (len(L) * H, worst_o, worst_s))
    assert worst_o <= TOL[BF16] and worst_s <= TOL[BF16]
