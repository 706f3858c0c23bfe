"""GPU parity at the full K3-shaped sizes, in the launch configuration the
benchmark times (library default plan, no initial state for prefill).

Every unit the oracle can afford is compared element by element, with the
output buffers filled with NaN beforehand so that a (sequence, head) the
kernels never wrote cannot pass:

* dense B=1 T=32768 H=96: every output and every final state (the oracle
  runs 16 heads at a time to bound host memory);
* the 16-sequence varlen pack of 32768 tokens: every output and all 16 x 96
  final states;
* long context B=1 T=1,048,576 H=16 (the library runs it as a segment
  scan): outputs of the first 8192 tokens of every head and the final state
  of the 65536-token prefix against the oracle; the whole million tokens
  against the direct chain (every output and final state); the direct
  chain's split-and-resume is bitwise;
* batched decode 256 sequences x 96 heads: every output and every state
  after the first step, then 1000 steps with a seeded sample of 256 units
  tracked against the oracle on every step;
* the dense workload with a state checkpoint every 4096 tokens: all 8
  checkpoints of every head against the oracle's;
* the backward on the varlen pack: every gradient of all 1536 units against
  the oracle's adjoint.
"""
import numpy as np
import pytest
import torch

from gpu_common import TOL, f64, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16_TOL = TOL[torch.bfloat16]
HEAD_BATCH = 16


@pytest.fixture(scope="module")
def kda():
    import linear_attention_recurrence_delta_amd as m
    return m


def _nan_outputs(w, N):
    o = torch.full((w["T"], w["H"], w["d"]), float("nan"), dtype=w["dtype"], device=DEV)
    S = torch.full((N, w["H"], w["d"], w["d"]), float("nan"), dtype=torch.float32, device=DEV)
    return o, S


def _all_units_check(oracle, w, o, S, cu, label, t_limit=None):
    """Every (sequence, head) against the oracle, HEAD_BATCH heads per call
    (all sequences of the pack at once).  t_limit: only the first tokens of a
    single sequence (its final state is then not compared)."""
    T = w["T"] if t_limit is None else t_limit
    worst_o = worst_s = 0.0
    for h0 in range(0, w["H"], HEAD_BATCH):
        hi = torch.arange(h0, min(h0 + HEAD_BATCH, w["H"]), device=DEV)
        sl = lambda x: f64(x[:T].index_select(1, hi))
        ro, rs = oracle.prefill(sl(w["q"]), sl(w["k"]), sl(w["v"]), sl(w["g"]), sl(w["beta"]), None,
                                None if t_limit is not None else cu)
        worst_o = max(worst_o, rel_err(sl(o), ro))
        if S is not None:
            worst_s = max(worst_s, rel_err(f64(S.index_select(1, hi)), rs))
    n_seq = 1 if t_limit is not None or cu is None else len(cu) - 1
    say("  %s: all %d (sequence, head) units, rel err o=%.3e S=%.3e (tol %.0e)"
        % (label, n_seq * w["H"], worst_o, worst_s, BF16_TOL))
    assert np.isfinite(worst_o) and np.isfinite(worst_s)
    assert worst_o <= BF16_TOL and worst_s <= BF16_TOL


def test_k3_dense_32k_all_heads(kda, oracle_mod):
    from linear_attention_recurrence_delta_amd import synth
    say("CASE k3_dense_32k B=1 T=32768 H=96 default plan, every head")
    w = synth.workload_inputs("k3_dense_32k", DEV)
    o, S = _nan_outputs(w, 1)
    kda.kda_prefill(w["q"], w["k"], w["v"], w["g"], w["beta"], None, None, out=o, final_state=S)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    _all_units_check(oracle_mod, w, o, S, np.array([0, w["T"]]), "dense 32K")


def test_k3_varlen_32k_all_units(kda, oracle_mod):
    from linear_attention_recurrence_delta_amd import synth
    w = synth.workload_inputs("k3_varlen_32k", DEV)
    L = w["lengths"]
    say("CASE k3_varlen_32k N=16 T=%d lengths %d..%d, all 1536 units" % (w["T"], min(L), max(L)))
    o, S = _nan_outputs(w, len(L))
    kda.kda_prefill(w["q"], w["k"], w["v"], w["g"], w["beta"], None, w["cu"], out=o, final_state=S)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    cu = np.concatenate([[0], np.cumsum(L)])
    _all_units_check(oracle_mod, w, o, S, cu, "varlen 32K")


def test_long_context_1m_h16(kda, oracle_mod):
    from linear_attention_recurrence_delta_amd import synth
    say("CASE long_1m_h16 B=1 T=1048576 H=16 default plan (segment scan)")
    w = synth.workload_inputs("long_1m_h16", DEV)
    T, H = w["T"], w["H"]
    names = ("q", "k", "v", "g", "beta")
    assert kda.kda_prefill_ex_workspace_bytes(1, T, H, 128, 128, torch.bfloat16) > 0  # the scan is planned
    o, S = _nan_outputs(w, 1)
    kda.kda_prefill(*(w[n] for n in names), None, None, out=o, final_state=S)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()

    # outputs of the first 8192 tokens of every head
    _all_units_check(oracle_mod, w, o, None, None, "first 8192 tokens", t_limit=8192)

    # final state of the 65536-token prefix (itself run as a segment scan)
    P = 65536
    say("  prefix %d tokens" % P)
    pre = {n: w[n][:P].contiguous() for n in names}
    o_p, S_p = kda.kda_prefill(*(pre[n] for n in names), None, None)
    torch.cuda.synchronize()
    wp = dict(w, q=pre["q"], k=pre["k"], v=pre["v"], g=pre["g"], beta=pre["beta"], T=P)
    _all_units_check(oracle_mod, wp, o_p, S_p, np.array([0, P]), "prefix 65536 + state")
    del pre, o_p

    # The whole million tokens against the direct chain (one workgroup chain
    # per head slab over all 65536 chunks): every output and final state.
    o_d, S_d = kda.kda_prefill(*(w[n] for n in names), None, None, plan=dict(segments=1))
    torch.cuda.synchronize()
    e_o = ((o.float() - o_d.float()).abs().max() / o_d.float().abs().max()).item()
    e_s = ((S - S_d).abs().max() / S_d.abs().max()).item()
    say("  scan vs direct chain over 1M tokens: rel err o=%.3e S=%.3e" % (e_o, e_s))
    assert e_o <= BF16_TOL and e_s <= BF16_TOL

    # The direct chain split in half and resumed from the carried state
    # reproduces its single run bit for bit (same chunk boundaries, fp32
    # state handed over).
    half = T // 2
    say("  direct chain split at %d and resumed" % half)
    first = {n: w[n][:half].contiguous() for n in names}
    o_a, S_a = kda.kda_prefill(*(first[n] for n in names), None, None, plan=dict(segments=1))
    del first
    second = {n: w[n][half:].contiguous() for n in names}
    o_b, S_b = kda.kda_prefill(*(second[n] for n in names), S_a, None, plan=dict(segments=1))
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_d[:half]) and torch.equal(o_b, o_d[half:]) and torch.equal(S_b, S_d)


def test_k3_decode_1000_steps(kda, oracle_mod):
    from linear_attention_recurrence_delta_amd import synth
    N, H, d, steps, M = 256, 96, 128, 1000, 256
    say("CASE decode N=%d H=%d d=%d bf16: step 1 all units, %d steps with %d tracked units" % (N, H, d, steps, M))
    S = synth.decode_state(N, H, d, 0.05, 4, DEV)
    pick = np.sort(np.random.default_rng(7).choice(N * H, size=M, replace=False))
    n_idx = torch.from_numpy(pick // H).to(DEV)
    h_idx = torch.from_numpy(pick % H).to(DEV)
    S_ref = f64(S[n_idx, h_idx]).reshape(M, 1, d, d)
    # step 1: every (sequence, head) unit, outputs and updated states
    q, k, v, g, beta = synth.decode_inputs(N, H, d, torch.bfloat16, 5000, DEV)
    S_all = f64(S)
    o = torch.full((N, H, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    kda.kda_decode_step(q, k, v, g, beta, S, out=o)
    torch.cuda.synchronize()
    o1_ref, S1_ref = oracle_mod.decode_step(f64(q), f64(k), f64(v), f64(g), f64(beta), S_all)
    e_o1, e_s1 = rel_err(f64(o), o1_ref), rel_err(f64(S), S1_ref)
    say("  step 1, all %d units: rel err o=%.3e S=%.3e" % (N * H, e_o1, e_s1))
    assert e_o1 <= BF16_TOL and e_s1 <= BF16_TOL
    del S_all, S1_ref
    sel = lambda x: f64(x[n_idx, h_idx]).reshape(M, 1, *x.shape[2:])
    o_ref, S_ref = oracle_mod.decode_step(sel(q), sel(k), sel(v), sel(g), sel(beta), S_ref)
    worst_o = rel_err(sel(o), o_ref)
    for st in range(1, steps):
        q, k, v, g, beta = synth.decode_inputs(N, H, d, torch.bfloat16, 5000 + st, DEV)
        o = kda.kda_decode_step(q, k, v, g, beta, S)
        o_ref, S_ref = oracle_mod.decode_step(sel(q), sel(k), sel(v), sel(g), sel(beta), S_ref)
        worst_o = max(worst_o, rel_err(sel(o), o_ref))
        if st % 250 == 0:
            say("  step %d worst rel err o so far %.3e" % (st, worst_o))
    es = rel_err(f64(S[n_idx, h_idx]).reshape(M, 1, d, d), S_ref)
    say("  after %d steps: worst rel err o=%.3e, tracked states %.3e" % (steps, worst_o, es))
    assert torch.isfinite(S).all()
    assert worst_o <= BF16_TOL and es <= BF16_TOL


def test_k3_dense_32k_checkpoints(kda, oracle_mod):
    """State checkpoints every 4096 tokens of the dense workload: every
    checkpoint against the oracle, the last one equal to the final state,
    and prefill resumed from a checkpoint reproducing the rest of the run."""
    from linear_attention_recurrence_delta_amd import synth
    say("CASE k3_dense_32k checkpoints every 4096 tokens")
    w = synth.workload_inputs("k3_dense_32k", DEV)
    names = ("q", "k", "v", "g", "beta")
    I = 4096
    o, S, ck, first = kda.kda_prefill_checkpointed(*(w[n] for n in names), None, None, checkpoint_interval=I)
    o_ref, S_ref = kda.kda_prefill(*(w[n] for n in names), None, None)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
    assert ck.shape[0] == w["T"] // I == 8 and first.cpu().tolist() == [0, 8]
    assert torch.equal(ck[7], S[0])
    # every checkpoint of every head against the oracle's, which are the final
    # states of its recurrence over the 4096, 8192, ... token prefixes
    err = 0.0
    for h0 in range(0, w["H"], HEAD_BATCH):
        hi = torch.arange(h0, min(h0 + HEAD_BATCH, w["H"]), device=DEV)
        sl = lambda x: f64(x.index_select(1, hi))
        rck, rfirst = oracle_mod.prefill_checkpoints(sl(w["q"]), sl(w["k"]), sl(w["v"]), sl(w["g"]), sl(w["beta"]),
                                                     interval=I)
        assert list(rfirst) == [0, 8]
        err = max(err, rel_err(f64(ck.index_select(1, hi)), rck))
    say("  all 8 checkpoints of all %d heads: rel err %.3e" % (w["H"], err))
    assert err <= BF16_TOL
    # resume from checkpoint 3 (after 16384 tokens): the rest of the run again
    R = 4 * I
    rest = {n: w[n][R:].contiguous() for n in names}
    o_r, S_r = kda.kda_prefill(*(rest[n] for n in names), ck[3:4].contiguous(), None)
    torch.cuda.synchronize()
    e_o = (o_r.float() - o[R:].float()).abs().max().item() / o[R:].float().abs().max().item()
    e_s = (S_r - S).abs().max().item() / S.abs().max().item()
    say("  resumed from checkpoint 3: rel err o=%.3e S=%.3e" % (e_o, e_s))
    assert e_o <= 1e-6 and e_s <= 1e-6


def test_k3_varlen_32k_backward_all_units(kda, oracle_mod):
    """The backward on the 16-sequence K3 varlen batch (1536 (sequence, head)
    units, 3072 workgroups): every gradient of every unit against the oracle,
    16 heads (all sequences) per oracle call."""
    from linear_attention_recurrence_delta_amd import synth
    w = synth.workload_inputs("k3_varlen_32k", DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(708)
    d_o = torch.randn(w["v"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    say("CASE backward k3 varlen 32K x 96, all 1536 units")
    got = kda.kda_prefill_backward(w["q"], w["k"], w["v"], w["g"], w["beta"], d_o, cu_seqlens=w["cu"])
    torch.cuda.synchronize()
    for x in got:
        assert torch.isfinite(x.float()).all()
    cu = np.concatenate([[0], np.cumsum(w["lengths"])])
    errs = [0.0] * 6
    for h0 in range(0, w["H"], HEAD_BATCH):
        hi = torch.arange(h0, min(h0 + HEAD_BATCH, w["H"]), device=DEV)
        sl = lambda x: f64(x.index_select(1, hi))
        ref = oracle_mod.prefill_backward(sl(w["q"]), sl(w["k"]), sl(w["v"]), sl(w["g"]), sl(w["beta"]), sl(d_o),
                                          cu_seqlens=cu)
        for i in range(6):
            errs[i] = max(errs[i], rel_err(sl(got[i]), ref[i]))
        say("  heads %d..%d done" % (h0, h0 + len(hi) - 1))
    say("  all 1536 units: dq=%.2e dk=%.2e dv=%.2e dg=%.2e dbeta=%.2e dS0=%.2e" % tuple(errs))
    assert max(errs) <= TOL[torch.bfloat16]
