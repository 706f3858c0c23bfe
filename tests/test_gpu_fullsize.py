"""GPU parity at the full K3-shaped sizes, in the launch configuration the
benchmark times (library default chunk, no initial state for prefill).

The oracle cannot replay every unit of these workloads in seconds, so each
test checks sampled (sequence, head) units element by element against it,
plus properties that hold at any size:

* dense B=1 T=32768 H=96 and the 16-sequence varlen pack of about 32K
  tokens: whole outputs and final states of sampled units;
* long context B=1 T=1,048,576 H=16: outputs of the first 8192 tokens of
  every head, the final state of the 65536-token prefix, and, for the full
  million tokens, that splitting the sequence and resuming from the carried
  state changes nothing;
* batched decode 256 sequences x 96 heads: 1000 steps, a seeded sample of
  256 units tracked against the oracle on every step.
"""
import numpy as np
import pytest
import torch

from gpu_common import TOL, f64, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16_TOL = TOL[torch.bfloat16]


@pytest.fixture(scope="module")
def kda():
    import linear_attention_recurrence_delta_amd as m
    return m


def _unit_check(oracle, w, o, S, units, t_limit=None, label=""):
    """Compare sampled units with the oracle; units of one sequence go to the
    oracle in one call so that its threads run the heads side by side."""
    cu_list = [0] + [int(x) for x in np.cumsum(w["lengths"])]
    by_seq = {}
    for n, h in units:
        by_seq.setdefault(n, []).append(h)
    worst_o = worst_s = 0.0
    for n, heads in sorted(by_seq.items()):
        a, b = cu_list[n], cu_list[n + 1]
        if t_limit is not None:
            b = min(b, a + t_limit)
        hi = torch.tensor(heads, device=w["q"].device)
        sl = lambda x: f64(x[a:b].index_select(1, hi))
        ro, rs = oracle.prefill(sl(w["q"]), sl(w["k"]), sl(w["v"]), sl(w["g"]), sl(w["beta"]))
        worst_o = max(worst_o, rel_err(sl(o), ro))
        if S is not None:
            worst_s = max(worst_s, rel_err(f64(S[n].index_select(0, hi)), rs[0]))
    say("  %s: %d units, rel err o=%.3e S=%.3e (tol %.0e)" % (label, len(units), worst_o, worst_s, BF16_TOL))
    assert np.isfinite(worst_o) and np.isfinite(worst_s)
    assert worst_o <= BF16_TOL and worst_s <= BF16_TOL


def test_k3_dense_32k_sampled_heads(kda, oracle_mod):
    from linear_attention_recurrence_delta_amd import synth
    say("CASE k3_dense_32k B=1 T=32768 H=96 default chunk, heads 0, 41, 95")
    w = synth.workload_inputs("k3_dense_32k", DEV)
    o, S = kda.kda_prefill(w["q"], w["k"], w["v"], w["g"], w["beta"], None, None)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    _unit_check(oracle_mod, w, o, S, [(0, 0), (0, 41), (0, 95)], label="dense 32K")


def test_k3_varlen_32k_sampled_units(kda, oracle_mod):
    from linear_attention_recurrence_delta_amd import synth
    w = synth.workload_inputs("k3_varlen_32k", DEV)
    L = w["lengths"]
    longest, shortest = int(np.argmax(L)), int(np.argmin(L))
    units = [(longest, 7), (shortest, 88), (len(L) // 2, 50), (len(L) - 1, 95), (0, 0)]
    say("CASE k3_varlen_32k N=16 T=%d lengths %d..%d, units %s" % (w["T"], min(L), max(L), units))
    o, S = kda.kda_prefill(w["q"], w["k"], w["v"], w["g"], w["beta"], None, w["cu"])
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(S).all()
    _unit_check(oracle_mod, w, o, S, units, label="varlen 32K")


def test_long_context_1m_h16(kda, oracle_mod):
    from linear_attention_recurrence_delta_amd import synth
    say("CASE long_1m_h16 B=1 T=1048576 H=16 default chunk")
    w = synth.workload_inputs("long_1m_h16", DEV)
    T, H = w["T"], w["H"]
    names = ("q", "k", "v", "g", "beta")
    o, S = kda.kda_prefill(*(w[n] for n in names), None, None)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(S).all()

    # outputs of the first 8192 tokens of every head
    _unit_check(oracle_mod, w, o, None, [(0, h) for h in range(H)], t_limit=8192, label="first 8192 tokens")

    # final state of the 65536-token prefix
    P = 65536
    say("  prefix %d tokens" % P)
    pre = {n: w[n][:P].contiguous() for n in names}
    o_p, S_p = kda.kda_prefill(*(pre[n] for n in names), None, None)
    torch.cuda.synchronize()
    wp = dict(w, q=pre["q"], k=pre["k"], v=pre["v"], g=pre["g"], beta=pre["beta"], lengths=[P])
    _unit_check(oracle_mod, wp, o_p, S_p, [(0, h) for h in range(H)], label="prefix 65536 state")
    # The prefix run's outputs are the full run's first P outputs.
    assert torch.equal(o_p, o[:P])

    # Splitting the million tokens and resuming from the carried state
    # reproduces the single run (same chunk boundaries, fp32 state handed over).
    half = T // 2
    say("  split at %d and resume" % half)
    first = {n: w[n][:half].contiguous() for n in names}
    o_a, S_a = kda.kda_prefill(*(first[n] for n in names), None, None)
    del first
    second = {n: w[n][half:].contiguous() for n in names}
    o_b, S_b = kda.kda_prefill(*(second[n] for n in names), S_a, None)
    torch.cuda.synchronize()
    e_o = (o_b.float() - o[half:].float()).abs().max().item() / o[half:].float().abs().max().item()
    e_s = (S_b - S).abs().max().item() / S.abs().max().item()
    say("  resume rel err o=%.3e S=%.3e" % (e_o, e_s))
    assert torch.equal(o_a, o[:half])
    assert e_o <= 1e-6 and e_s <= 1e-6


def test_k3_decode_1000_steps_tracked_units(kda, oracle_mod):
    from linear_attention_recurrence_delta_amd import synth
    N, H, d, steps, M = 256, 96, 128, 1000, 256
    say("CASE decode N=%d H=%d d=%d bf16, %d steps, %d tracked units" % (N, H, d, steps, M))
    S = synth.decode_state(N, H, d, 0.05, 4, DEV)
    pick = np.sort(np.random.default_rng(7).choice(N * H, size=M, replace=False))
    n_idx = torch.from_numpy(pick // H).to(DEV)
    h_idx = torch.from_numpy(pick % H).to(DEV)
    S_ref = f64(S[n_idx, h_idx]).reshape(M, 1, d, d)
    worst_o = 0.0
    for st in range(steps):
        q, k, v, g, beta = synth.decode_inputs(N, H, d, torch.bfloat16, 5000 + st, DEV)
        o = kda.kda_decode_step(q, k, v, g, beta, S)
        sel = lambda x: f64(x[n_idx, h_idx]).reshape(M, 1, *x.shape[2:])
        o_ref, S_ref = oracle_mod.decode_step(sel(q), sel(k), sel(v), sel(g), sel(beta), S_ref)
        worst_o = max(worst_o, rel_err(sel(o), o_ref))
        if st % 250 == 0:
            say("  step %d worst rel err o so far %.3e" % (st, worst_o))
    es = rel_err(f64(S[n_idx, h_idx]).reshape(M, 1, d, d), S_ref)
    say("  after %d steps: worst rel err o=%.3e, tracked states %.3e" % (steps, worst_o, es))
    assert torch.isfinite(S).all()
    assert worst_o <= BF16_TOL and es <= BF16_TOL


def test_k3_dense_32k_checkpoints(kda, oracle_mod):
    """State checkpoints every 4096 tokens of the dense workload: sampled
    checkpoints against the oracle, the last one equal to the final state,
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
    # checkpoint 0 of three heads against the oracle's 4096-token prefix
    heads = [0, 41, 95]
    hi = torch.tensor(heads, device=DEV)
    sl = lambda x: f64(x[:I].index_select(1, hi))
    _, rs = oracle_mod.prefill(sl(w["q"]), sl(w["k"]), sl(w["v"]), sl(w["g"]), sl(w["beta"]))
    err = rel_err(f64(ck[0].index_select(0, hi)), rs[0])
    say("  checkpoint 0, heads %s: rel err %.3e" % (heads, err))
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


def test_k3_varlen_32k_backward_sampled_units(kda, oracle_mod):
    """The backward on the 16-sequence K3 varlen batch (1536 (sequence, head)
    units, 3072 workgroups): the longest and the shortest sequence on two
    heads each against the oracle, with the gradient tensors restricted to
    those tokens and heads."""
    from linear_attention_recurrence_delta_amd import synth
    w = synth.workload_inputs("k3_varlen_32k", DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(708)
    d_o = torch.randn(w["v"].shape, generator=gen, device=DEV).to(torch.bfloat16)
    say("CASE backward k3 varlen 32K x 96")
    got = kda.kda_prefill_backward(w["q"], w["k"], w["v"], w["g"], w["beta"], d_o, cu_seqlens=w["cu"])
    torch.cuda.synchronize()
    lengths = w["lengths"]
    cu = [0] + [int(x) for x in np.cumsum(lengths)]
    picks = [int(np.argmax(lengths)), int(np.argmin(lengths))]
    heads = torch.tensor([3, 77], device=DEV)
    for n in picks:
        a, b = cu[n], cu[n + 1]
        sl = lambda x: f64(x[a:b].index_select(1, heads))
        ref = oracle_mod.prefill_backward(sl(w["q"]), sl(w["k"]), sl(w["v"]), sl(w["g"]), sl(w["beta"]), sl(d_o))
        errs = [rel_err(sl(x), r) for x, r in zip(got[:5], ref[:5])]
        errs.append(rel_err(f64(got[5][n].index_select(0, heads)), ref[5][0]))
        say("  sequence %d (%d tokens): " % (n, b - a) + " ".join("%.2e" % e for e in errs))
        assert max(errs) <= TOL[torch.bfloat16]
