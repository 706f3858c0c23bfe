"""kda_prefill_output_gated: the prefill with y = Sigmoid(gate) * RMSNorm(o) *
weight returned in place of o ("Understanding Kimi K3's attention", output
equation).

The readout o is checked against the oracle by the prefill tests; here y is
checked against the oracle's fp64 output gate evaluated on that same o (the
kernels' bf16 o, bit for bit what kda_prefill returns for the same inputs),
row by row, with the bar of the standalone gate (max over rows of |d| / max
|ref| in the row <= 8e-3: one bf16 rounding of y on fp32 arithmetic).  A
row-wise bar is the meaningful one: RMSNorm scales every row to unit size, so
rows of very different magnitude in o end up alike in y.  Paths: the gate
fused into the o store (whole heads per workgroup: more (sequence, head)
units than half the compute units), the separate pass after a sliced or
segment-scan prefill, fp32, and y written over the gate logits.
"""
import numpy as np
import pytest
import torch

from gpu_common import TOL, f64, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
GATE_TOL = {torch.bfloat16: 8e-3, torch.float32: 1e-5}


@pytest.fixture(scope="module")
def kda():
    import linear_attention_recurrence_delta_amd as m
    return m


def _max_rel_row(got, ref):
    got, ref = f64(got), np.asarray(ref)
    den = np.max(np.abs(ref), axis=-1, keepdims=True)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(got - ref) / den))


def _inputs(lengths, H, d, dtype, seed, init_std=0.05, dense=False):
    from linear_attention_recurrence_delta_amd import synth
    T = sum(lengths)
    q, k, v, g, beta, gen = synth.token_inputs(T, H, d, d, dtype, seed, DEV)
    S0 = synth.initial_state(len(lengths), H, d, d, init_std, gen, DEV) if init_std else None
    gate = (1.5 * torch.randn((T, H, d), generator=gen, device=DEV)).to(dtype)
    w = 1.0 + 0.25 * torch.randn((d,), generator=gen, device=DEV)
    cu = None if dense else torch.tensor([0] + [int(x) for x in np.cumsum(lengths)], dtype=torch.int32, device=DEV)
    return dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0, gate=gate, w=w, cu=cu, N=len(lengths))


def _check(kda, oracle_mod, x, label, scale=1.0, eps=1e-6, in_place=False):
    names = ("q", "k", "v", "g", "beta")
    args = tuple(x[n] for n in names)
    nseq = x["N"] if x["cu"] is None else None
    o, S = kda.kda_prefill(*args, x["S0"], x["cu"], scale=scale, num_seqs=nseq)
    gate = x["gate"].clone()
    out = gate if in_place else torch.full_like(o, float("nan"))
    y, S_y = kda.kda_prefill_output_gated(*args, gate, x["w"], x["S0"], x["cu"], eps=eps, scale=scale,
                                          num_seqs=nseq, out=out)
    torch.cuda.synchronize()
    ref = oracle_mod.output_gate(f64(o), f64(x["gate"]), f64(x["w"]), eps)
    err = _max_rel_row(y, ref)
    say("  %s: y vs the oracle's gate over o: max row-relative error %.3e" % (label, err))
    assert np.isfinite(f64(y)).all()
    assert err <= GATE_TOL[o.dtype]
    assert torch.equal(S_y, S)  # the final states are those of kda_prefill
    return o, y


def test_fused_whole_heads(kda, oracle_mod):
    # 8 sequences x 17 heads = 136 (sequence, head) units: whole-head
    # workgroups, so the gate is applied before the o store
    say("CASE gated prefill, whole heads (fused): ragged lengths, S0, scale 0.9")
    x = _inputs([1, 0, 17, 64, 130, 255, 700, 33], 17, 128, torch.bfloat16, 4100)
    o, y = _check(kda, oracle_mod, x, "fused", scale=0.9)
    # and the readout it gated is the oracle's to the prefill bar
    ro, _ = oracle_mod.prefill(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["g"]), f64(x["beta"]),
                               f64(x["S0"]), x["cu"].cpu().numpy(), scale=0.9)
    assert rel_err(f64(o), ro) <= TOL[torch.bfloat16]


def test_fused_in_place_over_gate(kda, oracle_mod):
    say("CASE gated prefill, whole heads, y over the gate logits")
    x = _inputs([300, 5, 160], 48, 128, torch.bfloat16, 4101, init_std=None)
    _check(kda, oracle_mod, x, "fused, in place", in_place=True)


def test_fused_zero_rows_and_eps(kda, oracle_mod):
    # beta = 0, no initial state and q = 0 on some tokens: rows of o that are
    # exactly zero give y = 0 (eps keeps the norm finite)
    say("CASE gated prefill, zero rows of o")
    x = _inputs([200, 77], 70, 128, torch.bfloat16, 4102, init_std=None)
    x["q"][10:20].zero_()
    _check(kda, oracle_mod, x, "fused, zero rows", eps=1e-5)


def test_separate_pass_sliced_heads(kda, oracle_mod):
    # 2 x 3 units: the prefill splits heads over workgroups; the gate is a
    # second pass over y
    say("CASE gated prefill, sliced heads (separate pass)")
    x = _inputs([333, 190], 3, 128, torch.bfloat16, 4103)
    _check(kda, oracle_mod, x, "separate pass")


def test_separate_pass_after_segment_scan(kda, oracle_mod):
    say("CASE gated prefill after a segment scan (1 x 40000 tokens, 2 heads)")
    x = _inputs([40000], 2, 128, torch.bfloat16, 4104, init_std=0.02, dense=True)
    assert kda.kda_prefill_ex_workspace_bytes(1, 40000, 2, 128, 128, torch.bfloat16) > 0
    _check(kda, oracle_mod, x, "segment scan + pass")


@pytest.mark.parametrize("d", [16, 64])
def test_fp32(kda, oracle_mod, d):
    say("CASE gated prefill fp32 d=%d" % d)
    x = _inputs([70, 0, 33], 2, d, torch.float32, 4105 + d)
    _check(kda, oracle_mod, x, "fp32 d=%d" % d)


def test_k3_varlen_32k_gated_all_units(kda, oracle_mod):
    """The 16-sequence K3 pack (1536 units, whole heads: the fused path) with
    the gate: every row of y against the oracle's gate over the prefill's o."""
    from linear_attention_recurrence_delta_amd import synth
    say("CASE gated prefill, K3 varlen 32K x 96 (fused)")
    w = synth.workload_inputs("k3_varlen_32k", DEV)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(4106)
    gate = (1.5 * torch.randn(w["v"].shape, generator=gen, device=DEV)).to(torch.bfloat16)
    wt = 1.0 + 0.25 * torch.randn((128,), generator=gen, device=DEV)
    names = ("q", "k", "v", "g", "beta")
    o, S = kda.kda_prefill(*(w[n] for n in names), None, w["cu"])
    y = torch.full_like(o, float("nan"))
    kda.kda_prefill_output_gated(*(w[n] for n in names), gate, wt, None, w["cu"], out=y)
    torch.cuda.synchronize()
    worst = 0.0
    for h0 in range(0, 96, 16):
        sl = slice(h0, h0 + 16)
        ref = oracle_mod.output_gate(f64(o[:, sl]), f64(gate[:, sl]), f64(wt), 1e-6)
        worst = max(worst, _max_rel_row(y[:, sl], ref))
    say("  all 3,145,728 rows: max row-relative error %.3e" % worst)
    assert worst <= GATE_TOL[torch.bfloat16]
