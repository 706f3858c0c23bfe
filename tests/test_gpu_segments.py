"""GPU parity of the sequence-segment scan (kda_prefill_ex with segments >= 2,
and the library's own choice for long sequences with few heads).

The scan cuts each sequence into segments, computes every segment's affine
map (M, B) in parallel, chains them into start states, and re-runs the
segments from those states.  The result is the recurrence's up to rounding
("Understanding Kimi K3's attention", state-update equation: affine in the
state), so it must meet the oracle at the bf16 tolerance on every output
and final state, with the state carried across segment boundaries (weak and
zero decay make that carry visible), ragged last chunks, initial states and
a readout scale.
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


def _dense(B, T, H, seed, g_mode="k3", init_std=0.05):
    from linear_attention_recurrence_delta_amd import synth
    q, k, v, g, beta, gen = synth.token_inputs(B * T, H, 128, 128, BF16, seed, DEV, g_mode)
    S0 = synth.initial_state(B, H, 128, 128, init_std, gen, DEV) if init_std else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0, B=B, T=T, H=H)


def _oracle_check(oracle_mod, w, o, S, scale, label):
    B, T = w["B"], w["T"]
    cu = np.arange(B + 1) * T
    ro, rs = oracle_mod.prefill(f64(w["q"]), f64(w["k"]), f64(w["v"]), f64(w["g"]), f64(w["beta"]),
                                None if w["S0"] is None else f64(w["S0"]), cu, scale=scale)
    eo, es = rel_err(f64(o), ro), rel_err(f64(S), rs)
    say("  %s: rel err o=%.3e S=%.3e" % (label, eo, es))
    assert np.isfinite(eo) and np.isfinite(es)
    assert eo <= TOL[BF16] and es <= TOL[BF16]


def _run(kda, w, scale=1.0, **plan):
    names = ("q", "k", "v", "g", "beta")
    o = torch.full((w["B"] * w["T"], w["H"], 128), float("nan"), dtype=BF16, device=DEV)
    S = torch.full((w["B"], w["H"], 128, 128), float("nan"), dtype=torch.float32, device=DEV)
    kda.kda_prefill(*(w[n] for n in names), w["S0"], None, num_seqs=w["B"], scale=scale, plan=plan,
                    out=o, final_state=S)
    torch.cuda.synchronize()
    return o, S


@pytest.mark.parametrize("G", [2, 3, 5, 12])
@pytest.mark.parametrize("g_mode", ["mild", "zero", "k3"])
def test_segments_vs_oracle(kda, oracle_mod, G, g_mode):
    # two dense sequences of 3000 tokens (a ragged last chunk), 3 heads
    say("CASE segment scan G=%d g=%s B=2 T=3000 H=3 S0 scale 0.9" % (G, g_mode))
    w = _dense(2, 3000, 3, 2000 + G, g_mode)
    o, S = _run(kda, w, scale=0.9, kernel=1, segments=G)
    _oracle_check(oracle_mod, w, o, S, 0.9, "G=%d" % G)
    # the direct chain agrees to the same bar, and the scan is deterministic
    o_d, S_d = _run(kda, w, scale=0.9, kernel=1, segments=1)
    assert rel_err(f64(o), f64(o_d)) <= TOL[BF16] and rel_err(f64(S), f64(S_d)) <= TOL[BF16]
    o2, S2 = _run(kda, w, scale=0.9, kernel=1, segments=G)
    assert torch.equal(o, o2) and torch.equal(S, S2)


def test_segments_slab_width_bitwise(kda):
    # the scan is built for whole heads and 64-column slabs: same bits
    w = _dense(1, 2500, 2, 2100, "mild")
    ref = _run(kda, w, segments=6, slab_columns=128)
    got = _run(kda, w, segments=6, slab_columns=64)
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
    with pytest.raises(kda.KdaError) as e:  # narrower slabs are not built with the scan
        _run(kda, w, segments=6, slab_columns=32)
    assert e.value.status == 3


def test_smallest_segments(kda, oracle_mod):
    # 96 tokens = 6 chunks: G = 6 gives segments of one chunk, G = 5 a last
    # segment of two
    say("CASE segment scan, one-chunk segments")
    w = _dense(3, 96, 2, 2200, "zero")
    for G in (5, 6):
        o, S = _run(kda, w, segments=G)
        _oracle_check(oracle_mod, w, o, S, 1.0, "T=96 G=%d" % G)
    with pytest.raises(kda.KdaError) as e:  # 6 chunks cannot hold 7 segments
        _run(kda, w, segments=7)
    assert e.value.status == 3


def test_library_picks_the_scan_for_long_sequences(kda, oracle_mod):
    # 2 heads of one 40,000-token sequence: 2 units on a 256-CU device, so the
    # library cuts the sequence into segments (the workspace query says so)
    say("CASE automatic segment scan B=1 T=40000 H=2")
    w = _dense(1, 40000, 2, 2300, "mild", init_std=0.02)
    ws = kda.kda_prefill_ex_workspace_bytes(1, 40000, 2, 128, 128, BF16)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say("  workspace %d bytes on %d CUs" % (ws, cus))
    assert ws > 0
    o = torch.full((40000, 2, 128), float("nan"), dtype=BF16, device=DEV)
    o, S = kda.kda_prefill(w["q"], w["k"], w["v"], w["g"], w["beta"], w["S0"], out=o)
    torch.cuda.synchronize()
    _oracle_check(oracle_mod, w, o, S, 1.0, "auto")


def test_empty_and_packed_calls_take_no_scan(kda):
    # cu_seqlens: the direct chain, no workspace, explicit scan refused
    w = _dense(1, 2048, 2, 2400)
    cu = torch.tensor([0, 1000, 2048], dtype=torch.int32, device=DEV)
    names = ("q", "k", "v", "g", "beta")
    with pytest.raises(kda.KdaError) as e:
        kda.kda_prefill(*(w[n] for n in names), None, cu, plan=dict(segments=3))
    assert e.value.status == 3
    o, S = kda.kda_prefill(*(w[n] for n in names), None, cu)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and S.shape == (2, 2, 128, 128)
